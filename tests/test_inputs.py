"""The seeded input generator: determinism, bf16 exactness and the stated distributions (CPU)."""
import numpy as np
import pytest

import oracle.moe_oracle as orc
from expert_routing_grouped_moe_amd import inputs as gen


def test_deterministic_and_seed_sensitive():
    a = gen.make_inputs("tiny-fp32")
    b = gen.make_inputs("tiny-fp32")
    c = gen.make_inputs("tiny-fp32", seed=5)
    for key in ("x", "w_router", "w_gate", "w_up", "w_down"):
        np.testing.assert_array_equal(getattr(a, key), getattr(b, key))
    assert not np.array_equal(a.x, c.x)


def test_bf16_values_are_exact_bits():
    inp = gen.make_inputs("zonos3mini-decode-cfg")
    for key in ("x", "w_router", "w_gate", "w_up", "w_down"):
        bits = inp.bits[key]
        assert bits.dtype == np.uint16
        np.testing.assert_array_equal(gen.bf16_bits_to_f32(bits), getattr(inp, key))
        # low 16 bits of every fp32 value are zero
        assert (getattr(inp, key).view(np.uint32) & 0xFFFF).max() == 0


def test_bf16_rounding_is_rne():
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -9, 1.0 + 2 ** -9, -2.5], dtype=np.float32)
    got = gen.bf16_bits_to_f32(gen.bf16_round_bits(vals))
    # bf16 ulp at 1 is 2^-7: 1+2^-8 is the halfway point (ties to even -> 1.0), 1+3*2^-9 lies
    # above it (-> 1+2^-7), 1+2^-9 below it (-> 1.0)
    np.testing.assert_array_equal(got, np.array([1.0, 1.0, 1.0 + 2 ** -7, 1.0, -2.5], np.float32))


def test_distribution_moments():
    inp = gen.make_inputs("zonos3mini-prefill")
    assert abs(inp.x.std() - 1.0) < 0.01
    assert abs(inp.w_gate.std() * np.sqrt(inp.d) - 1.0) < 0.01
    assert abs(inp.w_down.std() * np.sqrt(inp.H) - 1.0) < 0.01
    assert abs(inp.sel_bias.var() - 0.5) < 0.25  # 64 draws
    assert inp.router_bias is None


def test_skewed_prefill_shares():
    inp = gen.make_inputs("zonos2-skewed-prefill")
    assert inp.router_bias[14] == -30 and inp.router_bias[15] == -30
    assert 1.2 < inp.router_bias[0] < 1.6
    L = orc.router_logits_ref(inp.x, inp.w_router, inp.router_bias)
    counts = np.bincount(L.argmax(axis=1), minlength=inp.E)
    assert counts[14] == 0 and counts[15] == 0
    assert abs(counts[0] / inp.T - 0.40) < 0.03
