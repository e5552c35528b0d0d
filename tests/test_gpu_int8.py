"""int8 expert weights on the decode path: moe_quantize_rows_i8 bit-exact against the oracle's
codes and scales, and moe_layer_forward with int8 weights against the fp64 oracle evaluated on
the dequantised weights s * q (codes from the oracle's quantiser, so the layer test does not
depend on the GPU quantiser)."""
import dataclasses

import numpy as np
import pytest

import oracle.moe_oracle as orc
from expert_routing_grouped_moe_amd import inputs as gen

from _parity import DEV, check_layer, upload

pytestmark = pytest.mark.gpu

KEYS = ("w_gate", "w_up", "w_down")


def _bf16_dev(a32):
    import torch
    bits = gen.bf16_round_bits(np.ascontiguousarray(a32, dtype=np.float32))
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(DEV)


def _tie_row(K, scale_exp):
    """A row whose quotients w / s are exactly j + 1/2 (ties) plus one extreme at 127."""
    j = (np.arange(K) % 253) - 126                  # -126 .. 126
    v = (j + 0.5) * 2.0 ** scale_exp
    v[0] = 127 * 2.0 ** scale_exp                   # s = 2^scale_exp exactly
    return v.astype(np.float32)


@pytest.mark.parametrize("shape", [(4, 96, 64), (16, 256, 2048), (3, 7, 512)])
def test_quantize_bit_exact_bf16(shape):
    from expert_routing_grouped_moe_amd import moe
    rng = np.random.default_rng(sum(shape))
    w = gen.bf16_bits_to_f32(gen.bf16_round_bits(
        (rng.standard_normal(shape) * 0.05).astype(np.float32)))
    w[0, 1] = 0.0                                   # all-zero row
    w[1, 0] = _tie_row(shape[-1], -4)               # exact ties (bf16-representable)
    w[1, 1] = -_tie_row(shape[-1], 3)               # negative extreme
    q, s = moe.moe_quantize_rows_i8(_bf16_dev(w))
    rq, rs = orc.quantize_rows_i8_ref(w)
    np.testing.assert_array_equal(s.cpu().numpy(), rs)
    np.testing.assert_array_equal(q.cpu().numpy(), rq)


def test_quantize_bit_exact_f32():
    import torch
    from expert_routing_grouped_moe_amd import moe
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((33, 320)) * 3).astype(np.float32)
    w[4] = 0.0
    q, s = moe.moe_quantize_rows_i8(torch.from_numpy(w).to(DEV))
    rq, rs = orc.quantize_rows_i8_ref(w)
    np.testing.assert_array_equal(s.cpu().numpy(), rs)
    np.testing.assert_array_equal(q.cpu().numpy(), rq)


def _run_int8_layer(inp, q, s):
    import torch
    from expert_routing_grouped_moe_amd import moe
    dv = upload(inp)
    T, E, k = inp.T, inp.E, inp.k
    outs = dict(
        logits=torch.empty((T, E), dtype=torch.float32, device=DEV),
        topk_ids=torch.empty((T, k), dtype=torch.int32, device=DEV),
        topk_w=torch.empty((T, k), dtype=torch.float32, device=DEV),
        expert_counts=torch.empty((E,), dtype=torch.int32, device=DEV),
    )
    qd = {key: torch.from_numpy(q[key]).to(DEV) for key in KEYS}
    sd = tuple(torch.from_numpy(s[key]).to(DEV) for key in KEYS)
    y = moe.moe_layer_forward(dv["x"], dv["w_router"], qd["w_gate"], qd["w_up"], qd["w_down"], k,
                              inp.scoring, router_bias=dv["router_bias"], sel_bias=dv["sel_bias"],
                              w_scales=sd, **outs)
    torch.cuda.synchronize()
    res = {key: v.cpu().numpy() for key, v in outs.items()}
    res["y"] = y.cpu().numpy()
    return res


def _quantised(inp):
    q, s = {}, {}
    for key in KEYS:
        q[key], s[key] = orc.quantize_rows_i8_ref(getattr(inp, key))
    deq = {key: orc.dequantize_rows_ref(q[key], s[key]) for key in KEYS}
    return q, s, dataclasses.replace(inp, **deq)


@pytest.mark.parametrize("name", ["zonos2-decode", "zonos3mini-decode-cfg", "zonos2-layer26-decode"])
def test_int8_layer_workload(name):
    inp = gen.make_inputs(name)
    q, s, inp_d = _quantised(inp)
    res = _run_int8_layer(inp, q, s)
    rep = check_layer(inp_d, res)
    print(f"{name} int8: {rep}")


EDGE = [
    # name, T, d, E, k, H, scoring, sel_bias_var, router_bias
    ("T1", 1, 256, 16, 1, 256, orc.SOFTMAX, None, None),
    ("sigmoid-k2", 64, 512, 16, 2, 512, orc.SIGMOID, None, None),
    ("E256-k8", 64, 256, 256, 8, 256, orc.SELECTED_SOFTMAX, 0.5, None),
    ("hot-expert", 200, 256, 16, 1, 256, orc.SOFTMAX, None, "hot5"),     # many passes
    ("rows-17-32", 96, 256, 8, 2, 512, orc.SELECTED_SOFTMAX, 0.5, None),  # two-group passes
    # d = H = 768: six 128-k blocks per row, outside the unrolled widths, so the reduction loop
    # runs rolled over three trips with the prefetch carried across its back edge
    ("generic-K768", 48, 768, 16, 2, 768, orc.SELECTED_SOFTMAX, 0.5, None),
]


@pytest.mark.parametrize("case", EDGE, ids=[c[0] for c in EDGE])
def test_int8_layer_edge_cases(case):
    name, T, d, E, k, H, scoring, sbv, rb = case
    router_bias = None
    if rb == "hot5":
        router_bias = np.full(E, -30.0, np.float32)
        router_bias[5] = 30.0
    inp = gen.make_inputs_custom(T, d, E, k, H, scoring, "bf16", seed=3 * T + E + k,
                                 sel_bias_var=sbv, router_bias=router_bias)
    q, s, inp_d = _quantised(inp)
    res = _run_int8_layer(inp, q, s)
    rep = check_layer(inp_d, res)
    print(f"{name}: {rep}")
    if rb == "hot5":
        assert res["expert_counts"][5] == T


def test_int8_layer_deterministic():
    inp = gen.make_inputs("zonos3mini-decode-cfg")
    q, s, _ = _quantised(inp)
    a = _run_int8_layer(inp, q, s)
    b = _run_int8_layer(inp, q, s)
    np.testing.assert_array_equal(a["y"], b["y"])


def test_int8_rejected_outside_decode_path():
    import torch
    from expert_routing_grouped_moe_amd import moe
    inp = gen.make_inputs_custom(3000, 256, 8, 1, 256, orc.SOFTMAX, "bf16", seed=9)
    q, s, _ = _quantised(inp)
    dv = upload(inp)
    qd = {key: torch.from_numpy(q[key]).to(DEV) for key in KEYS}
    sd = tuple(torch.from_numpy(s[key]).to(DEV) for key in KEYS)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_layer_forward(dv["x"], dv["w_router"], qd["w_gate"], qd["w_up"], qd["w_down"], 1,
                              inp.scoring, w_scales=sd)
    assert ei.value.status == moe.MOE_ERR_UNSUPPORTED
