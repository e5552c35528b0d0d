"""4-bit affine expert weights on the decode path: moe_quantize_groups_q4 bit-exact against the
oracle's codes (in the packed order) and (scale, bias) pairs, and moe_layer_forward with 4-bit
weights against the fp64 oracle evaluated on the dequantised weights s * q + b (codes from the
oracle's quantiser, so the layer test does not depend on the GPU quantiser)."""
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


def _special_rows(K):
    """Rows of groups whose codes hinge on ties, a bf16-rounded scale or bias, and s = 0."""
    ramp = np.arange(64, dtype=np.float32)
    ties = np.where(ramp % 2 == 0, ramp % 16, (ramp % 15) + 0.5).astype(np.float32)
    ties[0], ties[1] = 0.0, 15.0                    # s = 1, b = 0: codes are ties to even
    neg = (-0.5 * ties).astype(np.float32)          # s = 1/2, b = -7.5
    const = np.full(64, 0.3, np.float32)            # s = 0, b = bf16(0.3)
    third = (ramp / 63).astype(np.float32)          # s = bf16(1/15) rounds
    groups = [ties, neg, const, third]
    row = np.concatenate([groups[i % 4] for i in range(K // 64)])
    return np.stack([row, -row[::-1]])


def _check_quant(w32, q, qpar):
    rq, rs, rb = orc.quantize_groups_q4_ref(w32)
    np.testing.assert_array_equal(q.cpu().numpy(), orc.pack_q4_ref(rq))
    np.testing.assert_array_equal(qpar.cpu().numpy().view(np.uint32), orc.pack_q4_params_ref(rs, rb))


@pytest.mark.parametrize("shape", [(4, 96, 128), (16, 256, 2048), (3, 7, 512)])
def test_quantize_q4_bit_exact_bf16(shape):
    from expert_routing_grouped_moe_amd import moe
    rng = np.random.default_rng(sum(shape) + 1)
    w = gen.bf16_bits_to_f32(gen.bf16_round_bits(
        (rng.standard_normal(shape) * 0.05).astype(np.float32)))
    w[0, :2] = _special_rows(shape[-1])
    w = gen.bf16_bits_to_f32(gen.bf16_round_bits(w))   # the specials are bf16 values
    q, qpar = moe.moe_quantize_groups_q4(_bf16_dev(w))
    _check_quant(w, q, qpar)


def test_quantize_q4_bit_exact_f32():
    import torch
    from expert_routing_grouped_moe_amd import moe
    rng = np.random.default_rng(7)
    w = (rng.standard_normal((33, 384)) * 3).astype(np.float32)
    w[4] = 0.0
    w[5:7] = _special_rows(384)
    q, qpar = moe.moe_quantize_groups_q4(torch.from_numpy(w).to(DEV))
    _check_quant(w, q, qpar)


def _quantised(inp):
    q, p, deq = {}, {}, {}
    for key in KEYS:
        codes, s, b = orc.quantize_groups_q4_ref(getattr(inp, key))
        q[key] = orc.pack_q4_ref(codes)
        p[key] = orc.pack_q4_params_ref(s, b).view(np.int32)
        deq[key] = orc.dequantize_groups_q4_ref(codes, s, b)
    return q, p, dataclasses.replace(inp, **deq)


def _run_q4_layer(inp, q, p):
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
    pd = tuple(torch.from_numpy(p[key]).to(DEV) for key in KEYS)
    y = moe.moe_layer_forward(dv["x"], dv["w_router"], qd["w_gate"], qd["w_up"], qd["w_down"], k,
                              inp.scoring, router_bias=dv["router_bias"], sel_bias=dv["sel_bias"],
                              w_scales=pd, **outs)
    torch.cuda.synchronize()
    res = {key: v.cpu().numpy() for key, v in outs.items()}
    res["y"] = y.cpu().numpy()
    return res


@pytest.mark.parametrize("name", ["zonos2-decode", "zonos3mini-decode-cfg", "zonos2-layer26-decode"])
def test_q4_layer_workload(name):
    inp = gen.make_inputs(name)
    q, p, inp_d = _quantised(inp)
    res = _run_q4_layer(inp, q, p)
    rep = check_layer(inp_d, res)
    print(f"{name} q4: {rep}")


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
def test_q4_layer_edge_cases(case):
    name, T, d, E, k, H, scoring, sbv, rb = case
    router_bias = None
    if rb == "hot5":
        router_bias = np.full(E, -30.0, np.float32)
        router_bias[5] = 30.0
    inp = gen.make_inputs_custom(T, d, E, k, H, scoring, "bf16", seed=5 * T + E + k,
                                 sel_bias_var=sbv, router_bias=router_bias)
    q, p, inp_d = _quantised(inp)
    res = _run_q4_layer(inp, q, p)
    rep = check_layer(inp_d, res)
    print(f"{name}: {rep}")
    if rb == "hot5":
        assert res["expert_counts"][5] == T


def test_q4_layer_with_gpu_quantiser_matches_oracle_codes():
    # the library's own quantiser feeding the layer gives the same output as the oracle's codes
    import torch
    from expert_routing_grouped_moe_amd import moe
    inp = gen.make_inputs("zonos3mini-decode-cfg")
    q, p, _ = _quantised(inp)
    ref = _run_q4_layer(inp, q, p)
    dv = upload(inp)
    gq, gp = {}, {}
    for key in KEYS:
        gq[key], gp[key] = moe.moe_quantize_groups_q4(dv[key])
    y = moe.moe_layer_forward(dv["x"], dv["w_router"], gq["w_gate"], gq["w_up"], gq["w_down"],
                              inp.k, inp.scoring, sel_bias=dv["sel_bias"],
                              w_scales=tuple(gp[key] for key in KEYS))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(y.cpu().numpy(), ref["y"])


def test_q4_layer_deterministic():
    inp = gen.make_inputs("zonos3mini-decode-cfg")
    q, p, _ = _quantised(inp)
    a = _run_q4_layer(inp, q, p)
    b = _run_q4_layer(inp, q, p)
    np.testing.assert_array_equal(a["y"], b["y"])


def test_q4_rejected_outside_decode_path():
    import torch
    from expert_routing_grouped_moe_amd import moe
    inp = gen.make_inputs_custom(3000, 256, 8, 1, 256, orc.SOFTMAX, "bf16", seed=9)
    q, p, _ = _quantised(inp)
    dv = upload(inp)
    qd = {key: torch.from_numpy(q[key]).to(DEV) for key in KEYS}
    pd = tuple(torch.from_numpy(p[key]).to(DEV) for key in KEYS)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_layer_forward(dv["x"], dv["w_router"], qd["w_gate"], qd["w_up"], qd["w_down"], 1,
                              inp.scoring, w_scales=pd)
    assert ei.value.status == moe.MOE_ERR_UNSUPPORTED
