"""moe_layer_forward on the GPU against the fp64 oracle: the workloads at full size, every token
compared, edge cases, larger-than-workload prefills on token samples, determinism and HIP-graph
replay."""
import numpy as np
import pytest

import oracle.moe_oracle as orc
from expert_routing_grouped_moe_amd import inputs as gen

from _parity import DEV, check_layer, run_layer, upload

pytestmark = pytest.mark.gpu


def _sample(T, n, seed):
    if T <= n:
        return np.arange(T)
    rng = np.random.default_rng(seed)
    s = rng.choice(T, size=n, replace=False)
    return np.sort(np.concatenate([s, [0, T - 1]]))


@pytest.mark.parametrize("name", gen.WORKLOAD_ORDER)
def test_layer_workload(name):
    inp = gen.make_inputs(name)
    res = run_layer(inp)
    rep = check_layer(inp, res)                 # all tokens: the bound is on the whole output
    print(f"{name}: {rep}")
    # the layer's ids equal moe_route on the logits the layer computed (same fp32 values)
    import torch
    from expert_routing_grouped_moe_amd import moe
    ids, w, counts = moe.moe_route(torch.from_numpy(res["logits"]).to(DEV), inp.k, inp.scoring,
                                   sel_bias=None if inp.sel_bias is None else
                                   torch.from_numpy(inp.sel_bias).to(DEV))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ids.cpu().numpy(), res["topk_ids"])
    np.testing.assert_array_equal(counts.cpu().numpy(), res["expert_counts"])
    np.testing.assert_array_equal(w.cpu().numpy(), res["topk_w"])


def test_skewed_workload_loads():
    inp = gen.make_inputs("zonos2-skewed-prefill")
    res = run_layer(inp, with_logits=False)
    c = res["expert_counts"]
    assert c[14] == 0 and c[15] == 0
    assert abs(c[0] / inp.T - 0.40) < 0.03


EDGE = [
    # name, T, d, E, k, H, scoring, dtype, sel_bias_var, router_bias
    ("T1-bf16", 1, 128, 16, 1, 128, orc.SOFTMAX, "bf16", None, None),
    ("T1-f32", 1, 64, 8, 2, 64, orc.SELECTED_SOFTMAX, "f32", 0.5, None),
    ("ragged-bf16", 37, 256, 64, 2, 256, orc.SELECTED_SOFTMAX, "bf16", 0.5, None),
    ("E1", 50, 128, 1, 1, 128, orc.SOFTMAX, "bf16", None, None),
    ("kE-f32", 40, 64, 8, 8, 64, orc.SOFTMAX, "f32", None, None),
    ("k3-bf16", 90, 128, 16, 3, 192, orc.SELECTED_SOFTMAX, "bf16", 0.5, None),
    ("E256-k8", 64, 128, 256, 8, 64, orc.SELECTED_SOFTMAX, "bf16", 0.5, None),
    ("all-one-expert", 500, 128, 16, 1, 256, orc.SOFTMAX, "bf16", None, "hot5"),
    ("prefill-ragged", 1111, 192, 8, 2, 320, orc.SOFTMAX, "bf16", None, None),
    # prefill with about one row tile per expert: ragged, one hot expert over several tiles
    # with the others empty, and the ZONOS2 widths (K = 2048, 2816)
    ("prefill-few-rows-ragged", 777, 512, 16, 2, 512, orc.SELECTED_SOFTMAX, "bf16", 0.5, None),
    ("prefill-few-rows-hot-expert", 600, 1024, 8, 1, 512, orc.SOFTMAX, "bf16", None, "hot5"),
    ("prefill-zonos2-widths", 1200, 2048, 16, 1, 2816, orc.SOFTMAX, "bf16", None, None),
    # many experts: 29 empty, 20 with 1..32 rows, 15 larger (one with 1212 rows)
    ("prefill-small-experts", 1500, 256, 64, 2, 256, orc.SELECTED_SOFTMAX, "bf16", 2.0, None),
    # >= one full row tile per expert on average: the wide tiles, here with empty experts
    ("prefill-xcd-hot-expert", 2100, 128, 8, 1, 192, orc.SOFTMAX, "bf16", None, "hot5"),
    # k = 1 with long down reductions (H >= 1024, 32 or 34 K steps; the weighted output is stored
    # straight into y): the wide tiles with one hot expert, and a ragged last tile
    ("prefill-long-down-hot", 2100, 256, 8, 1, 1024, orc.SOFTMAX, "bf16", None, "hot5"),
    ("prefill-long-down-ragged", 333, 128, 4, 1, 1088, orc.SOFTMAX, "bf16", None, None),
    ("f32-prefill", 600, 128, 4, 1, 128, orc.SOFTMAX, "f32", None, None),
    # few rows per expert (T*k <= 2048 and <= 32 E) with d, H multiples of 256: the
    # weight-streaming expert kernels (checked below); d = H = 768 runs their reduction loop rolled
    ("stream-k3", 40, 256, 16, 3, 256, orc.SELECTED_SOFTMAX, "bf16", 0.5, None),
    ("stream-E256-k8", 64, 256, 256, 8, 256, orc.SELECTED_SOFTMAX, "bf16", 0.5, None),
    ("stream-hot-expert", 200, 256, 16, 1, 256, orc.SOFTMAX, "bf16", None, "hot5"),
    ("stream-max-rows", 1024, 256, 64, 2, 256, orc.SELECTED_SOFTMAX, "bf16", 0.5, None),
    ("stream-generic-K768", 48, 768, 16, 2, 768, orc.SELECTED_SOFTMAX, "bf16", 0.5, None),
    # the split router (few tokens, router matrix >= 64K elements): ragged T, and d wide enough
    # for slices wider than 256
    ("split-router-ragged", 37, 1024, 64, 2, 256, orc.SELECTED_SOFTMAX, "bf16", 0.5, None),
    ("split-router-wide-d", 20, 4608, 16, 1, 256, orc.SOFTMAX, "bf16", None, None),
    # sigmoid scoring on the three expert-kernel families
    ("sigmoid-stream", 64, 512, 16, 2, 512, orc.SIGMOID, "bf16", None, None),
    ("sigmoid-prefill", 700, 256, 8, 2, 256, orc.SIGMOID, "bf16", None, None),
    ("sigmoid-f32", 48, 64, 8, 3, 128, orc.SIGMOID, "f32", None, None),
]


@pytest.mark.parametrize("case", EDGE, ids=[c[0] for c in EDGE])
def test_layer_edge_cases(case):
    name, T, d, E, k, H, scoring, dtype, sbv, rb = case
    if name.startswith("stream-"):  # the shape rule of the weight-streaming path
        assert T * k <= 2048 and T * k <= 32 * E and d % 256 == 0 and H % 256 == 0, name
    if "xcd" in name:               # the wide tiles: a full 256-row tile per expert or more
        assert T * k >= 256 * E, name
    router_bias = None
    if rb == "hot5":
        router_bias = np.full(E, -30.0, np.float32)
        router_bias[5] = 30.0
    inp = gen.make_inputs_custom(T, d, E, k, H, scoring, dtype, seed=T + E + k,
                                 sel_bias_var=sbv, router_bias=router_bias)
    res = run_layer(inp)
    rep = check_layer(inp, res)
    print(f"{name}: {rep}")
    if rb == "hot5":
        assert res["expert_counts"][5] == T


LARGE = [
    # beyond the workloads' sizes: 65536 assignment rows over 64 experts (row tiles of 256 narrow
    # tiles), and 32768 tokens over 16 experts (the wide gate/up tiles, 11 rounds of block slots),
    # checked on sampled tokens
    ("32k-top2-of-64", 32768, 1024, 64, 2, 512, orc.SELECTED_SOFTMAX, 0.5),
    ("32k-top1-of-16", 32768, 2048, 16, 1, 2816, orc.SOFTMAX, None),
]


@pytest.mark.parametrize("case", LARGE, ids=[c[0] for c in LARGE])
def test_layer_large_prefill(case):
    name, T, d, E, k, H, scoring, sbv = case
    inp = gen.make_inputs_custom(T, d, E, k, H, scoring, "bf16", seed=11, sel_bias_var=sbv)
    res = run_layer(inp, with_logits=False)
    ids, counts = res["topk_ids"], res["expert_counts"]
    assert ids.min() >= 0 and ids.max() < E
    np.testing.assert_array_equal(counts, np.bincount(ids.ravel(), minlength=E))
    rep = check_layer(inp, res, tokens=_sample(T, 384, seed=5))
    print(f"{name}: {rep}")


def test_layer_T0_is_noop():
    import torch
    from expert_routing_grouped_moe_amd import moe
    inp = gen.make_inputs_custom(4, 128, 8, 1, 128, orc.SOFTMAX, "bf16", seed=1)
    dev = upload(inp)
    y = torch.full((0, 128), 7.0, device=DEV)
    moe.moe_layer_forward(dev["x"][:0], dev["w_router"], dev["w_gate"], dev["w_up"], dev["w_down"],
                          1, "softmax", y=y)
    torch.cuda.synchronize()


@pytest.mark.parametrize("name", ["zonos2-decode", "zonos3mini-decode-cfg", "zonos3mini-prefill",
                                  "zonos2-skewed-prefill"])
def test_layer_deterministic(name):
    inp = gen.make_inputs(name)
    dev = upload(inp)
    a = run_layer(inp, dev)
    b = run_layer(inp, dev)
    for key in ("y", "topk_ids", "topk_w", "expert_counts", "logits"):
        np.testing.assert_array_equal(a[key], b[key], err_msg=key)


@pytest.mark.parametrize("name", ["zonos2-decode", "zonos3mini-decode-cfg", "tiny-fp32"])
def test_layer_graph_replay(name):
    """The fused call captured in a HIP graph and replayed; every replay equals the eager run."""
    import torch
    from expert_routing_grouped_moe_amd import moe
    inp = gen.make_inputs(name)
    dev = upload(inp)
    T, d, E, H, k = inp.T, inp.d, inp.E, inp.H, inp.k
    y = torch.empty((T, d), dtype=torch.float32, device=DEV)
    ws = torch.empty(moe.moe_workspace_size(T, d, E, H, k, 1 if inp.dtype == "bf16" else 0),
                     dtype=torch.uint8, device=DEV)
    args = moe.make_layer_args(dev["x"], dev["w_router"], dev["w_gate"], dev["w_up"],
                               dev["w_down"], k, inp.scoring, y, dev["router_bias"],
                               dev["sel_bias"])
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        moe.moe_layer_forward(dev["x"], dev["w_router"], dev["w_gate"], dev["w_up"], dev["w_down"],
                              k, inp.scoring, y=y, workspace=ws, args=args)
    torch.cuda.synchronize()
    eager = y.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        moe.moe_layer_forward(dev["x"], dev["w_router"], dev["w_gate"], dev["w_up"], dev["w_down"],
                              k, inp.scoring, y=y, workspace=ws, args=args)
    for i in range(4):
        y.fill_(float("nan"))
        ws.fill_(0xAB)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, eager), f"replay {i} differs"
