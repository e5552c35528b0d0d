"""moe_layer_forward_noalloc (the layer on the library's fixed scratch array, for callers that
cannot allocate) against moe_layer_forward with its own workspace, through the C ABI: identical
outputs on consecutive calls that reuse the same array, each call smaller than the one before."""
import ctypes

import numpy as np
import pytest

from expert_routing_grouped_moe_amd import inputs as gen

from _parity import DEV, check_layer, upload

pytestmark = pytest.mark.gpu

# largest first: every later call finds the previous, larger call's data in the array
SEQUENCE = ["zonos2-skewed-prefill", "zonos3mini-prefill", "zonos3mini-decode-cfg", "tiny-fp32"]


def _outputs(inp):
    import torch
    T, E, k = inp.T, inp.E, inp.k
    return dict(y=torch.empty((T, inp.d), dtype=torch.float32, device=DEV),
                topk_ids=torch.empty((T, k), dtype=torch.int32, device=DEV),
                topk_w=torch.empty((T, k), dtype=torch.float32, device=DEV),
                expert_counts=torch.empty((E,), dtype=torch.int32, device=DEV))


def test_noalloc_equals_layer_forward_on_consecutive_calls():
    import torch
    from expert_routing_grouped_moe_amd import moe
    for i, name in enumerate(SEQUENCE):
        inp = gen.make_inputs(name)
        dv = upload(inp)
        ref, got = _outputs(inp), _outputs(inp)
        moe.moe_layer_forward(dv["x"], dv["w_router"], dv["w_gate"], dv["w_up"], dv["w_down"],
                              inp.k, inp.scoring, router_bias=dv["router_bias"],
                              sel_bias=dv["sel_bias"], **ref)
        for t in got.values():
            t.fill_(-7) if t.dtype == torch.int32 else t.fill_(float("nan"))
        args = moe.make_layer_args(dv["x"], dv["w_router"], dv["w_gate"], dv["w_up"], dv["w_down"],
                                   inp.k, inp.scoring, got["y"], dv["router_bias"], dv["sel_bias"],
                                   topk_ids=got["topk_ids"], topk_w=got["topk_w"],
                                   expert_counts=got["expert_counts"])
        st = moe.LIB.moe_layer_forward_noalloc(ctypes.byref(args), moe._stream(None))
        assert st == moe.MOE_OK, (name, st)
        torch.cuda.synchronize()
        for key in ref:
            assert torch.equal(ref[key], got[key]), (name, key)
        # and the oracle's bar on the first call and on the last, smallest one
        if i in (0, len(SEQUENCE) - 1):
            res = {key: v.cpu().numpy() for key, v in got.items()}
            print(name, check_layer(inp, res))


def test_noalloc_refuses_sizes_past_the_array():
    import torch
    from expert_routing_grouped_moe_amd import moe
    T, d, E, H, k = 16384, 2048, 16, 2816, 1
    x = torch.zeros((T, d), dtype=torch.bfloat16, device=DEV)
    wr = torch.zeros((E, d), dtype=torch.bfloat16, device=DEV)
    wg = torch.zeros((E, H, d), dtype=torch.bfloat16, device=DEV)
    wd = torch.zeros((E, d, H), dtype=torch.bfloat16, device=DEV)
    y = torch.full((T, d), 3.0, device=DEV)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_layer_forward_noalloc(x, wr, wg, wg, wd, k, "softmax", y=y)
    assert ei.value.status == moe.MOE_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((y == 3.0).all())                       # nothing was enqueued
