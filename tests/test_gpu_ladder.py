"""Graph ladder (moe_ladder_*): one captured graph of the layer per batch-size bucket. The rows
below T of a replayed bucket equal moe_layer_forward on the first T rows bit for bit when both take
the same kernel path, the expert counts cover those T rows only (not the bucket's padding rows),
the layer output matches the oracle, and buckets replay in any order."""
import numpy as np
import pytest

import oracle.moe_oracle as orc
from expert_routing_grouped_moe_amd import inputs as gen

from _parity import DEV, check_layer, upload

pytestmark = pytest.mark.gpu


def _direct(dv, inp, T):
    import torch
    from expert_routing_grouped_moe_amd import moe
    ids = torch.empty((T, inp.k), dtype=torch.int32, device=DEV)
    counts = torch.empty((inp.E,), dtype=torch.int32, device=DEV)
    y = moe.moe_layer_forward(dv["x"][:T], dv["w_router"], dv["w_gate"], dv["w_up"], dv["w_down"],
                              inp.k, inp.scoring, router_bias=dv["router_bias"],
                              sel_bias=dv["sel_bias"], topk_ids=ids, expert_counts=counts)
    torch.cuda.synchronize()
    return y.cpu().numpy(), ids.cpu().numpy(), counts.cpu().numpy()


def _ladder(dv, inp, buckets, stream, with_ids=True):
    import torch
    from expert_routing_grouped_moe_amd import moe
    ids = torch.empty((inp.T, inp.k), dtype=torch.int32, device=DEV) if with_ids else None
    counts = torch.full((inp.E,), -1, dtype=torch.int32, device=DEV)
    lad = moe.MoeGraphLadder(dv["x"], dv["w_router"], dv["w_gate"], dv["w_up"], dv["w_down"],
                             inp.k, inp.scoring, buckets, router_bias=dv["router_bias"],
                             sel_bias=dv["sel_bias"], topk_ids=ids, expert_counts=counts,
                             stream=stream)
    lad.counts = counts
    return lad, ids


CASES = [
    # name, workload or custom shape, buckets, T values to run (in this order)
    ("zonos3mini-decode-cfg", None, [1, 2, 4, 8, 16, 32, 64], [64, 1, 3, 13, 33, 8, 64]),
    ("zonos2-decode", None, [8, 16, 32, 64], [5, 64, 17]),
    ("prefill-shape", (2048, 256, 8, 2, 256, orc.SELECTED_SOFTMAX, 0.5), [512, 1024, 2048],
     [700, 2048, 513]),
    # ZONOS3-Mini widths with a largest batch past the split router's limit (256 tokens): the
    # workspace sized for 300 tokens must also hold the split router's partials of the smaller
    # buckets
    ("zonos3mini-widths-T300", (300, 1024, 64, 2, 512, orc.SELECTED_SOFTMAX, 0.5),
     [16, 64, 256, 300], [300, 16, 200, 64, 256]),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_ladder_rows_equal_direct_calls(case):
    import torch
    name, shape, buckets, ts = case
    if shape is None:
        inp = gen.make_inputs(name)
    else:
        T, d, E, k, H, scoring, sbv = shape
        inp = gen.make_inputs_custom(T, d, E, k, H, scoring, "bf16", seed=21, sel_bias_var=sbv)
    dv = upload(inp)
    stream = torch.cuda.Stream()
    lad, ids = _ladder(dv, inp, buckets, stream)
    try:
        for T in ts:
            with torch.cuda.stream(stream):
                used = lad.run(T, stream)
            stream.synchronize()
            assert used == min(b for b in buckets if b >= T)
            y_l = lad.y[:T].cpu().numpy()
            ids_l = ids[:T].cpu().numpy()
            counts_l = lad.counts.cpu().numpy()
            y_d, ids_d, counts_d = _direct(dv, inp, T)
            np.testing.assert_array_equal(ids_l, ids_d)
            np.testing.assert_array_equal(y_l, y_d)
            # the first T rows only, also when the bucket is larger
            np.testing.assert_array_equal(counts_l, np.bincount(ids_d.ravel(), minlength=inp.E))
            np.testing.assert_array_equal(counts_l, counts_d)
    finally:
        lad.close()


@pytest.mark.parametrize("name", ["zonos3mini-decode-cfg", "zonos2-decode"])
def test_ladder_counts_without_topk_ids(name):
    """With no topk_ids buffer the ids live in the workspace, at an offset that depends on the
    bucket; the recount after a padded replay must find them there."""
    import torch
    inp = gen.make_inputs(name)
    dv = upload(inp)
    stream = torch.cuda.Stream()
    lad, _ = _ladder(dv, inp, [8, 16, 64], stream, with_ids=False)
    try:
        for T in (5, 64, 11, 16, 1):
            with torch.cuda.stream(stream):
                lad.run(T, stream)
            stream.synchronize()
            _, ids_d, counts_d = _direct(dv, inp, T)
            np.testing.assert_array_equal(lad.counts.cpu().numpy(), counts_d)
            assert int(counts_d.sum()) == T * inp.k
    finally:
        lad.close()


def test_ladder_output_matches_oracle():
    import torch
    from expert_routing_grouped_moe_amd import moe
    inp = gen.make_inputs("zonos3mini-decode-cfg")
    dv = upload(inp)
    stream = torch.cuda.Stream()
    ids = torch.empty((inp.T, inp.k), dtype=torch.int32, device=DEV)
    w = torch.empty((inp.T, inp.k), dtype=torch.float32, device=DEV)
    lad = moe.MoeGraphLadder(dv["x"], dv["w_router"], dv["w_gate"], dv["w_up"], dv["w_down"],
                             inp.k, inp.scoring, [16, 32, 64], sel_bias=dv["sel_bias"],
                             topk_ids=ids, topk_w=w, stream=stream)
    try:
        T = 29                                # bucket 32: rows 29..31 are extra tokens
        with torch.cuda.stream(stream):
            lad.run(T, stream)
        stream.synchronize()
        res = {"y": lad.y.cpu().numpy(), "topk_ids": ids.cpu().numpy(), "topk_w": w.cpu().numpy()}
        print(check_layer(inp, res, tokens=np.arange(T)))
    finally:
        lad.close()


def test_ladder_rejects_T_beyond_largest_bucket():
    import torch
    from expert_routing_grouped_moe_amd import moe
    inp = gen.make_inputs("zonos3mini-decode-cfg")
    dv = upload(inp)
    stream = torch.cuda.Stream()
    lad, _ = _ladder(dv, inp, [8, 16], stream)
    try:
        with pytest.raises(moe.MoeError) as ei:
            lad.run(17, stream)
        assert ei.value.status == moe.MOE_ERR_SHAPE
        with pytest.raises(moe.MoeError):
            lad.run(0, stream)
    finally:
        lad.close()
