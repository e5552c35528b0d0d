"""One GPU's share of expert parallelism at its real shape: with the skewed prefill's 16 experts
split over 8 GPUs (2 each), the GPU that owns experts 0 and 1 runs moe_expert_ffn on the ~3750
token rows routed to them (expert 0 takes ~40 % of all tokens, so this is the busiest shard). The
rows are those the oracle's routing sends there; the shard's expert outputs are checked against
the oracle on a sample of its tokens and, per expert, as a whole against the FFN of the same
rows."""
import numpy as np
import pytest

import oracle.moe_oracle as orc
from expert_routing_grouped_moe_amd import inputs as gen

from _parity import DEV, TOL, upload

pytestmark = pytest.mark.gpu

G = 8                                     # GPUs the 16 experts are split over


def _shard(inp, g):
    """Tokens of shard g (experts [g E/G, (g + 1) E/G)) under the oracle's routing, their local
    expert ids and the local grouping."""
    L = orc.router_logits_ref(inp.x, inp.w_router, inp.router_bias)
    ids = orc.select_topk_ref(L, inp.k)                       # [T, 1]
    per = inp.E // G
    lo = g * per
    tokens = np.nonzero((ids[:, 0] >= lo) & (ids[:, 0] < lo + per))[0]
    local = (ids[tokens] - lo).astype(np.int64)
    off, rows, pos = orc.permute_ref(local, per)
    return tokens, local, off, rows, pos, lo, per


def test_ep8_hot_shard_expert_ffn():
    import torch
    from expert_routing_grouped_moe_amd import moe
    inp = gen.make_inputs("zonos2-skewed-prefill")
    tokens, local, off, rows, pos, lo, per = _shard(inp, 0)
    counts = np.diff(off)
    assert counts[0] > 0.35 * inp.T and counts.sum() == len(tokens)   # the hot shard
    dev = upload(inp)
    x_sh = dev["x"][torch.from_numpy(tokens).to(DEV)].contiguous()
    wg = dev["w_gate"][lo:lo + per].contiguous()
    wu = dev["w_up"][lo:lo + per].contiguous()
    wd = dev["w_down"][lo:lo + per].contiguous()
    t32 = lambda a: torch.from_numpy(a.astype(np.int32)).to(DEV)
    eo = moe.moe_expert_ffn(x_sh, wg, wu, wd, 1, t32(off), t32(rows))
    torch.cuda.synchronize()
    eo = eo.cpu().numpy()
    # oracle on a sample of the shard's tokens (all of expert 1's, 400 of expert 0's)
    rng = np.random.default_rng(8)
    e0 = np.nonzero(local[:, 0] == 0)[0]
    e1 = np.nonzero(local[:, 0] == 1)[0]
    pick = np.sort(np.concatenate([rng.choice(e0, 400, replace=False), e1]))
    s_off, s_rows, s_pos = orc.permute_ref(local[pick], per)
    xs = inp.x[tokens[pick]]
    ref = orc.expert_ffn_ref(xs, inp.w_gate[lo:lo + per], inp.w_up[lo:lo + per],
                             inp.w_down[lo:lo + per], s_off, s_rows, 1)
    got = eo[pos[pick]]                       # the sampled tokens' rows of the shard's output
    want = ref[s_pos]
    rms = float(np.sqrt(np.mean(want ** 2)))
    err = float(np.abs(got - want).max())
    print(f"shard rows {counts.tolist()}, sampled {len(pick)}, max|err|/rms = {err / rms:.3e}")
    assert err <= TOL["bf16"] * rms
