"""Shared helpers of the GPU parity tests: upload of the seeded inputs and the comparison of a
layer run against the fp64 oracle (with the near-tie rule for routing decided in fp32)."""
from itertools import combinations

import numpy as np
import torch

import oracle.moe_oracle as orc
from expert_routing_grouped_moe_amd import inputs as gen

DEV = "cuda:0"

# max |y_gpu - y_ref| <= TOL * RMS(y_ref): bf16 weights/activations with fp32 accumulation, and
# the fp32 configuration ("1e-5 relative", normalised by the output RMS because an elementwise
# relative error is ill-posed near zero).
TOL = {"bf16": 2e-2, "f32": 1e-5}
W_ABS_TOL = 2e-6  # routing weights from identical fp32 logits: fp32 exp and a <= 256-term sum


def upload(inp: gen.MoeInputs) -> dict:
    def dev(key):
        if inp.dtype == "bf16":
            return torch.from_numpy(inp.bits[key].view(np.int16)).view(torch.bfloat16).to(DEV)
        return torch.from_numpy(np.ascontiguousarray(getattr(inp, key))).to(DEV)

    out = {key: dev(key) for key in ("x", "w_router", "w_gate", "w_up", "w_down")}
    for key in ("router_bias", "sel_bias"):
        v = getattr(inp, key)
        out[key] = None if v is None else torch.from_numpy(v).to(DEV)
    return out


def run_layer(inp: gen.MoeInputs, dev=None, with_logits=True):
    from expert_routing_grouped_moe_amd import moe
    dev = dev or upload(inp)
    T, E, k = inp.T, inp.E, inp.k
    outs = dict(
        logits=torch.empty((T, E), dtype=torch.float32, device=DEV) if with_logits else None,
        topk_ids=torch.empty((T, k), dtype=torch.int32, device=DEV),
        topk_w=torch.empty((T, k), dtype=torch.float32, device=DEV),
        expert_counts=torch.empty((E,), dtype=torch.int32, device=DEV),
    )
    y = moe.moe_layer_forward(dev["x"], dev["w_router"], dev["w_gate"], dev["w_up"], dev["w_down"],
                              k, inp.scoring, router_bias=dev["router_bias"],
                              sel_bias=dev["sel_bias"], **outs)
    torch.cuda.synchronize()
    res = {key: (None if v is None else v.cpu().numpy()) for key, v in outs.items()}
    res["y"] = y.cpu().numpy()
    return res


def candidate_selections(s_row, k, band):
    """Every ordered-by-oracle k-set an fp32 evaluation within `band` of the fp64 scores could
    pick: experts clearly above the k-th score are in, those within the band compete."""
    order = sorted(range(len(s_row)), key=lambda e: (-s_row[e], e))
    kth = s_row[order[k - 1]]
    sure = [e for e in order if s_row[e] > kth + band]
    near = [e for e in order if abs(s_row[e] - kth) <= band]
    need = k - len(sure)
    if need <= 0 or need > len(near):
        return [tuple(order[:k])]
    return [tuple(sure) + c for c in combinations(near, need)]


def check_layer(inp: gen.MoeInputs, res: dict, tokens=None, tol=None):
    """Compare a layer run with the oracle on `tokens` (default: all). Returns a report dict."""
    T, E, k = inp.T, inp.E, inp.k
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    x = inp.x[tokens]
    L64 = orc.router_logits_ref(x, inp.w_router, inp.router_bias)
    s64 = L64 if inp.sel_bias is None else L64 + inp.sel_bias.astype(np.float64)[None, :]
    B = orc.logit_error_bound(x, inp.w_router, inp.router_bias, inp.sel_bias)
    ids_gpu = res["topk_ids"][tokens]
    w_gpu = res["topk_w"][tokens]
    y_gpu = res["y"][tokens].astype(np.float64)

    if res.get("logits") is not None:
        err = np.abs(res["logits"][tokens].astype(np.float64) - L64)
        assert (err <= B[:, None]).all(), f"router logits outside the fp32 bound: {err.max()}"

    # a token is decided when no two of its k+1 best fp64 scores are within 2B of each other
    srt = -np.sort(-s64, axis=1)
    top = srt[:, :min(k + 1, E)]
    gaps = -np.diff(top, axis=1) if top.shape[1] > 1 else np.full((len(tokens), 1), np.inf)
    decided = (gaps > 2.0 * B[:, None]).all(axis=1)

    ref = orc.layer_ref(x, inp.w_router, inp.w_gate, inp.w_up, inp.w_down, k, inp.scoring,
                        router_bias=inp.router_bias, sel_bias=inp.sel_bias)
    y_ref = ref["y"].copy()
    w_ref = ref["w"].copy()
    bad = np.nonzero(decided & (ids_gpu != ref["ids"]).any(axis=1))[0]
    assert len(bad) == 0, f"routing differs on decided tokens {tokens[bad][:8]}"

    n_undecided = 0
    for i in np.nonzero(~decided)[0]:
        n_undecided += 1
        cands = candidate_selections(s64[i], k, 2.0 * B[i])
        got = set(int(v) for v in ids_gpu[i])
        match = [c for c in cands if set(c) == got]
        assert match, f"token {tokens[i]}: selection {sorted(got)} not among near-tied {cands}"
        sel = np.array([list(match[0])])
        alt = orc.layer_ref(x[i:i + 1], inp.w_router, inp.w_gate, inp.w_up, inp.w_down, k,
                            inp.scoring, router_bias=inp.router_bias, sel_bias=inp.sel_bias,
                            selection=sel)
        y_ref[i] = alt["y"][0]
        # compare weights slot by slot in the GPU's slot order
        wmap = {int(e): float(v) for e, v in zip(alt["ids"][0], alt["w"][0])}
        w_ref[i] = [wmap[int(e)] for e in ids_gpu[i]]

    w_err = np.abs(w_gpu.astype(np.float64) - w_ref)
    w_bound = W_ABS_TOL + B[:, None]
    assert (w_err <= w_bound).all(), f"routing weights off by {w_err.max()}"
    if res.get("expert_counts") is not None and len(tokens) == T:
        np.testing.assert_array_equal(res["expert_counts"],
                                      np.bincount(res["topk_ids"].ravel(), minlength=E))
        if decided.all():
            np.testing.assert_array_equal(res["expert_counts"], ref["counts"])

    tol = TOL[inp.dtype] if tol is None else tol
    rms = float(np.sqrt(np.mean(y_ref ** 2)))
    err = float(np.abs(y_gpu - y_ref).max())
    assert err <= tol * rms, f"max|y err| = {err:.3e} > {tol} * RMS {rms:.3e} (ratio {err / rms:.3e})"
    return dict(err_over_rms=err / rms, undecided=n_undecided, tokens=len(tokens))
