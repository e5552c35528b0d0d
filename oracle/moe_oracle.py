"""fp64 CPU oracle of the ZONOS2 / ZONOS3-Mini mixture-of-experts layer.

TEST INFRASTRUCTURE. Only the tests, the package's smoke check and the benchmark's CPU-baseline
leg may import this module. The library never calls it, and it shares no code, constant or helper
with the HIP implementation: it is plain numpy written from the definitions below.

What the layer computes (one token t, E experts, k of them selected):
  1. router logits   L[t,e] = sum_i x[t,i] * Wr[e,i] + b_r[e]      (b_r optional)
  2. rank scores     s[t,e] = L[t,e] + sel_bias[e]  (SelectedSoftmax), else s = L
  3. selection       the k experts with the largest s, ties to the lowest expert index,
                     slot 0 holding the best
  4. weights         SOFTMAX (ZONOS2): softmax over all E logits, each selected expert weighted
                     by its full probability, no renormalisation (zonos2.cpp INTERNALS,
                     "Model architecture" table, Router row: prob-weighted no-renorm top-k).
                     SELECTED_SOFTMAX (ZONOS3-Mini): rank by raw logit plus selection bias, then
                     softmax over the selected experts' logits only; the bias does not enter the
                     weights (audio.cpp PR #1271, "Framework change", MoeScoring::SelectedSoftmax).
                     SIGMOID: rank by logit, weight each selected expert by sigmoid(logit), no
                     renormalisation (same page and section: the pre-ranking sigmoid mode; ranking
                     on the logit is ranking on sigmoid(logit) in exact arithmetic).
  5. dispatch        counts, exclusive-scan offsets, assignment rows r = t*k + j grouped by
                     expert in ascending r, and the inverse position of every row
  6. expert FFN      SwiGLU: o = Wd[e] (silu(Wg[e] x) * (Wu[e] x)), silu(z) = z / (1 + e^-z)
                     (audio.cpp PR #1271, "Summary": SwiGLU FFN; zonos2.cpp INTERNALS,
                     "Recommended: F16 spine + K-quant experts": gate/up/down expert stacks)
  7. combine         y[t] = sum_j w[t,j] * o[t,j], fp32 output stream in the library
                     (zonos2.cpp INTERNALS, "Notes": activation/residual streams are F32).

Everything floating is fp64 with no intermediate rounding, except where the library contract fixes
fp32: ranking on given fp32 logits, where ``L + sel_bias`` is one fp32 round-to-nearest-even add
(numpy float32 addition is exactly that), and the int8 weight quantisation below, whose scale and
quotient are fp32 operations so that the integer codes are defined exactly.

Quantised expert weights (decode path; the ZONOS2-4bit MLX card and zonos2.cpp INTERNALS run
quantised expert stacks, "Performance notes" / "Recommended: F16 spine + K-quant experts"): each
weight row (one output feature of one expert) is quantised symmetrically to int8,
  s = fl32(max_i |w_i| / 127),   q_i = clamp(rint(fl32(w_i / s)), -127, 127)   (ties to even),
an all-zero row getting s = 0, q = 0; the layer then uses the weights s * q exactly.
The 4-bit form follows the same card's recipe for the experts (affine, 4 bits, groups of 64 along
the reduction index, ZONOS2-4bit card, "Quantization recipe"). The pages name the scheme but do not
spell out its arithmetic; the reading taken is the plain affine one, with the scale and bias kept as
bf16 (the model's dtype):
  lo, hi = min, max of the group;  s = bf16(fl32(fl32(hi - lo) / 15));  b = bf16(lo);
  q_i = clamp(rint(fl32(fl32(w_i - b) / s)), 0, 15)   (ties to even; s = 0 gives q = 0),
and the layer computes with the weights s * q + b exactly. bf16() is round-to-nearest-even.

Storage orders (the library's own, no arithmetic): the packed 4-bit code order and the
fragment-major order of bf16 values, int8 codes or packed 4-bit codes (pack_frag_ref), a pure
reordering of bytes so that each load instruction of the decode kernels reads one kilobyte.

Pins (checked by the CPU tests against values the mathematics fixes, not against this code):
brute-force selection, closed-form softmax weights, exact fp32 rounding cases, dispatch
invariants, the E=1 layer equal to a dense SwiGLU FFN computed with torch's silu, the full layer
equal to a dense run-every-expert brute force, hand-encoded packed words, and the storage orders
read back the way the matrix cores take their operands, summed per row, equal to plain products.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

f64 = np.float64

SOFTMAX = "softmax"
SELECTED_SOFTMAX = "selected_softmax"
SIGMOID = "sigmoid"


# ----------------------------------------------------------------------------- routing (steps 1-4)

def router_logits_ref(x, w_router, router_bias=None):
    """Step 1 in fp64: L = x @ Wr^T (+ b_r)."""
    L = np.asarray(x, dtype=f64) @ np.asarray(w_router, dtype=f64).T
    if router_bias is not None:
        L = L + np.asarray(router_bias, dtype=f64)[None, :]
    return L


def rank_scores_fp32(logits32, sel_bias=None):
    """Step 2 on fp32 logits: s = fl32(L + sel_bias), a single IEEE RNE fp32 add."""
    L = np.asarray(logits32, dtype=np.float32)
    if sel_bias is None:
        return L.copy()
    return (L + np.asarray(sel_bias, dtype=np.float32)[None, :]).astype(np.float32)


def select_topk_ref(scores, k):
    """Step 3: per token, order experts by (score descending, index ascending) and keep k.
    -0.0 and +0.0 compare equal, so their order falls to the index."""
    s = np.asarray(scores)
    T, E = s.shape
    ids = np.empty((T, k), dtype=np.int64)
    idx = np.arange(E)
    for t in range(T):
        order = np.lexsort((idx, -s[t].astype(f64)))
        ids[t] = order[:k]
    return ids


def routing_weights_ref(logits, ids, scoring):
    """Step 4 in fp64 from the (unbiased) logits."""
    L = np.asarray(logits, dtype=f64)
    ids = np.asarray(ids)
    with np.errstate(invalid="ignore", over="ignore"):
        if scoring == SOFTMAX:
            m = L.max(axis=1, keepdims=True)
            p = np.exp(L - m)
            p = p / p.sum(axis=1, keepdims=True)
            return np.take_along_axis(p, ids, axis=1)
        if scoring == SELECTED_SOFTMAX:
            sel = np.take_along_axis(L, ids, axis=1)
            m = sel.max(axis=1, keepdims=True)
            q = np.exp(sel - m)
            return q / q.sum(axis=1, keepdims=True)
        if scoring == SIGMOID:
            sel = np.take_along_axis(L, ids, axis=1)
            return 1.0 / (1.0 + np.exp(-sel))
    raise ValueError(f"unknown scoring {scoring}")


def expert_counts_ref(ids, E):
    counts = np.zeros(E, dtype=np.int64)
    for e in np.asarray(ids).ravel():
        counts[e] += 1
    return counts


def route_ref(logits32, sel_bias, k, scoring):
    """The routing call on given fp32 logits: ids [T,k], fp64 weights [T,k], counts [E]."""
    if scoring != SELECTED_SOFTMAX and sel_bias is not None:
        raise ValueError("a selection bias is only defined for SelectedSoftmax")
    s = rank_scores_fp32(logits32, sel_bias)
    ids = select_topk_ref(s, k)
    w = routing_weights_ref(np.asarray(logits32, dtype=np.float32), ids, scoring)
    return ids, w, expert_counts_ref(ids, np.asarray(logits32).shape[1])


# ------------------------------------------------------------------ int8 expert weights (decode)

def quantize_rows_i8_ref(w):
    """Per-row symmetric int8 codes of a [..., K] weight stack: q (int8, same shape) and s (fp32,
    shape [...]). The scale and the quotient are fp32 operations (numpy float32 array division is
    the elementwise IEEE round-to-nearest-even quotient), the rounding is to nearest with ties to
    even (np.rint)."""
    w32 = np.asarray(w, dtype=np.float32)
    m = np.max(np.abs(w32), axis=-1)                       # exact
    s = np.where(m > 0, m / np.float32(127), np.float32(0)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1)).astype(np.float32)
    quot = (w32 / safe[..., None]).astype(np.float32)
    q = np.clip(np.rint(quot), -127, 127)
    q = np.where(s[..., None] > 0, q, 0).astype(np.int8)
    return q, s


def dequantize_rows_ref(q, s):
    """The weights the int8 layer computes with: s * q per row, exactly (fp64)."""
    return np.asarray(q, dtype=f64) * np.asarray(s, dtype=f64)[..., None]


def bf16_round_ref(v):
    """fp32 values rounded to the nearest bf16 (ties to even), returned as fp32."""
    bits = np.asarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (bits + 0x7FFF + ((bits >> 16) & 1)) >> 16
    return (rounded.astype(np.uint32) << 16).view(np.float32)


def quantize_groups_q4_ref(w, group=64):
    """4-bit affine codes of a [..., K] weight stack, groups of `group` along K: q (uint8, values
    0..15, same shape), s and b (fp32 holding bf16 values, shape [..., K / group]). Every step is
    the fp32 (or bf16) operation named in the module docstring, applied to whole arrays."""
    w32 = np.asarray(w, dtype=np.float32)
    K = w32.shape[-1]
    assert K % group == 0
    g = w32.reshape(w32.shape[:-1] + (K // group, group))
    lo = g.min(axis=-1)
    hi = g.max(axis=-1)
    span = (hi - lo).astype(np.float32)
    s = bf16_round_ref((span / np.float32(15)).astype(np.float32))
    b = bf16_round_ref(lo)
    safe = np.where(s > 0, s, np.float32(1)).astype(np.float32)
    diff = (g - b[..., None]).astype(np.float32)
    quot = (diff / safe[..., None]).astype(np.float32)
    q = np.clip(np.rint(quot), 0, 15)
    q = np.where(s[..., None] > 0, q, 0).astype(np.uint8)
    return q.reshape(w32.shape), s, b


def pack_q4_ref(q):
    """The library's storage order of 4-bit codes ([..., K] values 0..15, K a multiple of 128)
    as bytes [..., K / 2]: block j of 128 k holds 64 bytes; bytes 16 g .. 16 g + 15 of it are
    four little-endian dwords c = 0..3, dword c holding k = 128 j + 32 c + 8 g + i (i = 0..7) with
    i = 2 m in bits 4 m .. 4 m + 3 and i = 2 m + 1 in bits 16 + 4 m .. 19 + 4 m."""
    q = np.asarray(q, dtype=np.uint32)
    K = q.shape[-1]
    assert K % 128 == 0
    # [..., j, c, g, i] -> [..., j, g, c, i]
    v = q.reshape(q.shape[:-1] + (K // 128, 4, 4, 8)).swapaxes(-3, -2)
    dw = np.zeros(v.shape[:-1], dtype=np.uint32)
    for m in range(4):
        dw |= v[..., 2 * m] << np.uint32(4 * m)
        dw |= v[..., 2 * m + 1] << np.uint32(16 + 4 * m)
    return dw.astype("<u4").view(np.uint8).reshape(q.shape[:-1] + (K // 2,))


def pack_frag_ref(w, fmt="bf16"):
    """The library's fragment-major storage of an expert weight matrix for the decode kernels: the
    matrix is cut into slabs of 16 rows, and each slab is stored as consecutive 1024-byte chunks,
    chunk i holding the 64 sixteen-byte pieces that the 64 lanes of a wave take in the decode
    kernel's i-th load instruction over that slab, lane l's piece at byte 16 l; every piece comes
    from row l mod 16 of the slab. Which bytes of the row lane l takes depends on the format:
      bf16 [..., R, K] values (K a multiple of 32): the eight values k = 32 i + 8 (l div 16) + 0..7,
        the A operand of lane l in a 16 x 16 x 32 MFMA (matrix-core ISA operand layout);
      "i8" int8 codes [..., R, K] (K a multiple of 128): the 16 codes k = 128 (i div 2) +
        32 (l div 16) + 16 (i mod 2) + 0..15 (per 128-k block, lane group g takes the 32 codes from
        32 g on, as two loads);
      "q4" packed 4-bit bytes [..., R, K / 2] in the order of pack_q4_ref (K a multiple of 128):
        bytes 64 i + 16 (l div 16) + 0..15 of the packed row (block i, the codes lane group
        l div 16 needs).
    A pure reordering of the bytes. Returns the same shape and dtype."""
    w = np.asarray(w)
    R = w.shape[-2]
    assert R % 16 == 0
    lead, n = w.shape[:-2], w.ndim - 2
    if fmt == "bf16":
        K = w.shape[-1]
        assert K % 32 == 0
        v = w.reshape(lead + (R // 16, 16, K // 32, 4, 8))        # b, r16, i, g, value
        order = (n, n + 2, n + 3, n + 1, n + 4)                     # b, i, g, r16, value
    elif fmt == "i8":
        K = w.shape[-1]
        assert K % 128 == 0
        v = w.reshape(lead + (R // 16, 16, K // 128, 4, 2, 16))   # b, r16, block, g, half, code
        order = (n, n + 2, n + 4, n + 3, n + 1, n + 5)              # b, block, half, g, r16, code
    elif fmt == "q4":
        nb = w.shape[-1]
        assert nb % 64 == 0
        v = w.reshape(lead + (R // 16, 16, nb // 64, 4, 16))      # b, r16, block, g, byte
        order = (n, n + 2, n + 3, n + 1, n + 4)                     # b, block, g, r16, byte
    else:
        raise ValueError(fmt)
    v = v.transpose(tuple(range(n)) + order)
    return np.ascontiguousarray(v).reshape(w.shape)


def pack_q4_params_ref(s, b):
    """Per-group (scale, bias) as one uint32: bf16 bits of s in the low half, of b in the high."""
    sb = np.asarray(s, dtype=np.float32).view(np.uint32) >> np.uint32(16)
    bb = np.asarray(b, dtype=np.float32).view(np.uint32) >> np.uint32(16)
    return (sb | (bb << np.uint32(16))).astype(np.uint32)


def dequantize_groups_q4_ref(q, s, b, group=64):
    """The weights the 4-bit layer computes with: s * q + b per group, exactly (fp64)."""
    q64 = np.asarray(q, dtype=f64)
    K = q64.shape[-1]
    g = q64.reshape(q64.shape[:-1] + (K // group, group))
    out = g * np.asarray(s, dtype=f64)[..., None] + np.asarray(b, dtype=f64)[..., None]
    return out.reshape(q64.shape)


# ------------------------------------------------------------------------------ dispatch (step 5)

def permute_ref(ids, E):
    """Step 5 with plain loops: offsets [E+1], sorted_rows [T*k], row_pos [T*k]."""
    flat = [int(v) for v in np.asarray(ids).ravel()]
    counts = [0] * E
    for e in flat:
        counts[e] += 1
    offsets = [0] * (E + 1)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    fill = offsets[:E]
    fill = list(fill)
    sorted_rows = [0] * len(flat)
    row_pos = [0] * len(flat)
    for r, e in enumerate(flat):
        sorted_rows[fill[e]] = r
        row_pos[r] = fill[e]
        fill[e] += 1
    return (np.array(offsets, dtype=np.int64), np.array(sorted_rows, dtype=np.int64),
            np.array(row_pos, dtype=np.int64))


# ------------------------------------------------------------------------- experts (steps 6-7)

def silu_ref(z):
    z = np.asarray(z, dtype=f64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu_ffn_ref(xrows, wg, wu, wd):
    """One expert on a block of token rows: Wd (silu(Wg x) * (Wu x)), fp64."""
    X = np.asarray(xrows, dtype=f64)
    g = X @ np.asarray(wg, dtype=f64).T
    u = X @ np.asarray(wu, dtype=f64).T
    h = silu_ref(g) * u
    return h @ np.asarray(wd, dtype=f64).T


def expert_ffn_ref(x, w_gate, w_up, w_down, offsets, sorted_rows, k):
    """Step 6 over every expert group: expert_out [T*k, d] in grouped (sorted) order."""
    x = np.asarray(x)
    E = np.asarray(w_gate).shape[0]
    d = x.shape[1]
    out = np.zeros((len(sorted_rows), d), dtype=f64)
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a == b:
            continue
        toks = np.asarray(sorted_rows[a:b]) // k
        out[a:b] = swiglu_ffn_ref(x[toks], w_gate[e], w_up[e], w_down[e])
    return out


def combine_ref(expert_out, row_pos, w, k):
    """Step 7: y[t] = sum over slots j (in slot order) of w[t,j] * expert_out[row_pos[t*k+j]]."""
    w = np.asarray(w, dtype=f64)
    T = w.shape[0]
    eo = np.asarray(expert_out, dtype=f64)
    y = np.zeros((T, eo.shape[1]), dtype=f64)
    for t in range(T):
        for j in range(k):
            y[t] += w[t, j] * eo[int(row_pos[t * k + j])]
    return y


# ----------------------------------------------------------------------------- the whole layer

def layer_ref(x, w_router, w_gate, w_up, w_down, k, scoring, router_bias=None, sel_bias=None,
              selection=None):
    """Steps 1-7 in fp64. ``selection`` ([T,k] expert ids) replaces step 3 when given: it is how a
    near-tied token is re-evaluated at the choice another implementation made."""
    if scoring != SELECTED_SOFTMAX and sel_bias is not None:
        raise ValueError("a selection bias is only defined for SelectedSoftmax")
    E = np.asarray(w_router).shape[0]
    L = router_logits_ref(x, w_router, router_bias)
    s = L if sel_bias is None else L + np.asarray(sel_bias, dtype=f64)[None, :]
    ids = select_topk_ref(s, k) if selection is None else np.asarray(selection, dtype=np.int64)
    w = routing_weights_ref(L, ids, scoring)
    counts = expert_counts_ref(ids, E)
    offsets, sorted_rows, row_pos = permute_ref(ids, E)
    eo = expert_ffn_ref(x, w_gate, w_up, w_down, offsets, sorted_rows, k)
    y = combine_ref(eo, row_pos, w, k)
    return dict(logits=L, scores=s, ids=ids, w=w, counts=counts, offsets=offsets,
                sorted_rows=sorted_rows, row_pos=row_pos, expert_out=eo, y=y)


def layer_tokens_ref(x, w_router, w_gate, w_up, w_down, k, scoring, tokens, router_bias=None,
                     sel_bias=None, selection=None):
    """The layer output for a subset of tokens, each computed on its own (every step is per
    token except the dispatch bookkeeping, which does not change y)."""
    tokens = np.asarray(tokens, dtype=np.int64)
    sel = None if selection is None else np.asarray(selection)[tokens]
    return layer_ref(np.asarray(x)[tokens], w_router, w_gate, w_up, w_down, k, scoring,
                     router_bias=router_bias, sel_bias=sel_bias, selection=sel)


def dense_bruteforce_ref(x, w_router, w_gate, w_up, w_down, k, scoring, router_bias=None,
                         sel_bias=None):
    """Run every expert on every token, then mask and weight. Selection by a full Python sort,
    weights from the definitions, one token at a time. Small inputs only."""
    x = np.asarray(x, dtype=f64)
    T, d = x.shape
    E = np.asarray(w_router).shape[0]
    y = np.zeros((T, d), dtype=f64)
    for t in range(T):
        L = [float(np.dot(x[t], np.asarray(w_router[e], dtype=f64))) for e in range(E)]
        if router_bias is not None:
            L = [L[e] + float(router_bias[e]) for e in range(E)]
        s = L if sel_bias is None else [L[e] + float(sel_bias[e]) for e in range(E)]
        chosen = sorted(range(E), key=lambda e: (-s[e], e))[:k]
        if scoring == SOFTMAX:
            m = max(L)
            z = sum(math.exp(v - m) for v in L)
            wt = {e: math.exp(L[e] - m) / z for e in chosen}
        elif scoring == SIGMOID:
            # sigmoid(v) written without overflow either side: e^v / (1 + e^v) for v < 0
            wt = {e: (1.0 / (1.0 + math.exp(-L[e])) if L[e] >= 0
                      else math.exp(L[e]) / (1.0 + math.exp(L[e]))) for e in chosen}
        else:
            m = max(L[e] for e in chosen)
            z = sum(math.exp(L[e] - m) for e in chosen)
            wt = {e: math.exp(L[e] - m) / z for e in chosen}
        for e in range(E):
            mask = 1.0 if e in wt else 0.0
            o = swiglu_ffn_ref(x[t:t + 1], w_gate[e], w_up[e], w_down[e])[0]
            y[t] += mask * wt.get(e, 0.0) * o
    return y


# ------------------------------------------------------------------- near ties in the full layer

def logit_error_bound(x, w_router, router_bias=None, sel_bias=None):
    """Per-token bound B_t on |fp32 rank score - exact rank score| for ANY summation order of the
    fp32 dot product (Higham, Accuracy and Stability of Numerical Algorithms, Thm 3.1:
    |fl(x.w) - x.w| <= gamma_n sum |x_i w_i|, gamma_n = n u / (1 - n u), u = 2^-24), with one
    extra gamma term for the product rounding of fp32 operands and one fp32 rounding for each
    bias add."""
    x = np.asarray(x, dtype=f64)
    W = np.asarray(w_router, dtype=f64)
    d = x.shape[1]
    u = 2.0 ** -24
    n = d + 3
    gamma = n * u / (1.0 - n * u)
    absdot = np.abs(x) @ np.abs(W).T
    mag = absdot.copy()
    if router_bias is not None:
        mag = mag + np.abs(np.asarray(router_bias, dtype=f64))[None, :]
    if sel_bias is not None:
        mag = mag + np.abs(np.asarray(sel_bias, dtype=f64))[None, :]
    return gamma * mag.max(axis=1) + 4.0 * u * mag.max(axis=1)


def decided_tokens(scores64, k, bound):
    """True where the gap between the k-th and (k+1)-th best fp64 score exceeds 2*bound, i.e.
    every fp32 evaluation within the bound must pick the same k experts."""
    s = np.asarray(scores64, dtype=f64)
    T, E = s.shape
    if k >= E:
        return np.ones(T, dtype=bool)
    srt = -np.sort(-s, axis=1)
    gap = srt[:, k - 1] - srt[:, k]
    return gap > 2.0 * np.asarray(bound)


def selection_admissible(scores64, k, bound, ids):
    """Whether a selection could come from an fp32 evaluation whose rank scores are each within
    `bound` of the exact ones. Two such scores can swap order only when the exact ones lie within
    2*bound of each other, so, with kth the k-th best exact score, a selection is admissible when
    its k experts are distinct, every expert scoring above kth + 2*bound is among them (no k
    others can overtake it), and none scores below kth - 2*bound (it cannot overtake the k
    experts above it)."""
    s = np.asarray(scores64, dtype=f64)
    srt = -np.sort(-s, axis=1)
    kth = srt[:, k - 1]
    ok = np.ones(s.shape[0], dtype=bool)
    for t in range(s.shape[0]):
        sel = [int(v) for v in ids[t]]
        band = 2.0 * float(bound[t])
        if len(set(sel)) != k:
            ok[t] = False
            continue
        if any(s[t, e] < kth[t] - band for e in sel):
            ok[t] = False
            continue
        sure = [e for e in range(s.shape[1]) if s[t, e] > kth[t] + band]
        if any(e not in sel for e in sure):
            ok[t] = False
    return ok
