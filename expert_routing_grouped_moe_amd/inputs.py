"""Seeded synthetic inputs for the MoE layer (router -> top-k -> dispatch -> SwiGLU experts -> combine).

This module only draws numbers. It holds none of the layer's arithmetic: no logits, no ranking,
no softmax, no FFN. Both the fp64 oracle (through the tests) and the HIP path take their inputs
from here, so neither side can influence what the other is checked on.

Recipe (the same for every workload):
  * generator: numpy ``Generator(PCG64(seed))``; fp32 standard normals (``standard_normal(...,
    dtype=float32)``), drawn in the fixed order x, W_router, W_gate, W_up, W_down, sel_bias;
  * scaling: ``N(0, v)`` means variance v, so each draw is multiplied by ``sqrt(v)`` in fp32;
    x ~ N(0,1); W_router, W_gate, W_up ~ N(0, 1/d); W_down ~ N(0, 1/H);
  * bf16 workloads round every fp32 value to bf16 with round-to-nearest-even; the fp32 copy kept
    here then holds exactly the bf16 value, so both sides read identical numbers;
  * the selection bias (top-2-of-64 SelectedSoftmax workloads) is drawn last, ~N(0, 0.5), fp32;
  * the skewed ZONOS2 prefill gets a router bias that is not drawn: experts 14 and 15 get -30
    (they never win) and expert 0 gets beta, where beta solves
    P(Z0 + beta > max of 13 other iid N(0,1)) = 0.40. The router logits of a token are iid N(0,1)
    across experts for x ~ N(0,1) and W_router ~ N(0,1/d), so expert 0 then takes ~40% of tokens.

Shapes follow the ZONOS2 / ZONOS3-Mini MoE blocks: ZONOS2 has 16 experts with top-1 routing at
width 2048 (zonos2.cpp INTERNALS, "Model architecture" table, MoE and Dims rows); ZONOS3-Mini has a
top-2-of-64 MoE at width 1024 (audio.cpp PR #1271, "Summary"). Expert hidden sizes (2816, 512)
are not printed on the pages and are taken as given workload parameters.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

SOFTMAX = "softmax"
SELECTED_SOFTMAX = "selected_softmax"


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    E: int
    k: int
    H: int
    scoring: str
    dtype: str  # "f32" or "bf16"
    seed: int
    sel_bias_var: Optional[float] = None
    skew_hot_share: Optional[float] = None  # share of tokens expert 0 should win
    skew_dead: tuple = ()  # experts given router bias -30
    shape: str = "decode"  # "decode" or "prefill" (what the step stands for)


WORKLOADS = {
    "tiny-fp32": Workload("tiny-fp32", T=64, d=128, E=8, k=1, H=256, scoring=SOFTMAX,
                          dtype="f32", seed=0, shape="decode"),
    "zonos2-decode": Workload("zonos2-decode", T=64, d=2048, E=16, k=1, H=2816, scoring=SOFTMAX,
                              dtype="bf16", seed=1, shape="decode"),
    "zonos3mini-decode-cfg": Workload("zonos3mini-decode-cfg", T=64, d=1024, E=64, k=2, H=512,
                                      scoring=SELECTED_SOFTMAX, dtype="bf16", seed=2,
                                      sel_bias_var=0.5, shape="decode"),
    "zonos3mini-prefill": Workload("zonos3mini-prefill", T=4096, d=1024, E=64, k=2, H=512,
                                   scoring=SELECTED_SOFTMAX, dtype="bf16", seed=3,
                                   sel_bias_var=0.5, shape="prefill"),
    "zonos2-skewed-prefill": Workload("zonos2-skewed-prefill", T=8192, d=2048, E=16, k=1, H=2816,
                                      scoring=SOFTMAX, dtype="bf16", seed=4,
                                      skew_hot_share=0.40, skew_dead=(14, 15), shape="prefill"),
    # ZONOS2's one top-2 layer (zonos2.cpp INTERNALS, "Model architecture" table, MoE row: top-2
    # only on layer 26), prob-weighted with no renormalisation: the SOFTMAX mode at k = 2
    "zonos2-layer26-decode": Workload("zonos2-layer26-decode", T=64, d=2048, E=16, k=2, H=2816,
                                      scoring=SOFTMAX, dtype="bf16", seed=5, shape="decode"),
}
WORKLOAD_ORDER = list(WORKLOADS)


@dataclass
class MoeInputs:
    """Host copies of one layer's inputs. Float arrays are fp32 and, for bf16 workloads, hold
    exactly the bf16 values whose raw bits are in the matching ``*_bits`` (uint16) arrays."""
    T: int
    d: int
    E: int
    k: int
    H: int
    scoring: str
    dtype: str
    x: np.ndarray
    w_router: np.ndarray
    w_gate: np.ndarray
    w_up: np.ndarray
    w_down: np.ndarray
    router_bias: Optional[np.ndarray] = None
    sel_bias: Optional[np.ndarray] = None
    bits: dict = field(default_factory=dict)
    name: str = "custom"


def bf16_round_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern, round to nearest, ties to even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(rng: np.random.Generator, shape, var: float) -> np.ndarray:
    a = rng.standard_normal(shape, dtype=np.float32)
    a *= np.float32(math.sqrt(var))
    return a


def _phi(z):
    return np.exp(-0.5 * z * z) / math.sqrt(2.0 * math.pi)


def _Phi(z):
    from scipy.special import ndtr
    return ndtr(z)


def hot_expert_beta(share: float, n_rivals: int) -> float:
    """beta with P(Z0 + beta > max of n_rivals iid N(0,1)) = share, Z0 ~ N(0,1).
    Plain quadrature of  int phi(z) Phi(z + beta)^n dz  plus bisection (a property of the
    input distribution, not of the layer)."""
    z = np.linspace(-12.0, 12.0, 24001)
    dz = z[1] - z[0]
    pz = _phi(z)

    def win(beta):
        return float(np.sum(pz * _Phi(z + beta) ** n_rivals) * dz)

    lo, hi = -10.0, 10.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if win(mid) < share:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def make_inputs_custom(T: int, d: int, E: int, k: int, H: int, scoring: str, dtype: str, seed: int,
                       sel_bias_var: Optional[float] = None,
                       router_bias: Optional[np.ndarray] = None,
                       name: str = "custom") -> MoeInputs:
    """Draw one layer's inputs with the recipe in the module docstring."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = _normal(rng, (T, d), 1.0)
    w_router = _normal(rng, (E, d), 1.0 / d)
    w_gate = _normal(rng, (E, H, d), 1.0 / d)
    w_up = _normal(rng, (E, H, d), 1.0 / d)
    w_down = _normal(rng, (E, d, H), 1.0 / H)
    sel_bias = None
    if sel_bias_var is not None:
        sel_bias = _normal(rng, (E,), sel_bias_var)
    inp = MoeInputs(T=T, d=d, E=E, k=k, H=H, scoring=scoring, dtype=dtype, x=x,
                    w_router=w_router, w_gate=w_gate, w_up=w_up, w_down=w_down,
                    router_bias=None if router_bias is None else
                    np.ascontiguousarray(router_bias, dtype=np.float32),
                    sel_bias=sel_bias, name=name)
    if dtype == "bf16":
        for key in ("x", "w_router", "w_gate", "w_up", "w_down"):
            b = bf16_round_bits(getattr(inp, key))
            inp.bits[key] = b
            setattr(inp, key, bf16_bits_to_f32(b))
    elif dtype != "f32":
        raise ValueError(f"unknown dtype {dtype}")
    return inp


def skew_router_bias(E: int, hot_share: float, dead) -> np.ndarray:
    b = np.zeros(E, dtype=np.float32)
    for e in dead:
        b[e] = np.float32(-30.0)
    rivals = E - len(dead) - 1
    b[0] = np.float32(hot_expert_beta(hot_share, rivals))
    return b


def make_inputs(workload: str, seed: Optional[int] = None, T: Optional[int] = None) -> MoeInputs:
    """Inputs of a named workload. ``T`` may shrink the token count (the weights stay as drawn
    for the full workload only when T is unchanged: the draw of x comes first)."""
    w = WORKLOADS[workload]
    rb = None
    if w.skew_hot_share is not None:
        rb = skew_router_bias(w.E, w.skew_hot_share, w.skew_dead)
    return make_inputs_custom(w.T if T is None else T, w.d, w.E, w.k, w.H, w.scoring, w.dtype,
                              w.seed if seed is None else seed, sel_bias_var=w.sel_bias_var,
                              router_bias=rb, name=w.name)


def make_logits(T: int, E: int, seed: int, kind: str = "normal") -> np.ndarray:
    """fp32 router logits [T,E] for routing-only tests, including adversarial patterns:
    'normal' iid N(0,1); 'ties' values on a coarse grid (many exact ties); 'equal' all rows
    constant; 'signed_zero' a mix of +0.0 and -0.0 with a few positives; 'neg_inf' rows with
    -inf entries (at least k finite per row is the caller's job)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if kind == "normal":
        return rng.standard_normal((T, E), dtype=np.float32)
    if kind == "ties":
        return (rng.integers(-3, 4, size=(T, E)).astype(np.float32) * np.float32(0.5))
    if kind == "equal":
        v = rng.standard_normal((T, 1), dtype=np.float32)
        return np.repeat(v, E, axis=1)
    if kind == "signed_zero":
        a = np.where(rng.random((T, E)) < 0.5, np.float32(0.0), np.float32(-0.0)).astype(np.float32)
        pos = rng.random((T, E)) < 0.05
        a[pos] = np.float32(1.0)
        return a
    if kind == "neg_inf":
        a = rng.standard_normal((T, E), dtype=np.float32)
        a[rng.random((T, E)) < 0.3] = -np.inf
        return a
    raise ValueError(kind)
