"""Python binding of libmoe.so (include/moe.h): argument marshalling only.

Each function takes torch tensors, checks device/dtype/shape/contiguity, allocates any output the
caller did not pass (torch owns all device memory), and calls the C entry point of the same name
on torch's current HIP stream. Every step of the computation runs in the library's HIP kernels;
there is no other implementation behind these names. If the library is missing the import fails.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, Structure, c_char_p, c_int, c_int32, c_size_t, c_uint32, c_void_p

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")

MOE_ABI_VERSION = 5  # include/moe.h; the library must report the same value

MOE_OK = 0
MOE_ERR_NULL = -1
MOE_ERR_SHAPE = -2
MOE_ERR_UNSUPPORTED = -3
MOE_ERR_WORKSPACE = -4
MOE_ERR_HIP = -5

MOE_F32 = 0
MOE_BF16 = 1
MOE_I8 = 2
MOE_Q4 = 3
MOE_BF16_FRAG = 4
MOE_I8_FRAG = 5
MOE_Q4_FRAG = 6

MOE_SCORING_SOFTMAX = 0
MOE_SCORING_SELECTED_SOFTMAX = 1
MOE_SCORING_SIGMOID = 2

SCORING = {"softmax": MOE_SCORING_SOFTMAX, "selected_softmax": MOE_SCORING_SELECTED_SOFTMAX,
           "sigmoid": MOE_SCORING_SIGMOID}

EXPORTS = ("moe_abi_version", "moe_status_string", "moe_workspace_size", "moe_router_logits",
           "moe_route", "moe_permute", "moe_expert_ffn", "moe_combine", "moe_layer_forward",
           "moe_quantize_rows_i8", "moe_quantize_groups_q4", "moe_ladder_create", "moe_ladder_run",
           "moe_ladder_destroy", "moe_layer_forward_noalloc", "moe_pack_weights_frag")

MOE_NOALLOC_SCRATCH_BYTES = 64 << 20

MOE_LADDER_MAX_BUCKETS = 256


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {moe_status_string(status)} (status {status})")


class MoeLayerArgs(Structure):
    _fields_ = [
        ("struct_size", c_uint32),
        ("T", c_int32), ("d", c_int32), ("E", c_int32), ("H", c_int32), ("k", c_int32),
        ("dtype", c_int32), ("scoring", c_int32),
        ("x", c_void_p), ("w_router", c_void_p), ("router_bias", c_void_p), ("sel_bias", c_void_p),
        ("w_gate", c_void_p), ("w_up", c_void_p), ("w_down", c_void_p), ("y", c_void_p),
        ("logits", c_void_p), ("topk_ids", c_void_p), ("topk_w", c_void_p),
        ("expert_counts", c_void_p),
        ("prof_events", c_void_p),   # void* const*: MOE_PROF_EVENTS hipEvent_t handles or NULL
        ("w_dtype", c_int32),
        ("w_gate_scale", c_void_p), ("w_up_scale", c_void_p), ("w_down_scale", c_void_p),
        ("y_dtype", c_int32),        # ABI 4: MOE_F32 or MOE_BF16
    ]


MOE_PROF_EVENTS = 5


def _load() -> ctypes.CDLL:
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is not built; run expert_routing_grouped_moe_amd/build.py "
                          "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(_LIB_PATH)
    lib.moe_abi_version.restype = c_int
    lib.moe_abi_version.argtypes = []
    lib.moe_status_string.restype = c_char_p
    lib.moe_status_string.argtypes = [c_int]
    lib.moe_workspace_size.restype = c_size_t
    lib.moe_workspace_size.argtypes = [c_int] * 6
    lib.moe_router_logits.restype = c_int
    lib.moe_router_logits.argtypes = [c_void_p, c_void_p, c_void_p, c_int, c_int, c_int, c_int,
                                      c_void_p, c_void_p]
    lib.moe_route.restype = c_int
    lib.moe_route.argtypes = [c_void_p, c_void_p, c_int, c_int, c_int, c_int, c_void_p, c_void_p,
                              c_void_p, c_void_p]
    lib.moe_permute.restype = c_int
    lib.moe_permute.argtypes = [c_void_p, c_void_p, c_int, c_int, c_int, c_void_p, c_void_p,
                                c_void_p, c_void_p]
    lib.moe_expert_ffn.restype = c_int
    lib.moe_expert_ffn.argtypes = [c_void_p, c_int, c_int, c_void_p, c_void_p, c_void_p, c_int,
                                   c_int, c_int, c_int, c_void_p, c_void_p, c_void_p, c_void_p,
                                   c_size_t, c_void_p]
    lib.moe_combine.restype = c_int
    lib.moe_combine.argtypes = [c_void_p, c_void_p, c_void_p, c_int, c_int, c_int, c_void_p,
                                c_int, c_void_p]
    lib.moe_layer_forward.restype = c_int
    lib.moe_layer_forward.argtypes = [POINTER(MoeLayerArgs), c_void_p, c_size_t, c_void_p]
    lib.moe_layer_forward_noalloc.restype = c_int
    lib.moe_layer_forward_noalloc.argtypes = [POINTER(MoeLayerArgs), c_void_p]
    lib.moe_quantize_rows_i8.restype = c_int
    lib.moe_quantize_rows_i8.argtypes = [c_void_p, ctypes.c_int64, c_int, c_int, c_void_p,
                                         c_void_p, c_void_p]
    lib.moe_quantize_groups_q4.restype = c_int
    lib.moe_quantize_groups_q4.argtypes = [c_void_p, ctypes.c_int64, c_int, c_int, c_void_p,
                                           c_void_p, c_void_p]
    lib.moe_pack_weights_frag.restype = c_int
    lib.moe_pack_weights_frag.argtypes = [c_void_p, ctypes.c_int64, c_int, c_int, c_void_p,
                                          c_void_p]
    lib.moe_ladder_create.restype = c_int
    lib.moe_ladder_create.argtypes = [POINTER(MoeLayerArgs), c_void_p, c_int, c_void_p, c_size_t,
                                      c_void_p, POINTER(c_void_p)]
    lib.moe_ladder_run.restype = c_int
    lib.moe_ladder_run.argtypes = [c_void_p, c_int, c_void_p, c_void_p]
    lib.moe_ladder_destroy.restype = None
    lib.moe_ladder_destroy.argtypes = [c_void_p]
    if lib.moe_abi_version() != MOE_ABI_VERSION:
        raise ImportError(f"{_LIB_PATH} reports ABI {lib.moe_abi_version()}, the binding expects "
                          f"{MOE_ABI_VERSION}; rebuild the library")
    return lib


LIB = _load()
LIB_PATH = _LIB_PATH


# ------------------------------------------------------------------------------------ helpers

def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        if torch.cuda.is_available():
            return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        return None
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _check(status: int, where: str):
    if status != MOE_OK:
        raise MoeError(status, where)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    raise TypeError(f"unsupported dtype {t.dtype}: x and weights are float32 or bfloat16")


def _need(t, name, shape, dtype=None):
    if t is None:
        return
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")


def _scoring_code(scoring) -> int:
    if isinstance(scoring, str):
        return SCORING[scoring]
    return int(scoring)


def _empty(shape, dtype, like):
    return torch.empty(shape, dtype=dtype, device=like.device)


# --------------------------------------------------------------------------------- entry points

def moe_abi_version() -> int:
    return LIB.moe_abi_version()


def moe_status_string(status: int) -> str:
    return LIB.moe_status_string(int(status)).decode()


def moe_workspace_size(T, d, E, H, k, dtype) -> int:
    return int(LIB.moe_workspace_size(T, d, E, H, k, dtype))


def moe_router_logits(x, w_router, router_bias=None, logits=None, stream=None):
    T, d = x.shape
    E = w_router.shape[0]
    dt = _dtype_code(x)
    _need(x, "x", (T, d))
    _need(w_router, "w_router", (E, d), x.dtype)
    _need(router_bias, "router_bias", (E,), torch.float32)
    if logits is None:
        logits = _empty((T, E), torch.float32, x)
    _need(logits, "logits", (T, E), torch.float32)
    _check(LIB.moe_router_logits(_ptr(x), _ptr(w_router), _ptr(router_bias), T, d, E, dt,
                                 _ptr(logits), _stream(stream)), "moe_router_logits")
    return logits


def moe_route(logits, k, scoring, sel_bias=None, topk_ids=None, topk_w=None, expert_counts=None,
              stream=None):
    T, E = logits.shape
    _need(logits, "logits", (T, E), torch.float32)
    _need(sel_bias, "sel_bias", (E,), torch.float32)
    topk_ids = _empty((T, k), torch.int32, logits) if topk_ids is None else topk_ids
    topk_w = _empty((T, k), torch.float32, logits) if topk_w is None else topk_w
    expert_counts = _empty((E,), torch.int32, logits) if expert_counts is None else expert_counts
    _need(topk_ids, "topk_ids", (T, k), torch.int32)
    _need(topk_w, "topk_w", (T, k), torch.float32)
    _need(expert_counts, "expert_counts", (E,), torch.int32)
    _check(LIB.moe_route(_ptr(logits), _ptr(sel_bias), T, E, k, _scoring_code(scoring),
                         _ptr(topk_ids), _ptr(topk_w), _ptr(expert_counts), _stream(stream)),
           "moe_route")
    return topk_ids, topk_w, expert_counts


def moe_permute(topk_ids, expert_counts, E, expert_offsets=None, sorted_rows=None, row_pos=None,
                stream=None):
    T, k = topk_ids.shape
    _need(topk_ids, "topk_ids", (T, k), torch.int32)
    _need(expert_counts, "expert_counts", (E,), torch.int32)
    expert_offsets = _empty((E + 1,), torch.int32, topk_ids) if expert_offsets is None else expert_offsets
    sorted_rows = _empty((T * k,), torch.int32, topk_ids) if sorted_rows is None else sorted_rows
    row_pos = _empty((T * k,), torch.int32, topk_ids) if row_pos is None else row_pos
    _need(expert_offsets, "expert_offsets", (E + 1,), torch.int32)
    _need(sorted_rows, "sorted_rows", (T * k,), torch.int32)
    _need(row_pos, "row_pos", (T * k,), torch.int32)
    _check(LIB.moe_permute(_ptr(topk_ids), _ptr(expert_counts), T, E, k, _ptr(expert_offsets),
                           _ptr(sorted_rows), _ptr(row_pos), _stream(stream)), "moe_permute")
    return expert_offsets, sorted_rows, row_pos


def moe_expert_ffn(x, w_gate, w_up, w_down, k, expert_offsets, sorted_rows, expert_out=None,
                   workspace=None, stream=None):
    T, d = x.shape
    E, H, _ = w_gate.shape
    dt = _dtype_code(x)
    _need(x, "x", (T, d))
    _need(w_gate, "w_gate", (E, H, d), x.dtype)
    _need(w_up, "w_up", (E, H, d), x.dtype)
    _need(w_down, "w_down", (E, d, H), x.dtype)
    _need(expert_offsets, "expert_offsets", (E + 1,), torch.int32)
    _need(sorted_rows, "sorted_rows", (T * k,), torch.int32)
    expert_out = _empty((T * k, d), torch.float32, x) if expert_out is None else expert_out
    _need(expert_out, "expert_out", (T * k, d), torch.float32)
    ws_bytes = moe_workspace_size(T, d, E, H, k, dt)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=x.device)
    _check(LIB.moe_expert_ffn(_ptr(x), T, d, _ptr(w_gate), _ptr(w_up), _ptr(w_down), E, H, k, dt,
                              _ptr(expert_offsets), _ptr(sorted_rows), _ptr(expert_out),
                              _ptr(workspace), workspace.numel(), _stream(stream)),
           "moe_expert_ffn")
    return expert_out


def _y_code(y) -> int:
    if y.dtype == torch.float32:
        return MOE_F32
    if y.dtype == torch.bfloat16:
        return MOE_BF16
    raise TypeError(f"y has dtype {y.dtype}: float32 or bfloat16")


def moe_combine(expert_out, row_pos, topk_w, y=None, stream=None, y_dtype=torch.float32):
    """y [T, d] = sum_j topk_w[:, j] * expert_out[row_pos[t*k + j]]; y is float32 or bfloat16
    (``y`` passed in decides, else ``y_dtype``)."""
    T, k = topk_w.shape
    d = expert_out.shape[1]
    _need(expert_out, "expert_out", (T * k, d), torch.float32)
    _need(row_pos, "row_pos", (T * k,), torch.int32)
    _need(topk_w, "topk_w", (T, k), torch.float32)
    y = _empty((T, d), y_dtype, expert_out) if y is None else y
    _need(y, "y", (T, d))
    _check(LIB.moe_combine(_ptr(expert_out), _ptr(row_pos), _ptr(topk_w), T, d, k, _ptr(y),
                           _y_code(y), _stream(stream)), "moe_combine")
    return y


def make_layer_args(x, w_router, w_gate, w_up, w_down, k, scoring, y, router_bias=None,
                    sel_bias=None, logits=None, topk_ids=None, topk_w=None, expert_counts=None,
                    w_scales=None, w_format="plain"):
    """Quantised expert weights: int8 codes (moe_quantize_rows_i8) with ``w_scales`` = their
    (gate, up, down) fp32 row scales, or uint8 packed 4-bit codes (moe_quantize_groups_q4) with
    ``w_scales`` = their int32 (scale, bias) pair arrays. ``w_format="frag"``: the expert stacks
    (bf16, int8 or packed 4-bit) reordered by moe_pack_weights_frag (same shapes and dtypes as the
    row-major stacks; scales unchanged)."""
    T, d = x.shape
    E, H, _ = w_gate.shape
    if w_format not in ("plain", "frag"):
        raise ValueError(f"w_format must be 'plain' or 'frag', not {w_format!r}")
    wt = w_gate.dtype if w_gate.dtype in (torch.int8, torch.uint8) else x.dtype
    if w_format == "frag" and (wt not in (torch.bfloat16, torch.int8, torch.uint8) or
                               x.dtype != torch.bfloat16):
        raise ValueError("w_format='frag' needs bfloat16 activations and bfloat16, int8 or "
                         "packed 4-bit expert stacks")
    q4 = wt == torch.uint8
    _need(x, "x", (T, d))
    _need(w_router, "w_router", (E, d), x.dtype)
    _need(w_gate, "w_gate", (E, H, d // 2 if q4 else d), wt)
    _need(w_up, "w_up", (E, H, d // 2 if q4 else d), wt)
    _need(w_down, "w_down", (E, d, H // 2 if q4 else H), wt)
    if wt in (torch.int8, torch.uint8):
        if w_scales is None:
            raise ValueError("quantised expert weights need w_scales = (gate, up, down)")
        if q4:
            _need(w_scales[0], "w_gate_scale", (E, H, d // 64), torch.int32)
            _need(w_scales[1], "w_up_scale", (E, H, d // 64), torch.int32)
            _need(w_scales[2], "w_down_scale", (E, d, H // 64), torch.int32)
        else:
            _need(w_scales[0], "w_gate_scale", (E, H), torch.float32)
            _need(w_scales[1], "w_up_scale", (E, H), torch.float32)
            _need(w_scales[2], "w_down_scale", (E, d), torch.float32)
    _need(router_bias, "router_bias", (E,), torch.float32)
    _need(sel_bias, "sel_bias", (E,), torch.float32)
    _need(y, "y", (T, d))
    _need(logits, "logits", (T, E), torch.float32)
    _need(topk_ids, "topk_ids", (T, k), torch.int32)
    _need(topk_w, "topk_w", (T, k), torch.float32)
    _need(expert_counts, "expert_counts", (E,), torch.int32)
    a = MoeLayerArgs()
    a.struct_size = ctypes.sizeof(MoeLayerArgs)
    a.T, a.d, a.E, a.H, a.k = T, d, E, H, k
    a.dtype = _dtype_code(x)
    a.w_dtype = {torch.int8: MOE_I8, torch.uint8: MOE_Q4}.get(wt, a.dtype)
    if w_format == "frag":
        a.w_dtype = {torch.int8: MOE_I8_FRAG, torch.uint8: MOE_Q4_FRAG}.get(wt, MOE_BF16_FRAG)
    if wt in (torch.int8, torch.uint8):
        a.w_gate_scale, a.w_up_scale, a.w_down_scale = (t.data_ptr() for t in w_scales)
    a.scoring = _scoring_code(scoring)
    a.y_dtype = _y_code(y)
    for name, t in (("x", x), ("w_router", w_router), ("router_bias", router_bias),
                    ("sel_bias", sel_bias), ("w_gate", w_gate), ("w_up", w_up), ("w_down", w_down),
                    ("y", y), ("logits", logits), ("topk_ids", topk_ids), ("topk_w", topk_w),
                    ("expert_counts", expert_counts)):
        setattr(a, name, None if t is None else t.data_ptr())
    return a


def moe_layer_forward(x, w_router, w_gate, w_up, w_down, k, scoring, router_bias=None,
                      sel_bias=None, y=None, logits=None, topk_ids=None, topk_w=None,
                      expert_counts=None, workspace=None, stream=None, args=None, w_scales=None,
                      y_dtype=torch.float32, w_format="plain"):
    """The fused layer. Returns y [T, d], float32 unless ``y`` (or ``y_dtype``) is bfloat16.
    Optional outputs are written when passed. With quantised expert weights
    (moe_quantize_rows_i8 or moe_quantize_groups_q4 codes) pass their scale arrays as
    w_scales; with fragment-major stacks (moe_pack_weights_frag) pass w_format="frag"."""
    T, d = x.shape
    E, H, _ = w_gate.shape
    y = _empty((T, d), y_dtype, x) if y is None else y
    if args is None:
        args = make_layer_args(x, w_router, w_gate, w_up, w_down, k, scoring, y, router_bias,
                               sel_bias, logits, topk_ids, topk_w, expert_counts, w_scales,
                               w_format)
    ws_bytes = moe_workspace_size(T, d, E, H, k, args.dtype)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=x.device)
    _check(LIB.moe_layer_forward(ctypes.byref(args), _ptr(workspace), workspace.numel(),
                                 _stream(stream)), "moe_layer_forward")
    return y


def moe_layer_forward_noalloc(x, w_router, w_gate, w_up, w_down, k, scoring, router_bias=None,
                              sel_bias=None, y=None, logits=None, topk_ids=None, topk_w=None,
                              expert_counts=None, stream=None, args=None, w_scales=None,
                              y_dtype=torch.float32, w_format="plain"):
    """The fused layer on the library's fixed scratch array (no workspace argument, nothing
    allocated by the library; see moe_layer_forward_noalloc in include/moe.h). Returns y."""
    T, d = x.shape
    y = _empty((T, d), y_dtype, x) if y is None else y
    if args is None:
        args = make_layer_args(x, w_router, w_gate, w_up, w_down, k, scoring, y, router_bias,
                               sel_bias, logits, topk_ids, topk_w, expert_counts, w_scales,
                               w_format)
    _check(LIB.moe_layer_forward_noalloc(ctypes.byref(args), _stream(stream)),
           "moe_layer_forward_noalloc")
    return y


def moe_quantize_rows_i8(w, q=None, scales=None, stream=None):
    """Per-row symmetric int8 codes of w [..., K] (bf16 or fp32): returns (q int8 [..., K],
    scales fp32 [...])."""
    K = w.shape[-1]
    rows = w.numel() // K if K else 0
    if not w.is_contiguous():
        raise ValueError("w must be contiguous")
    q = torch.empty(w.shape, dtype=torch.int8, device=w.device) if q is None else q
    scales = torch.empty(w.shape[:-1], dtype=torch.float32, device=w.device) if scales is None else scales
    _need(q, "q", tuple(w.shape), torch.int8)
    _need(scales, "scales", tuple(w.shape[:-1]), torch.float32)
    _check(LIB.moe_quantize_rows_i8(_ptr(w), rows, K, _dtype_code(w), _ptr(q), _ptr(scales),
                                    _stream(stream)), "moe_quantize_rows_i8")
    return q, scales


def moe_quantize_groups_q4(w, q=None, qpar=None, stream=None):
    """4-bit affine codes of w [..., K] (bf16 or fp32, K % 128 == 0) in groups of 64: returns
    (q uint8 [..., K / 2] packed codes, qpar int32 [..., K / 64] (scale, bias) bf16 pairs)."""
    K = w.shape[-1]
    rows = w.numel() // K if K else 0
    if not w.is_contiguous():
        raise ValueError("w must be contiguous")
    q = torch.empty(tuple(w.shape[:-1]) + (K // 2,), dtype=torch.uint8, device=w.device) if q is None else q
    qpar = (torch.empty(tuple(w.shape[:-1]) + (K // 64,), dtype=torch.int32, device=w.device)
            if qpar is None else qpar)
    _need(q, "q", tuple(w.shape[:-1]) + (K // 2,), torch.uint8)
    _need(qpar, "qpar", tuple(w.shape[:-1]) + (K // 64,), torch.int32)
    _check(LIB.moe_quantize_groups_q4(_ptr(w), rows, K, _dtype_code(w), _ptr(q), _ptr(qpar),
                                      _stream(stream)), "moe_quantize_groups_q4")
    return q, qpar


def moe_pack_weights_frag(w, out=None, stream=None):
    """Fragment-major copy of expert weights for w_format="frag" (bf16: every shape; codes: the
    decode path): w [..., R, K] bf16 values
    (K % 32 == 0), int8 codes (moe_quantize_rows_i8, K % 128 == 0) or uint8 packed 4-bit codes
    [..., R, K / 2] (moe_quantize_groups_q4, K % 128 == 0); R % 16 == 0. Returns the same shape
    and dtype, bytes reordered (moe_pack_weights_frag in include/moe.h)."""
    codes = {torch.bfloat16: MOE_BF16, torch.int8: MOE_I8, torch.uint8: MOE_Q4}
    if w.dtype not in codes or w.dim() < 2 or not w.is_contiguous():
        raise ValueError("w must be a contiguous bfloat16, int8 or uint8 tensor of at least two "
                         "dimensions")
    K = w.shape[-1] * (2 if w.dtype == torch.uint8 else 1)
    rows = w.numel() // w.shape[-1] if w.shape[-1] else 0
    out = torch.empty_like(w) if out is None else out
    _need(out, "out", tuple(w.shape), w.dtype)
    _check(LIB.moe_pack_weights_frag(_ptr(w), rows, K, codes[w.dtype], _ptr(out), _stream(stream)),
           "moe_pack_weights_frag")
    return out


class MoeGraphLadder:
    """moe_ladder_create / moe_ladder_run / moe_ladder_destroy over torch tensors: the layer is
    captured once per bucket of batch sizes on the buffers given here (every token-indexed tensor
    holds x.shape[0] rows), and run(T) replays the smallest bucket >= T. The object keeps every
    captured tensor referenced until close(). `stream` must be a torch.cuda.Stream other than the
    default stream (capture needs a stream of its own)."""

    def __init__(self, x, w_router, w_gate, w_up, w_down, k, scoring, buckets, y=None,
                 router_bias=None, sel_bias=None, logits=None, topk_ids=None, topk_w=None,
                 expert_counts=None, w_scales=None, stream=None, w_format="plain"):
        T, d = x.shape
        E, H, _ = w_gate.shape
        self.y = _empty((T, d), torch.float32, x) if y is None else y
        self.args = make_layer_args(x, w_router, w_gate, w_up, w_down, k, scoring, self.y,
                                    router_bias, sel_bias, logits, topk_ids, topk_w,
                                    expert_counts, w_scales, w_format)
        ws_bytes = moe_workspace_size(T, d, E, H, k, self.args.dtype)
        self.workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=x.device)
        self._keep = (x, w_router, w_gate, w_up, w_down, router_bias, sel_bias, logits, topk_ids,
                      topk_w, expert_counts, w_scales)
        b = (ctypes.c_int32 * len(buckets))(*buckets)
        self.buckets = list(buckets)
        self._h = c_void_p()
        _check(LIB.moe_ladder_create(ctypes.byref(self.args), b, len(buckets), _ptr(self.workspace),
                                     self.workspace.numel(), _stream(stream), ctypes.byref(self._h)),
               "moe_ladder_create")

    def run(self, T, stream=None):
        """Replays the bucket for T tokens; returns the bucket size used."""
        used = ctypes.c_int32()
        _check(LIB.moe_ladder_run(self._h, T, _stream(stream), ctypes.byref(used)), "moe_ladder_run")
        return used.value

    def close(self):
        if self._h:
            LIB.moe_ladder_destroy(self._h)
            self._h = c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:  # pragma: no cover (interpreter shutdown)
            pass
