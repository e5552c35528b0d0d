"""The C ABI without a GPU: the library loads, exports every declared entry point, and rejects
bad arguments before touching the device (CPU only; no call here launches a kernel)."""
import ctypes
import os
import re

import pytest

from expert_routing_grouped_moe_amd import moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

FAKE = ctypes.c_void_p(0x100000)      # 16-byte aligned, never dereferenced by these calls
MISALIGNED = ctypes.c_void_p(0x100004)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_bound_entry_points():
    assert declared_functions() == sorted(moe.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(moe.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version_and_status_strings():
    assert moe.moe_abi_version() == 5 == moe.MOE_ABI_VERSION
    hdr = re.search(r"#define MOE_ABI_VERSION (\d+)", open(HEADER).read())
    assert hdr and int(hdr.group(1)) == moe.MOE_ABI_VERSION
    for st in (0, -1, -2, -3, -4, -5):
        assert moe.moe_status_string(st) and moe.moe_status_string(st) != "unknown status"
    assert moe.moe_status_string(7) == "unknown status"


def test_workspace_size():
    L = moe.LIB
    assert L.moe_workspace_size(0, 128, 8, 256, 1, 0) == 0
    assert L.moe_workspace_size(64, 100, 8, 256, 1, 1) == 0          # d % 64 for bf16
    assert L.moe_workspace_size(64, 128, 8, 256, 9, 0) == 0          # k > 8
    a = L.moe_workspace_size(64, 2048, 16, 2816, 1, 1)
    b = L.moe_workspace_size(128, 2048, 16, 2816, 1, 1)
    assert 0 < a < b
    # h (2-byte fp16 on this path) alone is T*k*H*2 bytes
    assert a >= 64 * 2816 * 2
    # k >= 2 outside the weight-streaming path stages fp32 expert outputs: T*k*d*4 more bytes
    assert L.moe_workspace_size(64, 128, 8, 256, 2, 0) - L.moe_workspace_size(64, 128, 8, 256, 1, 0) \
        >= 64 * 2 * 128 * 4
    # every k >= 2 shape reserves the staged outputs (a bf16 y is combined from them, also on the
    # weight-streaming path, which adds k == 2 outputs into an fp32 y directly)
    assert L.moe_workspace_size(64, 1024, 64, 512, 2, 1) >= 64 * 2 * 1024 * 4


@pytest.mark.parametrize("d,E,H,k,dt", [(1024, 64, 512, 2, 1), (2048, 16, 2816, 1, 1),
                                        (128, 8, 256, 1, 0), (256, 8, 256, 8, 1),
                                        (1024, 64, 512, 1, 1), (256, 256, 256, 2, 1)])
def test_workspace_never_shrinks_as_T_grows(d, E, H, k, dt):
    # a workspace sized for the largest batch must serve every smaller one (the graph ladder and
    # callers that reuse one buffer rely on it), across the routing and expert kernel switches
    L = moe.LIB
    Ts = list(range(1, 700)) + [1000, 2047, 2048, 2049, 4096, 8192, 20000]
    sizes = [L.moe_workspace_size(T, d, E, H, k, dt) for T in Ts]
    assert all(s > 0 for s in sizes)
    bad = [(Ts[i], Ts[i + 1]) for i in range(len(Ts) - 1) if sizes[i + 1] < sizes[i]]
    assert not bad, bad[:4]


def test_size_limits():
    L = moe.LIB
    assert L.moe_workspace_size(1 << 24, 64, 8, 64, 1, 1) > 0
    assert L.moe_workspace_size((1 << 24) + 1, 64, 8, 64, 1, 1) == 0       # T > 2^24
    assert L.moe_workspace_size(1 << 20, 2048, 16, 2048, 1, 1) == 0       # T*k*max(d, H) = 2^31
    assert L.moe_workspace_size((1 << 20) - 1, 2048, 16, 2048, 1, 1) > 0
    assert L.moe_workspace_size(1 << 19, 1024, 64, 2048, 2, 1) == 0       # 2^19 * 2 * 2048
    assert L.moe_workspace_size(4, 65536 + 64, 8, 256, 1, 1) == 0         # d > 65536
    assert L.moe_workspace_size(4, 256, 8, 65536 + 64, 1, 1) == 0         # H > 65536
    call = lambda T, E=8, k=1: L.moe_route(FAKE, None, T, E, k, 0, FAKE, FAKE, FAKE, None)
    assert call((1 << 24) + 1) == moe.MOE_ERR_SHAPE
    assert L.moe_router_logits(FAKE, FAKE, None, (1 << 24) + 1, 128, 8, 1, FAKE, None) == moe.MOE_ERR_SHAPE
    assert L.moe_router_logits(FAKE, FAKE, None, 1 << 20, 2048, 8, 1, FAKE, None) == moe.MOE_ERR_SHAPE
    assert L.moe_combine(FAKE, FAKE, FAKE, 1 << 19, 2048, 2, FAKE, 0, None) == moe.MOE_ERR_SHAPE
    assert L.moe_quantize_rows_i8(FAKE, 1 << 25, 64, 1, FAKE, FAKE, None) == moe.MOE_ERR_SHAPE
    assert L.moe_quantize_groups_q4(FAKE, 1 << 24, 1 << 12, 1, FAKE, FAKE, None) == moe.MOE_ERR_SHAPE


def test_route_validation():
    L = moe.LIB
    call = lambda logits, sb, T, E, k, sc, ids=FAKE, w=FAKE, c=FAKE: L.moe_route(
        logits, sb, T, E, k, sc, ids, w, c, None)
    assert call(FAKE, None, 0, 8, 1, 0) == moe.MOE_OK                  # T == 0: nothing to do
    assert call(FAKE, None, 4, 0, 1, 0) == moe.MOE_ERR_SHAPE
    assert call(FAKE, None, 4, 257, 1, 0) == moe.MOE_ERR_SHAPE
    assert call(FAKE, None, 4, 8, 0, 0) == moe.MOE_ERR_SHAPE
    assert call(FAKE, None, 4, 4, 5, 0) == moe.MOE_ERR_SHAPE           # k > E
    assert call(FAKE, None, 4, 64, 9, 0) == moe.MOE_ERR_SHAPE          # k > 8
    assert call(FAKE, None, -1, 8, 1, 0) == moe.MOE_ERR_SHAPE
    assert call(FAKE, None, 4, 8, 1, 7) == moe.MOE_ERR_UNSUPPORTED
    assert call(FAKE, FAKE, 4, 8, 1, 0) == moe.MOE_ERR_UNSUPPORTED     # bias needs SelectedSoftmax
    assert call(None, None, 4, 8, 1, 0) == moe.MOE_ERR_NULL
    assert call(FAKE, None, 4, 8, 1, 1, ids=None) == moe.MOE_ERR_NULL
    assert call(MISALIGNED, None, 4, 8, 1, 0) == moe.MOE_ERR_SHAPE
    assert call(FAKE, MISALIGNED, 4, 8, 1, 1) == moe.MOE_ERR_SHAPE


def test_permute_combine_logits_validation():
    L = moe.LIB
    perm = lambda T=4, k=1, c=FAKE, sr=FAKE: L.moe_permute(FAKE, c, T, 8, k, FAKE, sr, FAKE, None)
    assert perm(T=0) == moe.MOE_OK
    assert perm(k=9) == moe.MOE_ERR_SHAPE
    assert perm(c=None) == moe.MOE_ERR_NULL
    assert perm(sr=MISALIGNED) == moe.MOE_ERR_SHAPE
    assert L.moe_combine(FAKE, FAKE, FAKE, 4, 6, 1, FAKE, 0, None) == moe.MOE_ERR_SHAPE     # d % 4
    assert L.moe_combine(FAKE, None, FAKE, 4, 8, 1, FAKE, 0, None) == moe.MOE_ERR_NULL
    assert L.moe_combine(FAKE, FAKE, FAKE, 0, 8, 1, FAKE, 0, None) == moe.MOE_OK
    assert L.moe_combine(FAKE, FAKE, FAKE, 4, 8, 1, FAKE, 2, None) == moe.MOE_ERR_UNSUPPORTED  # y_dtype
    assert L.moe_combine(FAKE, None, FAKE, 4, 8, 1, FAKE, 1, None) == moe.MOE_ERR_NULL
    assert L.moe_router_logits(FAKE, FAKE, None, 4, 128, 8, 2, FAKE, None) == moe.MOE_ERR_UNSUPPORTED
    assert L.moe_router_logits(FAKE, FAKE, None, 4, 96, 8, 1, FAKE, None) == moe.MOE_ERR_SHAPE
    assert L.moe_router_logits(FAKE, None, None, 4, 128, 8, 1, FAKE, None) == moe.MOE_ERR_NULL


def test_expert_ffn_validation():
    L = moe.LIB
    ws = L.moe_workspace_size(16, 128, 8, 256, 1, 1)
    f = lambda T=16, d=128, E=8, H=256, k=1, dt=1, ws_ptr=FAKE, ws_bytes=ws, x=FAKE: L.moe_expert_ffn(
        x, T, d, FAKE, FAKE, FAKE, E, H, k, dt, FAKE, FAKE, FAKE, ws_ptr, ws_bytes, None)
    assert f(T=0) == moe.MOE_OK
    assert f(d=96) == moe.MOE_ERR_SHAPE
    assert f(H=100) == moe.MOE_ERR_SHAPE
    assert f(dt=5) == moe.MOE_ERR_UNSUPPORTED
    assert f(ws_ptr=None) == moe.MOE_ERR_WORKSPACE
    assert f(ws_bytes=ws - 1) == moe.MOE_ERR_WORKSPACE
    assert f(x=None) == moe.MOE_ERR_NULL
    assert f(x=MISALIGNED) == moe.MOE_ERR_SHAPE


def _args(**kw):
    a = moe.MoeLayerArgs()
    a.struct_size = ctypes.sizeof(moe.MoeLayerArgs)
    a.T, a.d, a.E, a.H, a.k, a.dtype, a.scoring = 16, 128, 8, 256, 1, 1, 0
    for name in ("x", "w_router", "w_gate", "w_up", "w_down", "y"):
        setattr(a, name, FAKE.value)
    for key, v in kw.items():
        setattr(a, key, v)
    return a


def test_layer_forward_validation():
    L = moe.LIB
    ws = L.moe_workspace_size(16, 128, 8, 256, 1, 1)
    run = lambda a, w=FAKE, n=ws: L.moe_layer_forward(ctypes.byref(a), w, n, None)
    assert L.moe_layer_forward(None, FAKE, ws, None) == moe.MOE_ERR_NULL
    assert run(_args(struct_size=8)) == moe.MOE_ERR_UNSUPPORTED
    assert run(_args(T=0)) == moe.MOE_OK
    assert run(_args(k=3, E=2)) == moe.MOE_ERR_SHAPE
    assert run(_args(scoring=4)) == moe.MOE_ERR_UNSUPPORTED
    assert run(_args(scoring=3)) == moe.MOE_ERR_UNSUPPORTED
    assert run(_args(scoring=2, sel_bias=FAKE.value)) == moe.MOE_ERR_UNSUPPORTED  # sigmoid: no bias
    assert run(_args(sel_bias=FAKE.value)) == moe.MOE_ERR_UNSUPPORTED
    assert run(_args(x=None)) == moe.MOE_ERR_NULL
    assert run(_args(y=MISALIGNED.value)) == moe.MOE_ERR_SHAPE
    assert run(_args(logits=MISALIGNED.value)) == moe.MOE_ERR_SHAPE
    assert run(_args(), n=ws - 256) == moe.MOE_ERR_WORKSPACE
    assert run(_args(), w=None) == moe.MOE_ERR_WORKSPACE
    # y_dtype (ABI 4): fp32 or bf16; layouts ending before the field mean fp32
    assert run(_args(y_dtype=2)) == moe.MOE_ERR_UNSUPPORTED
    assert run(_args(y_dtype=1), n=0) == moe.MOE_ERR_WORKSPACE
    assert run(_args(y_dtype=2, struct_size=moe.MoeLayerArgs.y_dtype.offset), n=0) == \
        moe.MOE_ERR_WORKSPACE
    # timing events pass validation like any other argument (the capture check comes last)
    assert run(_args(prof_events=FAKE.value), n=0) == moe.MOE_ERR_WORKSPACE


def test_layer_forward_noalloc_validation():
    # checked on the host before any device call: sizes past the fixed scratch array are refused
    L = moe.LIB
    run = lambda a: L.moe_layer_forward_noalloc(ctypes.byref(a), None)
    assert L.moe_layer_forward_noalloc(None, None) == moe.MOE_ERR_NULL
    assert run(_args(struct_size=8)) == moe.MOE_ERR_UNSUPPORTED
    assert run(_args(T=0)) == moe.MOE_OK
    assert run(_args(k=3, E=2)) == moe.MOE_ERR_SHAPE
    big = dict(T=16384, d=2048, E=16, H=2816, k=1)          # h alone is 92 MB
    assert L.moe_workspace_size(16384, 2048, 16, 2816, 1, 1) > moe.MOE_NOALLOC_SCRATCH_BYTES
    assert run(_args(**big)) == moe.MOE_ERR_WORKSPACE
    hdr = re.search(r"#define MOE_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", open(HEADER).read())
    assert hdr and int(hdr.group(1)) << int(hdr.group(2)) == moe.MOE_NOALLOC_SCRATCH_BYTES
    # the five workloads fit
    for (T, d, E, H, k, dt) in ((64, 128, 8, 256, 1, 0), (64, 2048, 16, 2816, 1, 1),
                                (64, 1024, 64, 512, 2, 1), (4096, 1024, 64, 512, 2, 1),
                                (8192, 2048, 16, 2816, 1, 1)):
        assert 0 < L.moe_workspace_size(T, d, E, H, k, dt) <= moe.MOE_NOALLOC_SCRATCH_BYTES


def test_layer_int8_weight_validation():
    L = moe.LIB
    # a decode shape of the weight-streaming path (d, H multiples of 256, few rows per expert)
    T, d, E, H = 16, 256, 8, 256
    ws = L.moe_workspace_size(T, d, E, H, 1, 1)
    run = lambda a, n=ws: L.moe_layer_forward(ctypes.byref(a), FAKE, n, None)
    q8 = dict(T=T, d=d, E=E, H=H, w_dtype=moe.MOE_I8, w_gate_scale=FAKE.value,
              w_up_scale=FAKE.value, w_down_scale=FAKE.value)
    assert run(_args(**{**q8, "T": 0})) == moe.MOE_OK
    assert run(_args(**{**q8, "w_up_scale": None})) == moe.MOE_ERR_NULL
    assert run(_args(**{**q8, "w_down_scale": MISALIGNED.value})) == moe.MOE_ERR_SHAPE
    assert run(_args(**{**q8, "dtype": 0})) == moe.MOE_ERR_UNSUPPORTED          # fp32 activations
    assert run(_args(**{**q8, "d": 128, "H": 128})) == moe.MOE_ERR_UNSUPPORTED  # not streaming
    assert run(_args(**{**q8, "T": 2048, "k": 2}), n=1 << 40) == moe.MOE_ERR_UNSUPPORTED  # prefill
    assert run(_args(**{**q8, "w_dtype": 7})) == moe.MOE_ERR_UNSUPPORTED
    assert run(_args(**{**q8, "w_dtype": 0}), n=0) == moe.MOE_ERR_WORKSPACE      # 0: weights in dtype
    # the ABI-1 layout (no w_dtype field) is still accepted, and means weights in dtype
    assert run(_args(**{**q8, "struct_size": moe.MoeLayerArgs.w_dtype.offset}), n=0) == \
        moe.MOE_ERR_WORKSPACE
    assert run(_args(struct_size=moe.MoeLayerArgs.w_dtype.offset - 4)) == moe.MOE_ERR_UNSUPPORTED


def test_layer_q4_weight_validation():
    L = moe.LIB
    T, d, E, H = 16, 256, 8, 256
    ws = L.moe_workspace_size(T, d, E, H, 1, 1)
    run = lambda a, n=ws: L.moe_layer_forward(ctypes.byref(a), FAKE, n, None)
    q4 = dict(T=T, d=d, E=E, H=H, w_dtype=moe.MOE_Q4, w_gate_scale=FAKE.value,
              w_up_scale=FAKE.value, w_down_scale=FAKE.value)
    assert run(_args(**{**q4, "T": 0})) == moe.MOE_OK
    assert run(_args(**{**q4, "w_gate_scale": None})) == moe.MOE_ERR_NULL
    assert run(_args(**{**q4, "w_up_scale": MISALIGNED.value})) == moe.MOE_ERR_SHAPE
    assert run(_args(**{**q4, "dtype": 0})) == moe.MOE_ERR_UNSUPPORTED
    assert run(_args(**{**q4, "d": 128, "H": 128})) == moe.MOE_ERR_UNSUPPORTED
    assert run(_args(**{**q4, "T": 2048, "k": 2}), n=1 << 40) == moe.MOE_ERR_UNSUPPORTED
    assert run(_args(**q4), n=ws - 256) == moe.MOE_ERR_WORKSPACE


def test_quantize_q4_validation():
    L = moe.LIB
    q = lambda w=FAKE, rows=4, K=256, dt=1, qq=FAKE, p=FAKE: L.moe_quantize_groups_q4(
        w, rows, K, dt, qq, p, None)
    assert q(rows=0) == moe.MOE_OK
    assert q(rows=-1) == moe.MOE_ERR_SHAPE
    assert q(K=64) == moe.MOE_ERR_SHAPE           # groups of 64, blocks of 128
    assert q(K=192) == moe.MOE_ERR_SHAPE
    assert q(dt=2) == moe.MOE_ERR_UNSUPPORTED
    assert q(w=None) == moe.MOE_ERR_NULL
    assert q(p=None) == moe.MOE_ERR_NULL
    assert q(qq=MISALIGNED) == moe.MOE_ERR_SHAPE


def test_ladder_validation():
    L = moe.LIB
    out = ctypes.c_void_p()
    b = (ctypes.c_int32 * 3)(1, 8, 16)
    mk = lambda a, bb=b, n=3, s=FAKE, o=ctypes.byref(out): L.moe_ladder_create(
        ctypes.byref(a), bb, n, FAKE, 1 << 30, s, o)
    assert L.moe_ladder_create(None, b, 3, FAKE, 1 << 30, FAKE, ctypes.byref(out)) == moe.MOE_ERR_NULL
    assert mk(_args(), bb=None) == moe.MOE_ERR_NULL
    assert mk(_args(), o=None) == moe.MOE_ERR_NULL
    assert mk(_args(), n=0) == moe.MOE_ERR_SHAPE
    assert mk(_args(), n=moe.MOE_LADDER_MAX_BUCKETS + 1) == moe.MOE_ERR_SHAPE
    assert mk(_args(), bb=(ctypes.c_int32 * 3)(1, 8, 8)) == moe.MOE_ERR_SHAPE        # not ascending
    assert mk(_args(), bb=(ctypes.c_int32 * 3)(0, 8, 16)) == moe.MOE_ERR_SHAPE       # empty bucket
    assert mk(_args(), bb=(ctypes.c_int32 * 3)(1, 8, 17)) == moe.MOE_ERR_SHAPE       # > T = 16
    assert mk(_args(struct_size=8)) == moe.MOE_ERR_UNSUPPORTED
    assert mk(_args(), s=None) == moe.MOE_ERR_UNSUPPORTED                            # no null stream
    assert L.moe_ladder_run(None, 4, None, None) == moe.MOE_ERR_NULL
    L.moe_ladder_destroy(None)


def test_quantize_validation():
    L = moe.LIB
    q = lambda w=FAKE, rows=4, K=64, dt=1, qq=FAKE, s=FAKE: L.moe_quantize_rows_i8(w, rows, K, dt, qq, s, None)
    assert q(rows=0) == moe.MOE_OK
    assert q(rows=-1) == moe.MOE_ERR_SHAPE
    assert q(K=0) == moe.MOE_ERR_SHAPE
    assert q(K=40) == moe.MOE_ERR_SHAPE
    assert q(dt=2) == moe.MOE_ERR_UNSUPPORTED
    assert q(w=None) == moe.MOE_ERR_NULL
    assert q(s=None) == moe.MOE_ERR_NULL
    assert q(qq=MISALIGNED) == moe.MOE_ERR_SHAPE


def test_binding_checks_shapes_before_calling():
    torch = pytest.importorskip("torch")
    x = torch.zeros(4, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        moe.moe_router_logits(x, torch.zeros(8, 64, dtype=torch.bfloat16))
    with pytest.raises(TypeError):
        moe.moe_router_logits(x.half(), torch.zeros(8, 128, dtype=torch.half))


def test_frag_weights_validation():
    L = moe.LIB
    # moe_pack_weights_frag: rows % 16, K % 32 (bf16) or 128 (codes), rows * K < 2^36; NULL;
    # alignment; stored type
    pack = lambda w=FAKE, rows=32, K=64, out=FAKE, dt=moe.MOE_BF16: L.moe_pack_weights_frag(
        w, rows, K, dt, out, None)
    assert pack(rows=0) == moe.MOE_OK
    assert pack(dt=moe.MOE_F32) == moe.MOE_ERR_UNSUPPORTED
    assert pack(dt=moe.MOE_BF16_FRAG) == moe.MOE_ERR_UNSUPPORTED
    for dt in (moe.MOE_I8, moe.MOE_Q4):
        assert pack(dt=dt) == moe.MOE_ERR_SHAPE                      # K = 64: not a multiple of 128
        assert pack(dt=dt, K=192) == moe.MOE_ERR_SHAPE
        assert pack(dt=dt, K=256, rows=0) == moe.MOE_OK
        assert pack(dt=dt, K=256, out=None) == moe.MOE_ERR_NULL
    assert pack(rows=0, w=None) == moe.MOE_OK
    assert pack(rows=-16) == moe.MOE_ERR_SHAPE
    assert pack(rows=24) == moe.MOE_ERR_SHAPE
    assert pack(K=48) == moe.MOE_ERR_SHAPE
    assert pack(K=0) == moe.MOE_ERR_SHAPE
    assert pack(rows=1 << 26, K=1 << 10) == moe.MOE_ERR_SHAPE
    assert pack(rows=16, K=(1 << 20) + 32) == moe.MOE_ERR_SHAPE       # past the row-length limit
    assert pack(rows=16, K=1 << 30) == moe.MOE_ERR_SHAPE
    assert pack(w=None) == moe.MOE_ERR_NULL
    assert pack(out=None) == moe.MOE_ERR_NULL
    assert pack(w=MISALIGNED) == moe.MOE_ERR_SHAPE
    assert pack(out=MISALIGNED) == moe.MOE_ERR_SHAPE
    # MOE_BF16_FRAG in the layer: bf16 activations on the weight-streaming path; no scale arrays
    T, d, E, H = 16, 256, 8, 256
    ws = L.moe_workspace_size(T, d, E, H, 1, 1)
    run = lambda a, n=ws: L.moe_layer_forward(ctypes.byref(a), FAKE, n, None)
    fr = dict(T=T, d=d, E=E, H=H, w_dtype=moe.MOE_BF16_FRAG)
    assert run(_args(**{**fr, "T": 0})) == moe.MOE_OK
    assert run(_args(**fr), n=0) == moe.MOE_ERR_WORKSPACE            # accepted up to the workspace
    assert run(_args(**{**fr, "dtype": 0})) == moe.MOE_ERR_UNSUPPORTED          # fp32 activations
    # bf16 fragment-major weights also serve the grouped-GEMM (prefill) path
    assert run(_args(**{**fr, "T": 2048, "k": 2}), n=0) == moe.MOE_ERR_WORKSPACE
    assert run(_args(**{**fr, "d": 128, "H": 128}), n=0) == moe.MOE_ERR_WORKSPACE
    # the quantised fragment-major types need their scale arrays, like MOE_I8 and MOE_Q4
    for wd in (moe.MOE_I8_FRAG, moe.MOE_Q4_FRAG):
        q = dict(fr, w_dtype=wd, w_gate_scale=FAKE.value, w_up_scale=FAKE.value,
                 w_down_scale=FAKE.value)
        assert run(_args(**q), n=0) == moe.MOE_ERR_WORKSPACE
        assert run(_args(**{**q, "w_up_scale": None})) == moe.MOE_ERR_NULL
        assert run(_args(**{**q, "w_gate_scale": MISALIGNED.value})) == moe.MOE_ERR_SHAPE
        assert run(_args(**{**q, "dtype": 0})) == moe.MOE_ERR_UNSUPPORTED
        assert run(_args(**{**q, "T": 2048, "k": 2}), n=1 << 40) == moe.MOE_ERR_UNSUPPORTED
    assert run(_args(**{**fr, "w_dtype": 7})) == moe.MOE_ERR_UNSUPPORTED


def test_python_pack_wrapper_checks_its_input():
    import torch
    with pytest.raises(ValueError):
        moe.moe_pack_weights_frag(torch.zeros((16, 32), dtype=torch.float32))
    with pytest.raises(ValueError):
        moe.moe_pack_weights_frag(torch.zeros((32,), dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        moe.make_layer_args(torch.zeros((4, 256)), torch.zeros((8, 256)), torch.zeros((8, 256, 256)),
                            torch.zeros((8, 256, 256)), torch.zeros((8, 256, 256)), 1, "softmax",
                            torch.zeros((4, 256)), w_format="frag")
    with pytest.raises(ValueError):
        moe.make_layer_args(torch.zeros((4, 256)), torch.zeros((8, 256)), torch.zeros((8, 256, 256)),
                            torch.zeros((8, 256, 256)), torch.zeros((8, 256, 256)), 1, "softmax",
                            torch.zeros((4, 256)), w_format="tiled")
