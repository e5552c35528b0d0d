// C ABI of libmoe.so: argument validation, workspace layout and the launch sequences.
// Validation never touches the GPU, so a machine without one can exercise every error path.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "moe.h"
#include "common.hpp"
#include "kernels.hpp"

namespace {

using moe::DownArgs;
using moe::RouteOut;
using moe::RowSource;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr size_t kAlign = 256;
size_t up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Size limits of the contract (include/moe.h, "Shapes"): with at most 2^24 tokens, widths of at
// most 65536 and fewer than 2^31 elements in every activation-sized buffer, every launch of the
// library stays below 2^31 work-items and every grid dimension within its hardware limit.
constexpr int kMaxTokens = 1 << 24;
constexpr int kMaxWidth = 65536;
constexpr long long kMaxElems = 1ll << 31;

int check_dims(int T, int d, int E, int H, int k, int dtype) {
  if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (T < 0 || T > kMaxTokens || E < 1 || E > moe::kMaxE || k < 1 || k > moe::kMaxK || k > E)
    return MOE_ERR_SHAPE;
  if (d <= 0 || H <= 0 || d > kMaxWidth || H > kMaxWidth) return MOE_ERR_SHAPE;
  const int mult = dtype == MOE_BF16 ? 64 : 4;
  if (d % mult != 0 || H % mult != 0) return MOE_ERR_SHAPE;
  if (static_cast<long long>(T) * k * (d > H ? d : H) >= kMaxElems) return MOE_ERR_SHAPE;
  return MOE_OK;
}

int check_route_dims(int T, int E, int k) {
  if (T < 0 || T > kMaxTokens || E < 1 || E > moe::kMaxE || k < 1 || k > moe::kMaxK || k > E)
    return MOE_ERR_SHAPE;
  return MOE_OK;
}

int check_scoring(int scoring, const float* sel_bias) {
  if (scoring != MOE_SCORING_SOFTMAX && scoring != MOE_SCORING_SELECTED_SOFTMAX &&
      scoring != MOE_SCORING_SIGMOID)
    return MOE_ERR_UNSUPPORTED;
  // a selection bias is defined for SELECTED_SOFTMAX only
  if (scoring != MOE_SCORING_SELECTED_SOFTMAX && sel_bias != nullptr) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// Device workspace regions of the fused layer (the step calls use a subset).
struct Layout {
  size_t h, logits, ids, w, counts, offsets, sorted_rows, row_pos, eo, rpart, total;
  Layout(int T, int d, int E, int H, int k, int dtype) {
    const size_t rows = static_cast<size_t>(T) * k;
    size_t o = 0;
    h = o;           o += up(rows * H * (dtype == MOE_BF16 ? 2 : 4));
    logits = o;      o += up(static_cast<size_t>(T) * E * 4);
    ids = o;         o += up(rows * 4);
    w = o;           o += up(rows * 4);
    counts = o;      o += up(static_cast<size_t>(E) * 4);
    offsets = o;     o += up(static_cast<size_t>(E + 1) * 4);
    sorted_rows = o; o += up(rows * 4);
    row_pos = o;     o += up(rows * 4);
    // fp32 expert outputs staged for the combine kernel whenever k > 1 (the streaming path adds
    // k == 2 outputs straight into an fp32 y and leaves this region unused; a bf16 y needs it)
    eo = o;          o += k > 1 ? up(rows * d * 4) : 0;
    // partial logit tiles of the split router (bf16, batches of at most kRouteSplitMaxT tokens),
    // sized for min(T, kRouteSplitMaxT) tokens so that the total never shrinks as T grows (a
    // workspace sized for a large batch serves every smaller one)
    const int tr = T < moe::kRouteSplitMaxT ? T : moe::kRouteSplitMaxT;
    const int rks = dtype == MOE_BF16 ? moe::route_split_ks(tr, d, E) : 0;
    rpart = o;       o += up(static_cast<size_t>(rks) * tr * E * 4);
    total = o;
  }
};

template <class T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// Launch errors are read back with hipGetLastError(); an error left by an earlier, unrelated
// HIP call would otherwise be reported against this call's first launch.
void clear_stale_error() { (void)hipGetLastError(); }

// Stage marker (host launches only: moe_layer_forward refuses prof_events during capture).
hipError_t record_event(void* ev, hipStream_t s) {
  return hipEventRecord(static_cast<hipEvent_t>(ev), s);
}

bool capturing(hipStream_t s) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  return hipStreamIsCapturing(s, &cs) == hipSuccess && cs != hipStreamCaptureStatusNone;
}

#define MOE_TRY(expr)                          \
  do {                                         \
    const hipError_t _e = (expr);              \
    if (_e != hipSuccess) return MOE_ERR_HIP;  \
  } while (0)

}  // namespace

namespace moe {
hipError_t record_stage_event(void* ev, hipStream_t s) { return record_event(ev, s); }
size_t layer_ids_offset(int T, int d, int E, int H, int k, int dtype) {
  return Layout(T, d, E, H, k, dtype).ids;
}
}  // namespace moe

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "size out of range or pointer not 16-byte aligned";
    case MOE_ERR_UNSUPPORTED: return "unsupported dtype, scoring mode or argument combination";
    case MOE_ERR_WORKSPACE: return "workspace missing or smaller than required";
    case MOE_ERR_HIP: return "a HIP kernel launch failed";
    default: return "unknown status";
  }
}

size_t moe_workspace_size(int T, int d, int E, int H, int k, int dtype) {
  if (check_dims(T, d, E, H, k, dtype) != MOE_OK || T == 0) return 0;
  return Layout(T, d, E, H, k, dtype).total;
}

int moe_router_logits(const void* x, const void* w_router, const float* router_bias, int T, int d,
                      int E, int dtype, float* logits, void* stream) {
  if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (T < 0 || T > kMaxTokens || E < 1 || E > moe::kMaxE || d <= 0) return MOE_ERR_SHAPE;
  if (static_cast<long long>(T) * d >= kMaxElems) return MOE_ERR_SHAPE;
  if (d % (dtype == MOE_BF16 ? 64 : 4) != 0) return MOE_ERR_SHAPE;
  if (T == 0) return MOE_OK;
  if (!x || !w_router || !logits) return MOE_ERR_NULL;
  if (!aligned16(x) || !aligned16(w_router) || !aligned16(logits) ||
      (router_bias && !aligned16(router_bias)))
    return MOE_ERR_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  clear_stale_error();
  if (dtype == MOE_F32)
    return hip_status(moe::launch_logits_f32(static_cast<const float*>(x),
                                             static_cast<const float*>(w_router), router_bias, T,
                                             d, E, logits, s));
  return hip_status(moe::launch_logits_bf16(static_cast<const uint16_t*>(x),
                                            static_cast<const uint16_t*>(w_router), router_bias,
                                            T, d, E, logits, s));
}

int moe_route(const float* logits, const float* sel_bias, int T, int E, int k, int scoring,
              int32_t* topk_ids, float* topk_w, int32_t* expert_counts, void* stream) {
  int st = check_route_dims(T, E, k);
  if (st != MOE_OK) return st;
  st = check_scoring(scoring, sel_bias);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!logits || !topk_ids || !topk_w || !expert_counts) return MOE_ERR_NULL;
  if (!aligned16(logits) || !aligned16(topk_ids) || !aligned16(topk_w) ||
      !aligned16(expert_counts) || (sel_bias && !aligned16(sel_bias)))
    return MOE_ERR_SHAPE;
  clear_stale_error();
  const RouteOut o{topk_ids, topk_w, expert_counts, nullptr, 0};
  return hip_status(moe::launch_route_from_logits(logits, sel_bias, T, E, k, scoring, o,
                                                  static_cast<hipStream_t>(stream)));
}

int moe_permute(const int32_t* topk_ids, const int32_t* expert_counts, int T, int E, int k,
                int32_t* expert_offsets, int32_t* sorted_rows, int32_t* row_pos, void* stream) {
  const int st = check_route_dims(T, E, k);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!topk_ids || !expert_counts || !expert_offsets || !sorted_rows || !row_pos) return MOE_ERR_NULL;
  if (!aligned16(topk_ids) || !aligned16(expert_counts) || !aligned16(expert_offsets) ||
      !aligned16(sorted_rows) || !aligned16(row_pos))
    return MOE_ERR_SHAPE;
  clear_stale_error();
  return hip_status(moe::launch_dispatch(topk_ids, T * k, E, expert_offsets, sorted_rows, row_pos,
                                         nullptr, static_cast<hipStream_t>(stream)));
}

int moe_expert_ffn(const void* x, int T, int d, const void* w_gate, const void* w_up,
                   const void* w_down, int E, int H, int k, int dtype,
                   const int32_t* expert_offsets, const int32_t* sorted_rows, float* expert_out,
                   void* ws, size_t ws_bytes, void* stream) {
  const int st = check_dims(T, d, E, H, k, dtype);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!x || !w_gate || !w_up || !w_down || !expert_offsets || !sorted_rows || !expert_out)
    return MOE_ERR_NULL;
  if (!aligned16(x) || !aligned16(w_gate) || !aligned16(w_up) || !aligned16(w_down) ||
      !aligned16(expert_offsets) || !aligned16(sorted_rows) || !aligned16(expert_out))
    return MOE_ERR_SHAPE;
  const Layout lay(T, d, E, H, k, dtype);
  if (!ws || ws_bytes < lay.total) return MOE_ERR_WORKSPACE;
  if (!aligned16(ws)) return MOE_ERR_SHAPE;
  const DownArgs down{moe::kDownExpertOut, expert_out, nullptr, k, 0};
  hipStream_t s = static_cast<hipStream_t>(stream);
  clear_stale_error();
  if (dtype == MOE_BF16) {
    const RowSource rs{nullptr, T * k, expert_offsets, sorted_rows, nullptr};
    return hip_status(moe::launch_ffn_bf16(static_cast<const uint16_t*>(x), w_gate, w_up, w_down, T,
                                           d, E, H, k, rs, at<uint16_t>(ws, lay.h), down, s,
                                           moe::StageMarks{}, moe::QuantWeights{}));
  }
  return hip_status(moe::launch_ffn_f32(
      static_cast<const float*>(x), static_cast<const float*>(w_gate),
      static_cast<const float*>(w_up), static_cast<const float*>(w_down), T, d, E, H, k,
      expert_offsets, sorted_rows, at<float>(ws, lay.h), down, s, moe::StageMarks{}));
}

// Quantiser limits: fewer than 2^25 rows (one wave per row) and 2^36 elements (one lane per
// group of 64), so that every launch stays below 2^31 work-items.
constexpr long long kMaxQuantRows = 1ll << 25;
constexpr long long kMaxQuantElems = 1ll << 36;

int moe_quantize_rows_i8(const void* w, int64_t rows, int K, int dtype, int8_t* q, float* scales,
                         void* stream) {
  if (rows < 0 || K < 1 || K % 16 != 0) return MOE_ERR_SHAPE;
  if (rows >= kMaxQuantRows || rows * K >= kMaxQuantElems) return MOE_ERR_SHAPE;
  if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (rows == 0) return MOE_OK;
  if (!w || !q || !scales) return MOE_ERR_NULL;
  if (!aligned16(w) || !aligned16(q) || !aligned16(scales)) return MOE_ERR_SHAPE;
  clear_stale_error();
  return hip_status(moe::launch_quantize_rows_i8(w, rows, K, dtype == MOE_BF16, q, scales,
                                                 static_cast<hipStream_t>(stream)));
}

int moe_quantize_groups_q4(const void* w, int64_t rows, int K, int dtype, uint8_t* q,
                           uint32_t* qpar, void* stream) {
  if (rows < 0 || K < 128 || K % 128 != 0) return MOE_ERR_SHAPE;
  if (rows >= kMaxQuantRows || rows * K >= kMaxQuantElems) return MOE_ERR_SHAPE;
  if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (rows == 0) return MOE_OK;
  if (!w || !q || !qpar) return MOE_ERR_NULL;
  if (!aligned16(w) || !aligned16(q) || !aligned16(qpar)) return MOE_ERR_SHAPE;
  clear_stale_error();
  return hip_status(moe::launch_quantize_groups_q4(w, rows, K, dtype == MOE_BF16, q, qpar,
                                                   static_cast<hipStream_t>(stream)));
}

int moe_pack_weights_frag(const void* w, int64_t rows, int K, int w_dtype, void* out,
                          void* stream) {
  if (w_dtype != MOE_BF16 && w_dtype != MOE_I8 && w_dtype != MOE_Q4) return MOE_ERR_UNSUPPORTED;
  const int kmul = w_dtype == MOE_BF16 ? 32 : 128;
  // K <= 2^20 keeps a row's bytes (2 K for bf16) inside an int
  if (rows < 0 || rows % 16 != 0 || K < kmul || K % kmul != 0 || K > (1 << 20))
    return MOE_ERR_SHAPE;
  if (rows * K >= kMaxQuantElems) return MOE_ERR_SHAPE;
  if (rows == 0) return MOE_OK;
  if (!w || !out) return MOE_ERR_NULL;
  if (!aligned16(w) || !aligned16(out)) return MOE_ERR_SHAPE;
  const int row_bytes = w_dtype == MOE_BF16 ? 2 * K : (w_dtype == MOE_I8 ? K : K / 2);
  const int fmt = w_dtype == MOE_BF16 ? moe::kWBf16 : (w_dtype == MOE_I8 ? moe::kWI8 : moe::kWQ4);
  clear_stale_error();
  return hip_status(moe::launch_pack_frag(w, rows, row_bytes, fmt, out,
                                          static_cast<hipStream_t>(stream)));
}

int moe_combine(const float* expert_out, const int32_t* row_pos, const float* topk_w, int T,
                int d, int k, void* y, int y_dtype, void* stream) {
  if (T < 0 || T > kMaxTokens || d <= 0 || d % 4 != 0 || k < 1 || k > moe::kMaxK)
    return MOE_ERR_SHAPE;
  if (static_cast<long long>(T) * k * d >= kMaxElems) return MOE_ERR_SHAPE;
  if (y_dtype != MOE_F32 && y_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!expert_out || !row_pos || !topk_w || !y) return MOE_ERR_NULL;
  if (!aligned16(expert_out) || !aligned16(row_pos) || !aligned16(topk_w) || !aligned16(y))
    return MOE_ERR_SHAPE;
  clear_stale_error();
  return hip_status(moe::launch_combine(expert_out, row_pos, topk_w, T, d, k, y,
                                        y_dtype == MOE_BF16, static_cast<hipStream_t>(stream)));
}

int moe_layer_forward(const moe_layer_args* a, void* ws, size_t ws_bytes, void* stream) {
  if (!a) return MOE_ERR_NULL;
  if (a->struct_size < MOE_LAYER_ARGS_V1_SIZE) return MOE_ERR_UNSUPPORTED;
  const int T = a->T, d = a->d, E = a->E, H = a->H, k = a->k, dtype = a->dtype;
  int st = check_dims(T, d, E, H, k, dtype);
  if (st != MOE_OK) return st;
  st = check_scoring(a->scoring, a->sel_bias);
  if (st != MOE_OK) return st;
  // expert weight type: 0 (a zero-initialised struct) or the ABI-1 layout means the activation
  // dtype
  const bool abi2 = a->struct_size >= MOE_LAYER_ARGS_V2_SIZE;
  const int w_dtype = (abi2 && a->w_dtype != 0) ? a->w_dtype : dtype;
  moe::QuantWeights qw{};
  if (w_dtype != dtype) {
    // the prepared decode formats: int8 or 4-bit codes, and the fragment-major order of these or
    // of bf16 weights
    const bool frag = w_dtype == MOE_BF16_FRAG || w_dtype == MOE_I8_FRAG || w_dtype == MOE_Q4_FRAG;
    const int base = w_dtype == MOE_BF16_FRAG ? MOE_BF16
                     : (w_dtype == MOE_I8_FRAG ? MOE_I8 : (w_dtype == MOE_Q4_FRAG ? MOE_Q4 : w_dtype));
    // fragment-major bf16 weights serve both kernel families; the codes, the decode path only
    if ((base != MOE_BF16 && base != MOE_I8 && base != MOE_Q4) || dtype != MOE_BF16 ||
        (base != MOE_BF16 && !moe::ffn_bf16_streaming(T, d, E, H, k)))
      return MOE_ERR_UNSUPPORTED;
    const int fmt = (base == MOE_I8 ? moe::kWI8 : (base == MOE_Q4 ? moe::kWQ4 : moe::kWBf16)) |
                    (frag ? moe::kWFragMajor : 0);
    if (base == MOE_BF16) {
      qw = moe::QuantWeights{fmt, nullptr, nullptr, nullptr};
    } else {
      if (!a->w_gate_scale || !a->w_up_scale || !a->w_down_scale) return MOE_ERR_NULL;
      if (!aligned16(a->w_gate_scale) || !aligned16(a->w_up_scale) || !aligned16(a->w_down_scale))
        return MOE_ERR_SHAPE;
      qw = moe::QuantWeights{fmt, a->w_gate_scale, a->w_up_scale, a->w_down_scale};
    }
  }
  const bool abi4 = a->struct_size >= offsetof(moe_layer_args, y_dtype) + sizeof(a->y_dtype);
  const int y_dtype = abi4 ? a->y_dtype : MOE_F32;
  if (y_dtype != MOE_F32 && y_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!a->x || !a->w_router || !a->w_gate || !a->w_up || !a->w_down || !a->y) return MOE_ERR_NULL;
  const void* ptrs[] = {a->x, a->w_router, a->router_bias, a->sel_bias, a->w_gate, a->w_up,
                        a->w_down, a->y, a->logits, a->topk_ids, a->topk_w, a->expert_counts};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return MOE_ERR_SHAPE;
  const Layout lay(T, d, E, H, k, dtype);
  if (!ws || ws_bytes < lay.total) return MOE_ERR_WORKSPACE;
  if (!aligned16(ws)) return MOE_ERR_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // stage events are host-launch timing: refused, with nothing enqueued, during graph capture
  if (a->prof_events && capturing(s)) return MOE_ERR_UNSUPPORTED;
  clear_stale_error();
  void* const* ev = a->prof_events;
  auto mark = [&](int i) -> hipError_t { return ev ? record_event(ev[i], s) : hipSuccess; };

  int32_t* ids = a->topk_ids ? a->topk_ids : at<int32_t>(ws, lay.ids);
  float* w = a->topk_w ? a->topk_w : at<float>(ws, lay.w);
  int32_t* counts = a->expert_counts ? a->expert_counts : at<int32_t>(ws, lay.counts);
  int32_t* offsets = at<int32_t>(ws, lay.offsets);
  int32_t* sorted_rows = at<int32_t>(ws, lay.sorted_rows);
  int32_t* row_pos = at<int32_t>(ws, lay.row_pos);
  float* eo = at<float>(ws, lay.eo);
  // few rows per expert (decode): the expert kernels find their rows from the ids themselves
  const bool streaming = dtype == MOE_BF16 && moe::ffn_bf16_streaming(T, d, E, H, k);
  // k == 2 adds two weighted outputs into a cleared fp32 y with fp32 atomics (deterministic: two
  // addends onto 0) on the streaming path; elsewhere, for k > 2 and for a bf16 y, expert outputs
  // are staged and combined in slot order
  const bool y_bf16 = y_dtype == MOE_BF16;
  const bool atomic_y = k == 2 && streaming && !y_bf16;
  float* zero_y = atomic_y ? static_cast<float*>(a->y) : nullptr;

  DownArgs down{};
  down.topk_w = w;
  down.k = k;
  down.y_bf16 = y_bf16 ? 1 : 0;
  if (k == 1) {
    down.mode = moe::kDownStoreY;
    down.out = a->y;
  } else if (atomic_y) {
    down.mode = moe::kDownAtomicY;
    down.out = a->y;
  } else {
    down.mode = moe::kDownExpertOut;
    down.out = eo;
  }

  const RouteOut ro{ids, w, nullptr, zero_y, d};
  MOE_TRY(mark(0));
  if (dtype == MOE_BF16) {
    if (moe::route_split_ks(T, d, E) > 0)
      MOE_TRY(moe::launch_route_split_bf16(
          static_cast<const uint16_t*>(a->x), static_cast<const uint16_t*>(a->w_router),
          a->router_bias, a->sel_bias, T, d, E, k, a->scoring, a->logits, at<float>(ws, lay.rpart),
          ro, s));
    else
      MOE_TRY(moe::launch_route_fused_bf16(
          static_cast<const uint16_t*>(a->x), static_cast<const uint16_t*>(a->w_router),
          a->router_bias, a->sel_bias, T, d, E, k, a->scoring, a->logits, ro, s));
  } else {
    float* logits = a->logits ? a->logits : at<float>(ws, lay.logits);
    MOE_TRY(moe::launch_logits_f32(static_cast<const float*>(a->x),
                                   static_cast<const float*>(a->w_router), a->router_bias, T, d, E,
                                   logits, s));
    MOE_TRY(moe::launch_route_from_logits(logits, a->sel_bias, T, E, k, a->scoring, ro, s));
  }
  MOE_TRY(mark(1));
  if (!streaming)
    MOE_TRY(moe::launch_dispatch(ids, T * k, E, offsets, sorted_rows, row_pos, counts, s));
  // [2], [3]: the gate/up kernel's own start and end (see moe_layer_args.prof_events)
  const moe::StageMarks gu{ev ? ev[2] : nullptr, ev ? ev[3] : nullptr};
  if (dtype == MOE_BF16) {
    const RowSource rs = streaming ? RowSource{ids, T * k, nullptr, nullptr, counts}
                                   : RowSource{nullptr, T * k, offsets, sorted_rows, nullptr};
    MOE_TRY(moe::launch_ffn_bf16(static_cast<const uint16_t*>(a->x), a->w_gate, a->w_up,
                                 a->w_down, T, d, E, H, k, rs, at<uint16_t>(ws, lay.h), down, s,
                                 gu, qw));
  } else {
    MOE_TRY(moe::launch_ffn_f32(
        static_cast<const float*>(a->x), static_cast<const float*>(a->w_gate),
        static_cast<const float*>(a->w_up), static_cast<const float*>(a->w_down), T, d, E, H, k,
        offsets, sorted_rows, at<float>(ws, lay.h), down, s, gu));
  }
  // staged expert outputs (by assignment row on the streaming path, in dispatch order
  // otherwise) are combined in slot order
  if (k > 1 && !atomic_y)
    MOE_TRY(moe::launch_combine(eo, streaming ? nullptr : row_pos, w, T, d, k, a->y, y_bf16, s));
  MOE_TRY(mark(4));
  return MOE_OK;
}

}  // extern "C"
