// Host-side launchers of the MoE kernels (internal to libmoe.so). Each returns the
// hipGetLastError() of its launches. Arguments are validated by the C-ABI layer before these run.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

enum Scoring { kSoftmax = 0, kSelectedSoftmax = 1, kSigmoid = 2 };

constexpr int kTokTile = 16;  // tokens per routing block; also the dispatch block of rows

// How the down-projection epilogue delivers its result.
enum DownOut {
  kDownExpertOut = 0,  // expert_out[p, :] = o                       (fp32)
  kDownStoreY = 1,     // y[t, :] = w * o            (k == 1: each token written once)
  kDownAtomicY = 2     // y[t, :] += w * o on a zeroed y (k == 2: two addends, order-free)
};

struct DownArgs {
  int mode;                 // DownOut
  void* out;                // expert_out (fp32) or y (fp32, or bf16 bits when y_bf16)
  const float* topk_w;      // [T, k]
  int k;
  int y_bf16;               // kDownStoreY: y holds bf16 (the fp32 value rounded to nearest even)
};

// Outputs of the routing tail (any may be NULL except ids and w).
struct RouteOut {
  int32_t* ids;         // [T, k]
  float* w;             // [T, k]
  int32_t* counts;      // [E], accumulated with integer atomics on a zeroed array
  float* zero_y;        // [T, d] cleared (for the two-addend atomic combine)
  int d;
};

// Stage marker for the optional timing events: an event record on `s` (defined in moe_api.hip;
// the layer refuses timing events while `s` is being captured into a graph).
hipError_t record_stage_event(void* ev, hipStream_t s);

// Optional timing events around one kernel (hipEvent_t handles, or NULL).
struct StageMarks {
  void* start;
  void* end;
};

// Launches `kernel` on `s`. With both marks set the launch goes through hipExtLaunchKernelGGL
// so that the two events take the kernel's own start and end times; otherwise the marks that are
// set are recorded before and after the launch.
template <typename... Params, typename... Args>
hipError_t launch_marked(void (*kernel)(Params...), dim3 grid, dim3 block, hipStream_t s,
                         const StageMarks& m, Args... args) {
  hipError_t err;
  if (m.start && m.end) {
    hipExtLaunchKernelGGL(kernel, grid, block, 0, s, static_cast<hipEvent_t>(m.start),
                          static_cast<hipEvent_t>(m.end), 0, args...);
    return hipGetLastError();
  }
  if (m.start && (err = record_stage_event(m.start, s)) != hipSuccess) return err;
  kernel<<<grid, block, 0, s>>>(args...);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (m.end && (err = record_stage_event(m.end, s)) != hipSuccess) return err;
  return hipSuccess;
}

// ---------------------------------------------------------------- routing (route.hip)
hipError_t launch_zero_i32(int32_t* p, int n, hipStream_t s);
hipError_t launch_zero_f32(float* p, long long n, hipStream_t s);

hipError_t launch_logits_f32(const float* x, const float* wr, const float* rb, int T, int d,
                             int E, float* logits, hipStream_t s);
hipError_t launch_logits_bf16(const uint16_t* x, const uint16_t* wr, const float* rb, int T,
                              int d, int E, float* logits, hipStream_t s);

// top-k + weights from fp32 logits in global memory.
hipError_t launch_route_from_logits(const float* logits, const float* sel_bias, int T, int E,
                                    int k, int scoring, const RouteOut& o, hipStream_t s);

// Small batches (T <= kRouteSplitMaxT) with a large router matrix route in two kernels: partial
// logit tiles over d-slices spread across many CUs, then the sum and the selection.
// route_split_ks() is the number of slices (0: the fused router is used); `part` holds
// ks * T * E floats.
constexpr int kRouteSplitMaxT = 256;
int route_split_ks(int T, int d, int E);
hipError_t launch_route_split_bf16(const uint16_t* x, const uint16_t* wr, const float* rb,
                                   const float* sel_bias, int T, int d, int E, int k, int scoring,
                                   float* logits_out, float* part, const RouteOut& o,
                                   hipStream_t s);

// logits on MFMA + top-k + weights in one kernel (bf16 x / router weight); logits_out optional.
hipError_t launch_route_fused_bf16(const uint16_t* x, const uint16_t* wr, const float* rb,
                                   const float* sel_bias, int T, int d, int E, int k, int scoring,
                                   float* logits_out, const RouteOut& o, hipStream_t s);

// ---------------------------------------------------------------- dispatch (permute.hip)
// offsets [E+1], sorted_rows / row_pos [n_rows] from the expert ids; counts_out may be NULL.
hipError_t launch_dispatch(const int32_t* ids, int n_rows, int E, int32_t* offsets,
                           int32_t* sorted_rows, int32_t* row_pos, int32_t* counts_out,
                           hipStream_t s);
// counts[e] = #{r < n_rows : ids[r] == e} (one block; E <= kMaxE)
hipError_t launch_counts(const int32_t* ids, int n_rows, int E, int32_t* counts, hipStream_t s);
// Byte offset, inside the layer's workspace, of the expert ids that moe_layer_forward writes there
// when the caller passes no topk_ids (same sizes as moe_workspace_size).
size_t layer_ids_offset(int T, int d, int E, int H, int k, int dtype);

// ---------------------------------------------------------------- experts (ffn_*.hip)
// Where a grouped FFN finds the rows of expert e:
//   grouped (ids == NULL): rows sorted_rows[offsets[e] + i]; h and expert_out at offsets[e] + i
//   by ids  (ids != NULL): the rows r (ascending) with ids[r] == e; h and expert_out at row r
struct RowSource {
  const int32_t* ids;
  int n_rows;               // T * k
  const int32_t* offsets;   // [E + 1] (grouped)
  const int32_t* sorted_rows;
  int32_t* counts_out;      // by-ids mode may write expert counts here (or NULL)
};

// True when the weight-streaming kernels handle this shape (few rows per expert).
bool ffn_bf16_streaming(int T, int d, int E, int H, int k);
// Largest T*k the by-ids row scan supports.
constexpr int kMaxScanRows = 2048;

// Storage of the expert weights on the bf16 path.
enum WeightFormat {
  kWBf16 = 0,  // bf16 bits
  kWI8 = 1,    // int8 codes, fp32 row scales `gate`, `up`, `down` ([E,H], [E,H], [E,d])
  kWQ4 = 2,    // packed 4-bit codes, uint32 (scale, bias) pairs per group of 64 along K
  // flag on any of the above: the stacks' bytes in fragment-major order (moe_pack_weights_frag)
  kWFragMajor = 4
};
struct QuantWeights {
  int fmt;           // WeightFormat
  const void* gate;  // quantisation arrays of the three stacks (NULL for bf16)
  const void* up;
  const void* down;
};

// h is the [T*k, H] intermediate (bf16 bits or fp32). `gu` marks the gate/up launch (timing).
// wg, wu, wd are in the storage `qw.fmt` names; quantised formats on weight-streaming shapes
// only (hipErrorInvalidValue otherwise).
hipError_t launch_ffn_bf16(const uint16_t* x, const void* wg, const void* wu, const void* wd,
                           int T, int d, int E, int H, int k, const RowSource& rs, uint16_t* h,
                           const DownArgs& down, hipStream_t s, const StageMarks& gu,
                           const QuantWeights& qw);
hipError_t launch_ffn_f32(const float* x, const float* wg, const float* wu, const float* wd,
                          int T, int d, int E, int H, int k, const int32_t* offsets,
                          const int32_t* sorted_rows, float* h, const DownArgs& down,
                          hipStream_t s, const StageMarks& gu);

// ---------------------------------------------------------- quantised weights (quant.hip)
// Per-row symmetric int8 codes of a [rows, K] matrix (bf16 bits or fp32), K % 16 == 0.
hipError_t launch_quantize_rows_i8(const void* w, long long rows, int K, bool bf16, int8_t* q,
                                   float* scales, hipStream_t s);
// 4-bit affine codes in groups of 64 (packed order and pairs as in moe_quantize_groups_q4),
// K % 128 == 0.
hipError_t launch_quantize_groups_q4(const void* w, long long rows, int K, bool bf16, uint8_t* q,
                                     uint32_t* qpar, hipStream_t s);
// Fragment-major order (moe_pack_weights_frag) of a [rows, row_bytes] matrix stored as `fmt`
// (kWBf16, kWI8 or kWQ4; row_bytes = 2 K, K or K / 2); rows % 16 == 0, row_bytes % 64 == 0 (bf16)
// or K % 128 == 0 (codes).
hipError_t launch_pack_frag(const void* w, long long rows, int row_bytes, int fmt, void* out,
                            hipStream_t s);

// ---------------------------------------------------------------- combine (combine.hip)
// row_pos == NULL: expert_out is indexed by the assignment row itself. y_bf16: y holds bf16 bits
// (the fp32 sum rounded once to nearest even), else fp32.
hipError_t launch_combine(const float* expert_out, const int32_t* row_pos, const float* w, int T,
                          int d, int k, void* y, bool y_bf16, hipStream_t s);

}  // namespace moe
