// Host-side launchers of the MoE kernels (internal to libmoe.so). Each returns the
// hipGetLastError() of its launches. Arguments are validated by the C-ABI layer before these run.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

enum Scoring { kSoftmax = 0, kSelectedSoftmax = 1 };

// How the down-projection epilogue delivers its result.
enum DownOut {
  kDownExpertOut = 0,  // expert_out[p, :] = o                       (grouped order, fp32)
  kDownStoreY = 1,     // y[t, :] = w * o            (k == 1: each token written once)
  kDownAtomicY = 2     // y[t, :] += w * o on a zeroed y (k == 2: two addends, order-free)
};

struct DownArgs {
  int mode;                 // DownOut
  float* out;               // expert_out or y
  const int32_t* sorted_rows;
  const float* topk_w;      // [T, k]
  int k;
};

// Stage marker for the optional timing events: an external event node while `s` is being
// captured into a graph, a plain event record otherwise (defined in moe_api.hip).
hipError_t record_stage_event(void* ev, hipStream_t s);

// ---------------------------------------------------------------- routing (route.hip)
hipError_t launch_zero_i32(int32_t* p, int n, hipStream_t s);
hipError_t launch_zero_f32(float* p, long long n, hipStream_t s);

hipError_t launch_logits_f32(const float* x, const float* wr, const float* rb, int T, int d,
                             int E, float* logits, hipStream_t s);
hipError_t launch_logits_bf16(const uint16_t* x, const uint16_t* wr, const float* rb, int T,
                              int d, int E, float* logits, hipStream_t s);

// top-k + weights from fp32 logits in global memory. counts may be NULL; when not NULL they
// are overwritten. zero_y (may be NULL) gets rows [T, d] cleared.
hipError_t launch_route_from_logits(const float* logits, const float* sel_bias, int T, int E,
                                    int k, int scoring, int32_t* ids, float* w, int32_t* counts,
                                    float* zero_y, int d, hipStream_t s);

// logits on MFMA + top-k + weights in one kernel (bf16 x / router weight).
hipError_t launch_route_fused_bf16(const uint16_t* x, const uint16_t* wr, const float* rb,
                                   const float* sel_bias, int T, int d, int E, int k, int scoring,
                                   float* logits_out, int32_t* ids, float* w, float* zero_y,
                                   hipStream_t s);

// ---------------------------------------------------------------- dispatch (permute.hip)
// counts_in may be NULL (then computed); counts_out may be NULL.
hipError_t launch_permute(const int32_t* ids, const int32_t* counts_in, int n_rows, int E,
                          int32_t* offsets, int32_t* sorted_rows, int32_t* row_pos,
                          int32_t* counts_out, hipStream_t s);

// ---------------------------------------------------------------- experts (ffn_*.hip)
// h is the [T*k, H] intermediate in grouped order (bf16 bits or fp32). `mid_event` (a hipEvent_t
// or NULL) is recorded on `s` between the gate/up and the down launches.
hipError_t launch_ffn_bf16(const uint16_t* x, const uint16_t* wg, const uint16_t* wu,
                           const uint16_t* wd, int T, int d, int E, int H, int k,
                           const int32_t* offsets, const int32_t* sorted_rows, uint16_t* h,
                           const DownArgs& down, hipStream_t s, void* mid_event);
hipError_t launch_ffn_f32(const float* x, const float* wg, const float* wu, const float* wd,
                          int T, int d, int E, int H, int k, const int32_t* offsets,
                          const int32_t* sorted_rows, float* h, const DownArgs& down,
                          hipStream_t s, void* mid_event);

// ---------------------------------------------------------------- combine (combine.hip)
hipError_t launch_combine(const float* expert_out, const int32_t* row_pos, const float* w, int T,
                          int d, int k, float* y, hipStream_t s);

}  // namespace moe
