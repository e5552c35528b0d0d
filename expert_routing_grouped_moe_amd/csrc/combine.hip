// Weighted combine (step 7): y[t] = sum_j w[t, j] * expert_out[row_pos[t*k + j]], slot order,
// fp32 (zonos2.cpp INTERNALS, "Model architecture" table, Router row: the chosen experts'
// outputs weighted by their routing probabilities; "Notes": the residual stream is F32), stored
// as fp32 or, on request, rounded once to bf16 (nearest even).
// One thread per four consecutive columns of one token; rows of y are written once.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

__global__ void combine_kernel(const float* __restrict__ eo, const int32_t* __restrict__ row_pos,
                               const float* __restrict__ w, int T, int d, int k,
                               void* __restrict__ y, bool y_bf16) {
  const int vec = d / 4;
  const long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<long long>(T) * vec) return;
  const int t = static_cast<int>(i / vec);
  const int c = static_cast<int>(i % vec);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; ++j) {
    const long long r = static_cast<long long>(t) * k + j;
    const float wt = w[r];
    const long long src = row_pos ? row_pos[r] : r;
    const float4 o = reinterpret_cast<const float4*>(eo + src * d)[c];
    acc.x = acc.x + wt * o.x;
    acc.y = acc.y + wt * o.y;
    acc.z = acc.z + wt * o.z;
    acc.w = acc.w + wt * o.w;
  }
  const long long o = static_cast<long long>(t) * d;
  if (y_bf16) {
    const uint32_t lo = f32_to_bf16_bits(acc.x) | (static_cast<uint32_t>(f32_to_bf16_bits(acc.y)) << 16);
    const uint32_t hi = f32_to_bf16_bits(acc.z) | (static_cast<uint32_t>(f32_to_bf16_bits(acc.w)) << 16);
    reinterpret_cast<uint2*>(static_cast<uint16_t*>(y) + o)[c] = make_uint2(lo, hi);
  } else {
    reinterpret_cast<float4*>(static_cast<float*>(y) + o)[c] = acc;
  }
}

}  // namespace

hipError_t launch_combine(const float* expert_out, const int32_t* row_pos, const float* w, int T,
                          int d, int k, void* y, bool y_bf16, hipStream_t s) {
  const long long n = static_cast<long long>(T) * (d / 4);
  if (n == 0) return hipSuccess;
  combine_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, s>>>(expert_out, row_pos, w, T,
                                                                        d, k, y, y_bf16);
  return hipGetLastError();
}

}  // namespace moe
