// Symmetric per-row int8 codes of expert weights, for the quantised decode path (moe_quantize_rows_i8).
//   s = fp32(max_i |w_i| / 127),   q_i = clamp(rint(fp32(w_i / s)), -127, 127)   (ties to even)
// both divisions IEEE round-to-nearest-even (__fdiv_rn), so the codes are defined exactly; an
// all-zero row gets s = 0 and q = 0. The pages run quantised expert stacks for decode
// (ZONOS2-4bit MLX card, "Performance notes"; zonos2.cpp INTERNALS, "Recommended: F16 spine +
// K-quant experts"); this per-row int8 code is the library's own.
//
// One wave per row: the largest magnitude by a wave reduction, then the codes, four per lane per
// step (K % 16 == 0, so every four-code group is one aligned 32-bit store).
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kQRowsPerBlock = 4;

__device__ __forceinline__ void load4(const void* w, bool bf16, long long idx, float* v) {
  if (bf16) {
    const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(w) + idx);
    v[0] = __uint_as_float(u.x << 16);
    v[1] = __uint_as_float(u.x & 0xffff0000u);
    v[2] = __uint_as_float(u.y << 16);
    v[3] = __uint_as_float(u.y & 0xffff0000u);
  } else {
    const float4 f = *reinterpret_cast<const float4*>(static_cast<const float*>(w) + idx);
    v[0] = f.x;
    v[1] = f.y;
    v[2] = f.z;
    v[3] = f.w;
  }
}

__global__ __launch_bounds__(kWave * kQRowsPerBlock) void quantize_rows_i8_kernel(
    const void* __restrict__ w, long long rows, int K, bool bf16, int8_t* __restrict__ q,
    float* __restrict__ scales) {
  const long long row = static_cast<long long>(blockIdx.x) * kQRowsPerBlock + threadIdx.x / kWave;
  if (row >= rows) return;
  const int lane = lane_id();
  const long long base = row * K;
  float m = 0.f;
  for (int i = lane * 4; i < K; i += kWave * 4) {
    float v[4];
    load4(w, bf16, base + i, v);
#pragma unroll
    for (int j = 0; j < 4; ++j) m = fmaxf(m, fabsf(v[j]));
  }
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  const float s = m > 0.f ? __fdiv_rn(m, 127.f) : 0.f;
  if (lane == 0) scales[row] = s;
  for (int i = lane * 4; i < K; i += kWave * 4) {
    float v[4];
    load4(w, bf16, base + i, v);
    uint32_t packed = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int c = 0;
      if (s > 0.f) c = static_cast<int>(fminf(127.f, fmaxf(-127.f, rintf(__fdiv_rn(v[j], s)))));
      packed |= (static_cast<uint32_t>(c) & 0xffu) << (8 * j);
    }
    *reinterpret_cast<uint32_t*>(q + base + i) = packed;
  }
}

}  // namespace

hipError_t launch_quantize_rows_i8(const void* w, long long rows, int K, bool bf16, int8_t* q,
                                   float* scales, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const long long blocks = (rows + kQRowsPerBlock - 1) / kQRowsPerBlock;
  quantize_rows_i8_kernel<<<static_cast<unsigned>(blocks), kWave * kQRowsPerBlock, 0, s>>>(
      w, rows, K, bf16, q, scales);
  return hipGetLastError();
}

}  // namespace moe
