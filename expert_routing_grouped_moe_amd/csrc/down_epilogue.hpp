// Delivery of one down-projection output element (step 6 -> step 7).
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

// o = expert output of assignment row r (token t = r / k, slot j = r % k), stored at position p
// of the expert-output array. Combine rule (zonos2.cpp INTERNALS, "Model architecture" table,
// Router row: the chosen experts' outputs are summed with their routing weights; "Notes": the
// residual stream is F32):
//   kDownExpertOut  expert_out[p, n] = o
//   kDownStoreY     y[t, n] = w[t, j] * o           (k == 1; fp32, or bf16 rounded to nearest
//                   even when y_bf16)
//   kDownAtomicY    y[t, n] += w[t, j] * o          (k == 2, y cleared beforehand; two addends
//                   onto 0 give fl(a + b) in either order, so the result is deterministic)
struct DownRow {
  void* dst;    // row pointer in expert_out or y (fp32, or bf16 bits)
  float scale;  // routing weight (1 for expert_out)
};

__device__ __forceinline__ DownRow down_row(const DownArgs& a, int r, int p, int d) {
  DownRow out;
  if (a.mode == kDownExpertOut) {
    out.dst = static_cast<float*>(a.out) + static_cast<long long>(p) * d;
    out.scale = 1.0f;
  } else {
    const long long off = static_cast<long long>(r / a.k) * d;
    out.dst = (a.mode == kDownStoreY && a.y_bf16) ? static_cast<void*>(static_cast<uint16_t*>(a.out) + off)
                                                  : static_cast<void*>(static_cast<float*>(a.out) + off);
    out.scale = a.topk_w[r];
  }
  return out;
}

__device__ __forceinline__ void down_put(const DownArgs& a, const DownRow& r, int n, float o) {
  if (a.mode == kDownAtomicY) {
    unsafeAtomicAdd(static_cast<float*>(r.dst) + n, r.scale * o);
  } else if (a.mode == kDownStoreY) {
    if (a.y_bf16)
      static_cast<uint16_t*>(r.dst)[n] = f32_to_bf16_bits(r.scale * o);
    else
      static_cast<float*>(r.dst)[n] = r.scale * o;
  } else {
    static_cast<float*>(r.dst)[n] = o;
  }
}

// Four consecutive outputs n .. n + 3 (fp32 bits in v), delivered as down_put does for each:
// one 16-byte store (8 bytes for a bf16 y) where the mode stores.
__device__ __forceinline__ void down_put4(const DownArgs& a, const DownRow& r, int n, u32x4 v) {
  if (a.mode == kDownAtomicY) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      unsafeAtomicAdd(static_cast<float*>(r.dst) + n + i, r.scale * __uint_as_float(v[i]));
  } else if (a.mode == kDownStoreY) {
    float o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = r.scale * __uint_as_float(v[i]);
    if (a.y_bf16) {
      const uint32_t lo = f32_to_bf16_bits(o[0]) | (static_cast<uint32_t>(f32_to_bf16_bits(o[1])) << 16);
      const uint32_t hi = f32_to_bf16_bits(o[2]) | (static_cast<uint32_t>(f32_to_bf16_bits(o[3])) << 16);
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(r.dst) + n) = make_uint2(lo, hi);
    } else {
      store16(static_cast<float*>(r.dst) + n, u32x4{__float_as_uint(o[0]), __float_as_uint(o[1]),
                                                    __float_as_uint(o[2]), __float_as_uint(o[3])});
    }
  } else {
    store16(static_cast<float*>(r.dst) + n, v);
  }
}

}  // namespace moe
