// Prepared expert weights for the decode path: 4-bit affine group codes
// (moe_quantize_groups_q4, below), symmetric per-row int8 codes (moe_quantize_rows_i8) and the
// fragment-major order of any of these or of bf16 weights (moe_pack_weights_frag, exact). The int8
// codes:
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

// 4-bit affine codes, groups of 64 along K (moe_quantize_groups_q4): one thread per group.
//   lo, hi = min, max;  s = bf16(fp32(fp32(hi - lo) / 15));  b = bf16(lo)
//   q_i = clamp(rint(fp32(fp32(w_i - b) / s)), 0, 15)      (s == 0: q_i = 0)
// with IEEE round-to-nearest-even subtractions and divisions (__fsub_rn, __fdiv_rn) and bf16()
// rounding to nearest even, so codes, scale and bias are defined exactly. The ZONOS2-4bit card
// quantises the experts affinely at 4 bits in groups of 64 ("Quantization recipe"); this
// arithmetic is the library's reading of that scheme.
// Group G of a row covers k = 64 G .. 64 G + 63, i.e. MFMA steps c = 2 (G % 2) and 2 (G % 2) + 1
// of block G / 2 for all four lane groups: eight packed words, written separately.
constexpr int kQ4Group = 64;

__device__ __forceinline__ float bf16_round(float v) {
  const uint32_t u = __float_as_uint(v);
  return __uint_as_float(((u + 0x7fffu + ((u >> 16) & 1u)) >> 16) << 16);
}

__global__ __launch_bounds__(256) void quantize_groups_q4_kernel(
    const void* __restrict__ w, long long groups, int K, bool bf16, uint8_t* __restrict__ q,
    uint32_t* __restrict__ qpar) {
  const long long gi = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gi >= groups) return;
  const int gpr = K / kQ4Group;                 // groups per row
  const long long row = gi / gpr;
  const int G = static_cast<int>(gi - row * gpr);
  const long long base = row * K + static_cast<long long>(G) * kQ4Group;
  float v[kQ4Group];
#pragma unroll
  for (int i = 0; i < kQ4Group; i += 4) load4(w, bf16, base + i, v + i);
  float lo = v[0], hi = v[0];
#pragma unroll
  for (int i = 1; i < kQ4Group; ++i) {
    lo = fminf(lo, v[i]);
    hi = fmaxf(hi, v[i]);
  }
  const float sc = bf16_round(__fdiv_rn(__fsub_rn(hi, lo), 15.f));
  const float bs = bf16_round(lo);
  qpar[gi] = (__float_as_uint(sc) >> 16) | (__float_as_uint(bs) & 0xffff0000u);
  uint32_t* out = reinterpret_cast<uint32_t*>(q + row * (K / 2) + 64 * (G / 2));
  const int c0 = 2 * (G % 2);
#pragma unroll
  for (int cc = 0; cc < 2; ++cc) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      uint32_t word = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float x = v[32 * cc + 8 * g + i];  // k = 64 G + 32 cc + 8 g + i
        uint32_t code = 0;
        if (sc > 0.f)
          code = static_cast<uint32_t>(fminf(15.f, fmaxf(0.f, rintf(__fdiv_rn(__fsub_rn(x, bs), sc)))));
        word |= code << ((i & 1) ? 16 + 4 * (i >> 1) : 4 * (i >> 1));
      }
      out[4 * g + c0 + cc] = word;
    }
  }
}

// Fragment-major weights (moe_pack_weights_frag): one thread per 16-byte piece of the output. A
// slab of 16 rows is stored as row_bytes / 64 chunks of 1024 bytes; lane l's piece of chunk i is a
// piece of row l % 16: piece 4 i + l / 16 of the row for bf16 values and packed 4-bit codes (the
// 64 bytes of each row in chunk i go to four lane groups in order), piece 8 (i / 2) + 2 (l / 16) +
// i % 2 for int8 codes (lane group g's 32 codes of a 128-k block, as two pieces). The writes are
// contiguous; each wave reads 16 rows x 64 bytes (a one-time preparation).
__global__ __launch_bounds__(256) void pack_frag_kernel(const uint8_t* __restrict__ w,
                                                        long long pieces, int row_bytes, bool i8,
                                                        uint8_t* __restrict__ out) {
  const long long stride = static_cast<long long>(gridDim.x) * blockDim.x;
  const int chunks = row_bytes / 64;   // per slab
  for (long long p = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x; p < pieces;
       p += stride) {
    const long long chunk = p >> 6;
    const int l = static_cast<int>(p & 63);
    const long long b = chunk / chunks;
    const int i = static_cast<int>(chunk - b * chunks);
    const long long row = 16 * b + (l & 15);
    const int piece = i8 ? 8 * (i >> 1) + 2 * (l >> 4) + (i & 1) : 4 * i + (l >> 4);
    store16(out + 16 * p, load16(w + row * row_bytes + 16 * piece));
  }
}

}  // namespace

hipError_t launch_pack_frag(const void* w, long long rows, int row_bytes, int fmt, void* out,
                            hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const long long pieces = rows * row_bytes / 16;
  const long long blocks = (pieces + 255) / 256;
  const unsigned grid = static_cast<unsigned>(blocks < (1ll << 20) ? blocks : (1ll << 20));
  pack_frag_kernel<<<grid, 256, 0, s>>>(static_cast<const uint8_t*>(w), pieces, row_bytes,
                                        fmt == kWI8, static_cast<uint8_t*>(out));
  return hipGetLastError();
}

hipError_t launch_quantize_groups_q4(const void* w, long long rows, int K, bool bf16, uint8_t* q,
                                     uint32_t* qpar, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const long long groups = rows * (K / kQ4Group);
  const long long blocks = (groups + 255) / 256;
  quantize_groups_q4_kernel<<<static_cast<unsigned>(blocks), 256, 0, s>>>(w, groups, K, bf16, q,
                                                                          qpar);
  return hipGetLastError();
}

hipError_t launch_quantize_rows_i8(const void* w, long long rows, int K, bool bf16, int8_t* q,
                                   float* scales, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const long long blocks = (rows + kQRowsPerBlock - 1) / kQRowsPerBlock;
  quantize_rows_i8_kernel<<<static_cast<unsigned>(blocks), kWave * kQRowsPerBlock, 0, s>>>(
      w, rows, K, bf16, q, scales);
  return hipGetLastError();
}

}  // namespace moe
