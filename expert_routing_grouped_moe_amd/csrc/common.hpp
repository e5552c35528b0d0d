// Shared device helpers for the gfx950 MoE kernels: bf16 bit handling, 16-byte vector types,
// the CDNA4 bf16 MFMA wrapper and wave64 utilities.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int kWave = 64;
constexpr int kMaxE = 256;
constexpr int kMaxK = 8;

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x7FFFFFu)) return static_cast<uint16_t>((u >> 16) | 0x40);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ void store16(void* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) {
  return __builtin_bit_cast(bf16x8, v);
}

typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;

__device__ __forceinline__ f16x8 as_f16x8(u32x4 v) { return __builtin_bit_cast(f16x8, v); }

// fp32 -> fp16 bits, round to nearest even, saturated to +-65504 (no infinities from finite h);
// NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_f16_bits_sat(float f) {
  if (f != f) return 0x7e00;
  const float c = fminf(fmaxf(f, -65504.0f), 65504.0f);
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(c));
}

// Eight bf16 values (four dwords, lowest first) as eight fp16 values. Exact for every bf16
// value of magnitude >= 2^-17 and <= 65504 (fp16 holds bf16's 8 significant bits there); the
// pack rounds toward zero, which only affects smaller, fp16-subnormal magnitudes.
__device__ __forceinline__ u32x4 bf16x8_to_f16x8(u32x4 v) {
  u32x4 out;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = __uint_as_float(v[i] << 16);
    const float hi = __uint_as_float(v[i] & 0xffff0000u);
    out[i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
  }
  return out;
}

// 16 bytes per lane from `g` into LDS at byte address lds + 16 * lane (lds wave-uniform). Issued
// as inline asm so that the compiler's own wait-count tracking (which would otherwise wait for
// every outstanding DMA before any LDS read) leaves the pipeline alone; the waits are explicit.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(g), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

// D = A(16x32) * B(32x16) + C on the CDNA4 matrix cores, fp32 accumulate.
// Lane l supplies row (l % 16) of A and column (l % 16) of B, eight consecutive k each
// (k = 8 * (l / 16) + 0..7); it receives C rows 4 * (l / 16) + 0..3 of column (l % 16).
// Any fixed lane->k assignment used identically for A and B gives the same sum over k.
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}
// The same product on fp16 operands (same lane layout).
__device__ __forceinline__ f32x4 mfma16x16x32_f16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(a), as_f16x8(b), c, 0, 0, 0);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }
__device__ __forceinline__ float silu_precise(float z) { return z / (1.0f + expf(-z)); }

// Upper bound on the number of row tiles of height bm over E expert groups holding `rows` rows
// in total: sum_e ceil(c_e / bm) <= (rows + E (bm - 1)) / bm, and never more than rows.
__host__ __device__ inline int max_tiles(int rows, int E, int bm) {
  if (rows <= 0) return 0;
  const long long bound = (static_cast<long long>(rows) + static_cast<long long>(E) * (bm - 1)) / bm;
  return static_cast<int>(bound < rows ? bound : rows);
}

// Expert tile bookkeeping shared by the grouped FFN kernels. Expert e owns ceil(count_e / bm)
// row tiles; tiles are numbered expert by expert. tile_scan() loads the offsets and the inclusive
// per-expert tile counts into LDS (`sh`, 2 * (E + 1) ints) and returns the number of tiles; every
// thread of the block must call it. tile_lookup() then maps a tile index to its expert and rows.
struct TileInfo {
  int e;      // expert, or -1 when the tile index is past the last tile
  int row0;   // first position in the grouped row order covered by the tile
  int rows;   // rows of the tile that belong to expert e (1..bm)
};

__device__ inline int tile_scan(const int32_t* __restrict__ offsets, int E, int bm, int* sh) {
  int* soff = sh;
  int* scum = sh + E + 1;
  for (int i = threadIdx.x; i <= E; i += blockDim.x) soff[i] = offsets[i];
  __syncthreads();
  if (threadIdx.x < kWave) {
    // one wave scans E <= 256 tile counts, four per lane
    const int lane = threadIdx.x;
    int c[4];
    int run = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane * 4 + q;
      int n = 0;
      if (e < E) {
        const int cnt = soff[e + 1] - soff[e];
        n = (cnt + bm - 1) / bm;
      }
      run += n;
      c[q] = run;
    }
    int tot = run;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int v = __shfl_up(tot, o);
      if (lane >= o) tot += v;
    }
    const int excl = tot - run;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane * 4 + q;
      if (e < E) scum[e] = excl + c[q];
    }
  }
  __syncthreads();
  return scum[E - 1];
}

__device__ inline TileInfo tile_lookup(int E, int bm, int tile, const int* sh) {
  const int* soff = sh;
  const int* scum = sh + E + 1;
  TileInfo ti;
  ti.e = -1;
  ti.row0 = 0;
  ti.rows = 0;
  if (tile < 0 || tile >= scum[E - 1]) return ti;
  int lo = 0, hi = E - 1;  // first expert whose inclusive tile count exceeds `tile`
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (scum[mid] > tile) hi = mid; else lo = mid + 1;
  }
  const int before = lo > 0 ? scum[lo - 1] : 0;
  const int m0 = (tile - before) * bm;
  const int cnt = soff[lo + 1] - soff[lo];
  ti.e = lo;
  ti.row0 = soff[lo] + m0;
  ti.rows = min(bm, cnt - m0);
  return ti;
}

__device__ inline TileInfo find_tile(const int32_t* __restrict__ offsets, int E, int bm, int tile,
                                     int* sh) {
  tile_scan(offsets, E, bm, sh);
  return tile_lookup(E, bm, tile, sh);
}

}  // namespace moe
