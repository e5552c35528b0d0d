// Router logits, top-k selection and routing weights (steps 1-3 of the MoE layer).
//
// Scoring modes (zonos2.cpp INTERNALS, "Model architecture" table, Router row; audio.cpp PR #1271,
// "Framework change"):
//   SOFTMAX           rank by logit, weight = softmax over all E logits at the chosen expert
//                     (no renormalisation over the chosen set)
//   SELECTED_SOFTMAX  rank by fp32(logit + sel_bias), weight = softmax over the k chosen raw
//                     logits
//   SIGMOID           rank by logit, weight = sigmoid(logit) of the chosen expert, no
//                     renormalisation (audio.cpp PR #1271, "Framework change": the pre-ranking
//                     sigmoid mode)
// Selection order is (score descending, expert index ascending); -0.0 == +0.0 under the IEEE
// comparison, so signed zeros fall through to the index.
//
// Work layout: a block owns 16 tokens. Selection runs on 256 threads: the 16 lanes of one DPP row
// serve one token, lane q holding the scores of experts q, q + 16, ... in registers; each slot's
// winner, the softmax maximum and the softmax sum are reduced across the row with DPP row
// rotations (8, 4, 2, 1), after which every lane of the row holds the same value. The bf16
// routing kernel first computes the 16 x E logit tile on the matrix cores with 8 waves that split
// the experts (16 per MFMA tile) and, when there are few experts, the d-long reduction; each wave
// copies its operands into LDS in 128-k chunks of whole 128-byte lines (router_product_128) and
// partial tiles are added in a fixed order, so the logits are the same on every call.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kQ = 16;                      // lanes per token in the selection (one DPP row)
static_assert(kMaxE / 16 <= 16, "at most 16 experts per selection lane");
constexpr int kTailThreads = kTokTile * kQ; // 256
// waves of the fused routing kernel: 16 measured the same at T = 64 and 4096, 15 % slower at 8192
constexpr int kFusedWaves = 8;
constexpr int kFusedThreads = kFusedWaves * kWave;
static_assert(kFusedThreads >= kMaxE, "one thread per expert for the bias preload");

__global__ void zero_i32_kernel(int32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

__global__ void zero_f32_kernel(float* p, long long n) {
  const long long i = (static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x) * 4;
  if (i + 3 < n) {
    *reinterpret_cast<float4*>(p + i) = make_float4(0.f, 0.f, 0.f, 0.f);
  } else {
    for (long long j = i; j < n; ++j) p[j] = 0.f;
  }
}

// Is candidate (s, e) ahead of (bs, be) in the selection order?
__device__ __forceinline__ bool ahead(float s, int e, float bs, int be) {
  return s > bs || (s == bs && e < be);
}

// Value of lane (i - N) mod 16 of the caller's 16-lane row (DPP row rotation; every lane of the
// wave must be active).
template <int N>
__device__ __forceinline__ int row_ror(int v) {
  static_assert(N >= 1 && N <= 15, "row rotation");
  return __builtin_amdgcn_update_dpp(0, v, 0x120 + N, 0xF, 0xF, false);
}
template <int N>
__device__ __forceinline__ float row_ror(float v) {
  return __int_as_float(row_ror<N>(__float_as_int(v)));
}

// (score, expert, raw logit) of the better of this lane's candidate and lane (i - N)'s
template <int N>
__device__ __forceinline__ void argmax_step(float& bs, int& be, float& bl) {
  const float os = row_ror<N>(bs);
  const int oe = row_ror<N>(be);
  const float ol = row_ror<N>(bl);
  const bool take = ahead(os, oe, bs, be);
  bs = take ? os : bs;
  be = take ? oe : be;
  bl = take ? ol : bl;
}
// After rotations 8, 4, 2, 1 each lane has combined all 16; lanes i and i + 2^m hold equal values
// after every step, so the row agrees (also for the floating-point sum).
__device__ __forceinline__ void row_argmax(float& bs, int& be, float& bl) {
  argmax_step<8>(bs, be, bl);
  argmax_step<4>(bs, be, bl);
  argmax_step<2>(bs, be, bl);
  argmax_step<1>(bs, be, bl);
}
__device__ __forceinline__ float row_max(float v) {
  v = fmaxf(v, row_ror<8>(v));
  v = fmaxf(v, row_ror<4>(v));
  v = fmaxf(v, row_ror<2>(v));
  return fmaxf(v, row_ror<1>(v));
}
__device__ __forceinline__ float row_sum(float v) {
  v = v + row_ror<8>(v);
  v = v + row_ror<4>(v);
  v = v + row_ror<2>(v);
  return v + row_ror<1>(v);
}

// ------------------------------------------------------------- router product, 16 x 16 tiles
// acc += A[16 rows, k0 .. k0 + 128) . B[16 rows, same k]^T as four 32-k MFMA steps in k order,
// with the same fragments as loading each lane's operands (row l % 16, k 32 s + 8 (l / 16) of step
// s) straight from global memory; k at or past kend contributes zeros (kend - k0 is a multiple
// of 8). Loaded that way, each load instruction reads 16 rows x 64 bytes, half lines, which on
// this chip copy at about half the rate of whole 128-byte lines (the routing kernels' product
// phase took twice as long). Here the operands are copied into a wave-private LDS area (4 KB per
// operand) with global_load_lds_dwordx4, each instruction 4 rows x 256 bytes, piece p of row r
// stored at p ^ r so that the 16-row fragment reads are conflict-free, and read back as fragments.
// rows[i]: the row this lane copies in instruction i (row 4 i + l / 16 of the tile), any valid
// address for rows that are not used.
constexpr int kProdScratch = 2 * 16 * 128;   // bf16 elements of LDS per wave (8 KB)

__device__ __forceinline__ f32x4 router_product_128(const uint16_t* const (&arow)[4],
                                                    const uint16_t* const (&brow)[4], int k0,
                                                    int kend, uint16_t* scratch, f32x4 acc) {
  const int lane = lane_id();
  const uint32_t la = lds_addr(scratch), lb = la + 16 * 128 * 2;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * i + (lane >> 4);
    const int p = (lane & 15) ^ r;          // the logical piece that lands in this lane's slot
    const int kk = min(k0 + 8 * p, kend - 8);
    dma16(arow[i] + kk, la + 1024u * i);
    dma16(brow[i] + kk, lb + 1024u * i);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  const int fr = lane & 15;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int p = 4 * m + (lane >> 4);
    u32x4 af = *reinterpret_cast<const u32x4*>(scratch + fr * 128 + ((p ^ fr) * 8));
    const u32x4 bf = *reinterpret_cast<const u32x4*>(scratch + 16 * 128 + fr * 128 + ((p ^ fr) * 8));
    if (k0 + 8 * p >= kend) af = u32x4{0u, 0u, 0u, 0u};
    acc = mfma16x16x32(af, bf, acc);
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // fragments read before the next copy
  return acc;
}

// Selection + weights for the token whose logits are `row` (LDS). All kQ lanes of the token's
// DPP row call this with the same arguments and get the same ids/weights. `sbias` is LDS or NULL.
// L >= ceil(E / kQ) bounds the experts per lane; every lane reads its L entries unconditionally
// (clamped index) so the reads issue together, and a validity mask keeps the clamped copies out.
// A NaN score is ranked as -inf so that every slot names a valid expert (k <= E).
template <int L>
__device__ void select_and_weigh(const float* row, const float* sbias, int E, int k, int scoring,
                                 int q, int* ids, float* w) {
  float lg[L], sc[L];
#pragma unroll
  for (int i = 0; i < L; ++i) lg[i] = row[min(q + kQ * i, E - 1)];
  if (sbias) {
#pragma unroll
    for (int i = 0; i < L; ++i) sc[i] = sbias[min(q + kQ * i, E - 1)];
#pragma unroll
    for (int i = 0; i < L; ++i) sc[i] = __fadd_rn(lg[i], sc[i]);
  } else {
#pragma unroll
    for (int i = 0; i < L; ++i) sc[i] = lg[i];
  }
  uint32_t avail = 0;  // bit i: expert q + kQ*i exists and is not chosen yet
#pragma unroll
  for (int i = 0; i < L; ++i) {
    const bool ok = q + kQ * i < E;
    if (sc[i] != sc[i]) sc[i] = -INFINITY;
    lg[i] = ok ? lg[i] : -INFINITY;
    avail |= (ok ? 1u : 0u) << i;
  }
  float lw[kMaxK];  // raw logit of each chosen expert
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    lw[j] = 0.f;
    if (j < k) {
      float bs = -INFINITY, bl = 0.f;
      int be = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < L; ++i) {
        const int e = q + kQ * i;
        const bool take = ((avail >> i) & 1u) && ahead(sc[i], e, bs, be);
        bs = take ? sc[i] : bs;
        be = take ? e : be;
        bl = take ? lg[i] : bl;
      }
      row_argmax(bs, be, bl);
      ids[j] = be;
      lw[j] = bl;
      if (be < E && (be % kQ) == q) avail &= ~(1u << (be / kQ));
    }
  }
  if (scoring == kSoftmax) {
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < L; ++i) m = fmaxf(m, lg[i]);
    m = row_max(m);
    float z = 0.f;
#pragma unroll
    for (int i = 0; i < L; ++i) z += (q + kQ * i < E) ? expf(lg[i] - m) : 0.f;
    z = row_sum(z);
#pragma unroll
    for (int j = 0; j < kMaxK; ++j)
      if (j < k) w[j] = expf(lw[j] - m) / z;
  } else if (scoring == kSigmoid) {
#pragma unroll
    for (int j = 0; j < kMaxK; ++j)
      if (j < k) w[j] = 1.f / (1.f + expf(-lw[j]));
  } else {
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j)
      if (j < k) m = fmaxf(m, lw[j]);
    float z = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (j < k) {
        w[j] = expf(lw[j] - m);
        z += w[j];
      }
    }
#pragma unroll
    for (int j = 0; j < kMaxK; ++j)
      if (j < k) w[j] = w[j] / z;
  }
}

// Selection on the LDS logit tile of the block's 16 tokens, then the outputs. Called by every
// thread of the block (barriers inside); threads >= 256 only help with the epilogue loops.
template <int L>
__device__ void route_tail(const float* tile, int ld, const float* sbias, int t0, int T, int E,
                           int k, int scoring, const RouteOut& o, int* hist) {
  const int tl = threadIdx.x / kQ;
  const int q = threadIdx.x % kQ;
  const int t = t0 + tl;
  if (threadIdx.x < kTailThreads) {  // whole waves
    int ids[kMaxK];
    float w[kMaxK];
    select_and_weigh<L>(tile + tl * ld, sbias, E, k, scoring, q, ids, w);
    if (t < T && q == 0) {
#pragma unroll
      for (int j = 0; j < kMaxK; ++j) {
        if (j < k) {
          o.ids[static_cast<long long>(t) * k + j] = ids[j];
          o.w[static_cast<long long>(t) * k + j] = w[j];
          if (o.counts) atomicAdd(&hist[ids[j]], 1);
        }
      }
    }
  }
  __syncthreads();
  if (o.counts) {
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
      if (gridDim.x == 1) o.counts[e] = hist[e];
      else if (hist[e]) atomicAdd(&o.counts[e], hist[e]);
    }
  }
  if (o.zero_y) {
    const int rows = min(kTokTile, T - t0);
    const int vec = o.d / 4;
    float4* base = reinterpret_cast<float4*>(o.zero_y + static_cast<long long>(t0) * o.d);
    for (int i = threadIdx.x; i < rows * vec; i += blockDim.x) base[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

template <int L>
__global__ __launch_bounds__(kTailThreads) void route_from_logits_kernel(
    const float* __restrict__ logits, const float* __restrict__ sel_bias, int T, int E, int k,
    int scoring, RouteOut o) {
  extern __shared__ float smem[];
  const int ld = E + 1;
  float* tile = smem;                              // [16][E+1]
  float* sbias = tile + kTokTile * ld;             // [E]
  int* hist = reinterpret_cast<int*>(sbias + E);   // [E]
  const int t0 = blockIdx.x * kTokTile;
  for (int i = threadIdx.x; i < kTokTile * E; i += blockDim.x) {
    const int tl = i / E, e = i % E;
    const int t = t0 + tl;
    tile[tl * ld + e] = t < T ? logits[static_cast<long long>(t) * E + e] : 0.f;
  }
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    if (sel_bias) sbias[e] = sel_bias[e];
    hist[e] = 0;
  }
  __syncthreads();
  route_tail<L>(tile, ld, sel_bias ? sbias : nullptr, t0, T, E, k, scoring, o, hist);
}

// How the waves of the fused kernel split the logit tile: `neb` 16-expert column blocks, each
// reduced over `ksplit` slices of d (a power of two, neb * ksplit <= kFusedWaves when
// neb < kFusedWaves; every slice a whole number of 8-element loads).
__host__ __device__ inline int route_ksplit(int E, int d) {
  const int neb = (E + 15) / 16;
  if (neb >= kFusedWaves) return 1;
  int ks = 1;
  while (ks * 2 * neb <= kFusedWaves && d % (16 * ks) == 0) ks *= 2;
  return ks;
}

template <int L>
__global__ __launch_bounds__(kFusedThreads) void route_fused_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, const float* __restrict__ rb,
    const float* __restrict__ sel_bias, int T, int d, int E, int k, int scoring,
    float* __restrict__ logits_out, RouteOut o) {
  extern __shared__ float smem[];
  const int ld = E + 1;
  const int neb = (E + 15) / 16;
  const int ksplit = route_ksplit(E, d);
  float* part = smem;                                  // [ksplit][16][E+1]; part[0] = tile
  float* sbias = part + ksplit * kTokTile * ld;        // [E]
  float* srb = sbias + E;                              // [E]
  int* hist = reinterpret_cast<int*>(srb + E);         // [E]
  const int t0 = blockIdx.x * kTokTile;
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int r16 = lane & 15;
  const int kslice = d / ksplit;  // a multiple of 8 (d % 64 == 0, ksplit <= 8)
  // per-wave product scratch after the tables, 16-byte aligned
  uint16_t* scratch =
      reinterpret_cast<uint16_t*>((reinterpret_cast<uintptr_t>(hist + E) + 15) & ~uintptr_t{15}) +
      wave * kProdScratch;
  // the token rows this lane copies (rows past T copy row T - 1; their logits are not used)
  const uint16_t* xr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    xr[i] = x + static_cast<long long>(min(t0 + 4 * i + (lane >> 4), T - 1)) * d;

  // the per-expert vectors are loaded now and stored to LDS after the products, so their latency
  // hides behind the tile loads
  const int ex = threadIdx.x;
  const float sb_v = (sel_bias && ex < E) ? sel_bias[ex] : 0.f;
  const float rb_v = (rb && ex < E) ? rb[ex] : 0.f;

  for (int task = wave; task < neb * ksplit; task += kFusedWaves) {
    const int eb = task % neb;
    const int ks = task / neb;
    const int kbeg = ks * kslice;
    const int kend = kbeg + kslice;
    const uint16_t* wrw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      wrw[i] = wr + static_cast<long long>(min(eb * 16 + 4 * i + (lane >> 4), E - 1)) * d;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int k0 = kbeg; k0 < kend; k0 += 128)
      acc = router_product_128(xr, wrw, k0, kend, scratch, acc);
    const int e = eb * 16 + r16;
    if (e < E) {
      float* dst = part + ks * kTokTile * ld;
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[((lane >> 4) * 4 + r) * ld + e] = acc[r];
    }
  }
  if (ex < E) {
    sbias[ex] = sb_v;
    srb[ex] = rb_v;
    hist[ex] = 0;
  }
  __syncthreads();
  // fixed-order sum of the d slices, then the router bias (one more fp32 rounding)
  for (int i = threadIdx.x; i < kTokTile * E; i += blockDim.x) {
    const int tl = i / E, e = i % E;
    float v = part[tl * ld + e];
    for (int ks = 1; ks < ksplit; ++ks) v += part[(ks * kTokTile + tl) * ld + e];
    if (rb) v = v + srb[e];
    part[tl * ld + e] = v;
  }
  __syncthreads();
  if (logits_out) {
    for (int i = threadIdx.x; i < kTokTile * E; i += blockDim.x) {
      const int tl = i / E, e = i % E;
      if (t0 + tl < T) logits_out[static_cast<long long>(t0 + tl) * E + e] = part[tl * ld + e];
    }
  }
  if (o.ids == nullptr) return;  // logits only (uniform across the block)
  route_tail<L>(part, ld, sel_bias ? sbias : nullptr, t0, T, E, k, scoring, o, hist);
}

// ---------------------------------------------------------------- split router (small T)
// With few tokens the fused kernel runs on only T/16 CUs, each pulling all router weights. The
// split router spreads the logit tile instead: kernel A, one wave per (16 tokens, 16 experts,
// d-slice), writes partial 16 x 16 tiles (each wave issues all its loads at once); kernel B, one
// block per 16 tokens, adds the slices in slice order, adds the router bias and selects.

__global__ __launch_bounds__(kWave) void logit_partial_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, int T, int d, int E,
    int slice, float* __restrict__ part) {
  const int t0 = blockIdx.x * kTokTile, e0 = blockIdx.y * 16, ks = blockIdx.z;
  const int kbeg = ks * slice, kend = min(d, kbeg + slice);
  __shared__ __attribute__((aligned(16))) uint16_t scratch[kProdScratch];
  const int lane = lane_id();
  const int r16 = lane & 15;
  // rows past T or E read a valid row; their products are never stored
  const uint16_t* xr[4];
  const uint16_t* wrw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * i + (lane >> 4);
    xr[i] = x + static_cast<long long>(min(t0 + r, T - 1)) * d;
    wrw[i] = wr + static_cast<long long>(min(e0 + r, E - 1)) * d;
  }
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k0 = kbeg; k0 < kend; k0 += 128)
    acc = router_product_128(xr, wrw, k0, kend, scratch, acc);
  const int e = e0 + r16;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = t0 + (lane >> 4) * 4 + r;
    if (t < T && e < E) part[(static_cast<long long>(ks) * T + t) * E + e] = acc[r];
  }
}

constexpr int kPartThreads = 1024;
constexpr int kMaxSlices = 16;

template <int L>
__global__ __launch_bounds__(kPartThreads) void route_from_partials_kernel(
    const float* __restrict__ part, int nks, const float* __restrict__ rb,
    const float* __restrict__ sel_bias, int T, int E, int k, int scoring,
    float* __restrict__ logits_out, RouteOut o) {
  extern __shared__ float smem[];
  const int ld = E + 1;
  float* tile = smem;                              // [16][E+1]
  float* sbias = tile + kTokTile * ld;             // [E]
  int* hist = reinterpret_cast<int*>(sbias + E);   // [E]
  const int t0 = blockIdx.x * kTokTile;
  for (int i = threadIdx.x; i < kTokTile * E; i += blockDim.x) {
    const int tl = i / E, e = i % E;
    const int t = min(t0 + tl, T - 1);
    // every slice's partial is loaded before the sum (fixed order: slice 0, 1, ..., then the
    // router bias, one more fp32 rounding)
    float p[kMaxSlices];
#pragma unroll
    for (int ks = 0; ks < kMaxSlices; ++ks)
      p[ks] = ks < nks ? part[(static_cast<long long>(ks) * T + t) * E + e] : 0.f;
    float v = p[0];
#pragma unroll
    for (int ks = 1; ks < kMaxSlices; ++ks)
      if (ks < nks) v += p[ks];
    if (rb) v = v + rb[e];
    if (t0 + tl < T) {
      if (logits_out) logits_out[static_cast<long long>(t) * E + e] = v;
    } else {
      v = 0.f;
    }
    tile[tl * ld + e] = v;
  }
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    if (sel_bias) sbias[e] = sel_bias[e];
    hist[e] = 0;
  }
  __syncthreads();
  route_tail<L>(tile, ld, sel_bias ? sbias : nullptr, t0, T, E, k, scoring, o, hist);
}

// fp32 router logits: one thread per (token, expert), four interleaved partial sums.
__global__ void logits_f32_kernel(const float* __restrict__ x, const float* __restrict__ wr,
                                  const float* __restrict__ rb, int T, int d, int E,
                                  float* __restrict__ logits) {
  const long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<long long>(T) * E) return;
  const int t = static_cast<int>(i / E), e = static_cast<int>(i % E);
  const float4* xr = reinterpret_cast<const float4*>(x + static_cast<long long>(t) * d);
  const float4* wrow = reinterpret_cast<const float4*>(wr + static_cast<long long>(e) * d);
  float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
  for (int c = 0; c < d / 4; ++c) {
    const float4 a = xr[c], b = wrow[c];
    s0 = fmaf(a.x, b.x, s0);
    s1 = fmaf(a.y, b.y, s1);
    s2 = fmaf(a.z, b.z, s2);
    s3 = fmaf(a.w, b.w, s3);
  }
  float s = (s0 + s1) + (s2 + s3);
  if (rb) s = s + rb[e];
  logits[i] = s;
}

// Experts per selection lane, rounded up to a power of two (the template bound of the selection).
int lane_experts(int E) {
  const int need = (E + kQ - 1) / kQ;
  int L = 1;
  while (L < need) L *= 2;
  return L;
}

#define MOE_ROUTE_DISPATCH_L(E, LAUNCH) \
  switch (lane_experts(E)) {            \
    case 1: LAUNCH(1); break;           \
    case 2: LAUNCH(2); break;           \
    case 4: LAUNCH(4); break;           \
    case 8: LAUNCH(8); break;           \
    default: LAUNCH(16); break;         \
  }

size_t tail_smem(int E) {
  return sizeof(float) * (static_cast<size_t>(kTokTile) * (E + 1) + E) +
         sizeof(int) * E;
}

size_t fused_smem(int E, int d) {
  return sizeof(float) * (static_cast<size_t>(route_ksplit(E, d)) * kTokTile * (E + 1) + 2 * E) +
         sizeof(int) * E + 16 + sizeof(uint16_t) * kFusedWaves * kProdScratch;
}

}  // namespace

hipError_t launch_zero_i32(int32_t* p, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  zero_i32_kernel<<<(n + 255) / 256, 256, 0, s>>>(p, n);
  return hipGetLastError();
}

hipError_t launch_zero_f32(float* p, long long n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const long long nthreads = (n + 3) / 4;
  zero_f32_kernel<<<static_cast<unsigned>((nthreads + 255) / 256), 256, 0, s>>>(p, n);
  return hipGetLastError();
}

hipError_t launch_logits_f32(const float* x, const float* wr, const float* rb, int T, int d,
                             int E, float* logits, hipStream_t s) {
  const long long n = static_cast<long long>(T) * E;
  logits_f32_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, s>>>(x, wr, rb, T, d, E,
                                                                          logits);
  return hipGetLastError();
}

hipError_t launch_route_from_logits(const float* logits, const float* sel_bias, int T, int E,
                                    int k, int scoring, const RouteOut& o, hipStream_t s) {
  const int blocks = (T + kTokTile - 1) / kTokTile;
  if (o.counts && blocks > 1) {
    hipError_t err = launch_zero_i32(o.counts, E, s);
    if (err != hipSuccess) return err;
  }
#define MOE_LAUNCH_TAIL(L)                                                                  \
  route_from_logits_kernel<L><<<blocks, kTailThreads, tail_smem(E), s>>>(logits, sel_bias, T, E, \
                                                                         k, scoring, o)
  MOE_ROUTE_DISPATCH_L(E, MOE_LAUNCH_TAIL)
#undef MOE_LAUNCH_TAIL
  return hipGetLastError();
}

hipError_t launch_route_fused_bf16(const uint16_t* x, const uint16_t* wr, const float* rb,
                                   const float* sel_bias, int T, int d, int E, int k, int scoring,
                                   float* logits_out, const RouteOut& o, hipStream_t s) {
  const int blocks = (T + kTokTile - 1) / kTokTile;
  if (o.counts && blocks > 1) {
    hipError_t err = launch_zero_i32(o.counts, E, s);
    if (err != hipSuccess) return err;
  }
#define MOE_LAUNCH_FUSED(L)                                                                \
  route_fused_bf16_kernel<L><<<blocks, kFusedThreads, fused_smem(E, d), s>>>(              \
      x, wr, rb, sel_bias, T, d, E, k, scoring, logits_out, o)
  MOE_ROUTE_DISPATCH_L(E, MOE_LAUNCH_FUSED)
#undef MOE_LAUNCH_FUSED
  return hipGetLastError();
}

int route_split_slice(int d) {
  // 256-wide slices (8 MFMA steps, one batch of loads per lane), wider for d > 4096 so that at
  // most 16 slices exist; always a multiple of 64
  int slice = 256;
  while ((d + slice - 1) / slice > kMaxSlices) slice += 64;
  return slice;
}

int route_split_ks(int T, int d, int E) {
  // worth a second launch only when every fused block would pull a large router matrix
  // (>= 128 KB of bf16: 64 experts x 1024 measured 9.4 us split against 11.7 us fused, and with
  // the fused kernel's whole-line copies still 39.8 against 40.2 us per graph-replayed ZONOS3-Mini
  // decode step; 16 x 2048 measured 8.7 us split against 7.4 us fused)
  if (T > kRouteSplitMaxT || static_cast<long long>(E) * d < 65536) return 0;
  const int slice = route_split_slice(d);
  return (d + slice - 1) / slice;
}

hipError_t launch_route_split_bf16(const uint16_t* x, const uint16_t* wr, const float* rb,
                                   const float* sel_bias, int T, int d, int E, int k, int scoring,
                                   float* logits_out, float* part, const RouteOut& o,
                                   hipStream_t s) {
  const int blocks = (T + kTokTile - 1) / kTokTile;
  if (o.counts && blocks > 1) {
    hipError_t err = launch_zero_i32(o.counts, E, s);
    if (err != hipSuccess) return err;
  }
  const int slice = route_split_slice(d);
  const int nks = (d + slice - 1) / slice;
  logit_partial_kernel<<<dim3(blocks, (E + 15) / 16, nks), kWave, 0, s>>>(x, wr, T, d, E, slice,
                                                                           part);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
#define MOE_LAUNCH_PART(L)                                                                    \
  route_from_partials_kernel<L><<<blocks, kPartThreads, tail_smem(E), s>>>(                   \
      part, nks, rb, sel_bias, T, E, k, scoring, logits_out, o)
  MOE_ROUTE_DISPATCH_L(E, MOE_LAUNCH_PART)
#undef MOE_LAUNCH_PART
  return hipGetLastError();
}

hipError_t launch_logits_bf16(const uint16_t* x, const uint16_t* wr, const float* rb, int T,
                              int d, int E, float* logits, hipStream_t s) {
  RouteOut none{};
  return launch_route_fused_bf16(x, wr, rb, nullptr, T, d, E, 1, kSoftmax, logits, none, s);
}

}  // namespace moe
