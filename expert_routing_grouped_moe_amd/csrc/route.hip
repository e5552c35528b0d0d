// Router logits, top-k selection and routing weights (steps 1-3 of the MoE layer).
//
// Scoring modes (zonos2.cpp INTERNALS, "Model architecture" table, Router row; audio.cpp PR #1271,
// "Framework change"):
//   SOFTMAX           rank by logit, weight = softmax over all E logits at the chosen expert
//                     (no renormalisation over the chosen set)
//   SELECTED_SOFTMAX  rank by fp32(logit + sel_bias), weight = softmax over the k chosen raw
//                     logits
// Selection order is (score descending, expert index ascending); -0.0 == +0.0 under the IEEE
// comparison, so signed zeros fall through to the index.
//
// Work layout: a block owns 16 tokens. Selection runs on 256 threads, 16 lanes per token, each
// lane scanning every 16th expert; the per-token best is found with xor-shuffles inside the
// 16-lane group. The bf16 routing kernel first computes the 16 x E logit tile on the matrix cores
// with 8 waves that split the experts (16 per MFMA tile) and, when there are few experts, the
// d-long reduction; each wave issues the loads of 8 MFMA steps before using them. Partial tiles
// are added in a fixed order, so the logits are the same on every call.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kQ = 16;                      // lanes per token in the selection
constexpr int kTailThreads = kTokTile * kQ; // 256
constexpr int kFusedWaves = 8;
constexpr int kFusedThreads = kFusedWaves * kWave;
constexpr int kBatch = 8;                   // MFMA steps whose loads are issued together

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

// Selection + weights for the token whose logits are `row` (LDS). All kQ lanes of the token's
// group call this with the same arguments and get the same ids/weights. `sbias` is LDS or NULL.
// A NaN score is ranked as -inf so that every slot names a valid expert.
__device__ void select_and_weigh(const float* row, const float* sbias, int E, int k, int scoring,
                                 int q, int* ids, float* w) {
  uint32_t taken = 0;  // bit i: expert q + kQ*i already chosen
  const int nloc = (E - q + kQ - 1) / kQ;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (j < k) {
      float bs = -INFINITY;
      int be = 0x7fffffff;
      for (int i = 0; i < nloc; ++i) {
        if ((taken >> i) & 1u) continue;
        const int e = q + kQ * i;
        float s = row[e];
        if (sbias) s = __fadd_rn(s, sbias[e]);
        if (s != s) s = -INFINITY;
        if (ahead(s, e, bs, be)) { bs = s; be = e; }
      }
#pragma unroll
      for (int m = 1; m < kQ; m <<= 1) {
        const float os = __shfl_xor(bs, m);
        const int oe = __shfl_xor(be, m);
        if (ahead(os, oe, bs, be)) { bs = os; be = oe; }
      }
      ids[j] = be;
      if ((be % kQ) == q) taken |= 1u << (be / kQ);
    }
  }
  if (scoring == kSoftmax) {
    float m = -INFINITY;
    for (int i = 0; i < nloc; ++i) m = fmaxf(m, row[q + kQ * i]);
#pragma unroll
    for (int o = 1; o < kQ; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
    float z = 0.f;
    for (int i = 0; i < nloc; ++i) z += expf(row[q + kQ * i] - m);
#pragma unroll
    for (int o = 1; o < kQ; o <<= 1) z += __shfl_xor(z, o);
#pragma unroll
    for (int j = 0; j < kMaxK; ++j)
      if (j < k) w[j] = expf(row[ids[j]] - m) / z;
  } else {
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j)
      if (j < k) m = fmaxf(m, row[ids[j]]);
    float z = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (j < k) {
        w[j] = expf(row[ids[j]] - m);
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
__device__ void route_tail(const float* tile, int ld, const float* sbias, int t0, int T, int E,
                           int k, int scoring, const RouteOut& o, int* hist) {
  const int tl = threadIdx.x / kQ;
  const int q = threadIdx.x % kQ;
  const int t = t0 + tl;
  if (threadIdx.x < kTailThreads) {  // whole waves
    int ids[kMaxK];
    float w[kMaxK];
    select_and_weigh(tile + tl * ld, sbias, E, k, scoring, q, ids, w);
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
  route_tail(tile, ld, sel_bias ? sbias : nullptr, t0, T, E, k, scoring, o, hist);
}

// How the 8 waves of the fused kernel split the logit tile: `neb` 16-expert column blocks, each
// reduced over `ksplit` slices of d (a power of two, neb * ksplit <= 8 when neb < 8).
__host__ __device__ inline int route_ksplit(int E) {
  const int neb = (E + 15) / 16;
  if (neb >= kFusedWaves) return 1;
  int ks = 1;
  while (ks * 2 * neb <= kFusedWaves) ks *= 2;
  return ks;
}

__global__ __launch_bounds__(kFusedThreads) void route_fused_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, const float* __restrict__ rb,
    const float* __restrict__ sel_bias, int T, int d, int E, int k, int scoring,
    float* __restrict__ logits_out, RouteOut o) {
  extern __shared__ float smem[];
  const int ld = E + 1;
  const int neb = (E + 15) / 16;
  const int ksplit = route_ksplit(E);
  float* part = smem;                                  // [ksplit][16][E+1]; part[0] = tile
  float* sbias = part + ksplit * kTokTile * ld;        // [E]
  int* hist = reinterpret_cast<int*>(sbias + E);       // [E]
  const int t0 = blockIdx.x * kTokTile;
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int r16 = lane & 15;
  const int kq = (lane >> 4) * 8;
  const int t = t0 + r16;
  const bool tok_ok = t < T;
  const uint16_t* xrow = x + static_cast<long long>(min(t, T - 1)) * d;
  const int kslice = d / ksplit;  // a multiple of 8 (d % 64 == 0, ksplit <= 8)

  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    if (sel_bias) sbias[e] = sel_bias[e];
    hist[e] = 0;
  }

  for (int task = wave; task < neb * ksplit; task += kFusedWaves) {
    const int eb = task % neb;
    const int ks = task / neb;
    const int kbeg = ks * kslice;
    const int kend = kbeg + kslice;
    const int e = eb * 16 + r16;
    const bool e_ok = e < E;
    const uint16_t* wrow = wr + static_cast<long long>(min(e, E - 1)) * d;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int k0 = kbeg; k0 < kend; k0 += 32 * kBatch) {
      u32x4 a[kBatch], b[kBatch];
#pragma unroll
      for (int s = 0; s < kBatch; ++s) {
        const int kk = k0 + 32 * s + kq;  // kend - kk is a multiple of 8: kk < kend -> 8 in range
        const bool ok = kk < kend;
        a[s] = (ok && tok_ok) ? load16(xrow + kk) : u32x4{0u, 0u, 0u, 0u};
        b[s] = (ok && e_ok) ? load16(wrow + kk) : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int s = 0; s < kBatch; ++s) acc = mfma16x16x32(a[s], b[s], acc);
    }
    if (e_ok) {
      float* dst = part + ks * kTokTile * ld;
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[((lane >> 4) * 4 + r) * ld + e] = acc[r];
    }
  }
  __syncthreads();
  // fixed-order sum of the d slices, then the router bias (one more fp32 rounding)
  for (int i = threadIdx.x; i < kTokTile * E; i += blockDim.x) {
    const int tl = i / E, e = i % E;
    float v = part[tl * ld + e];
    for (int ks = 1; ks < ksplit; ++ks) v += part[(ks * kTokTile + tl) * ld + e];
    if (rb) v = v + rb[e];
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
  route_tail(part, ld, sel_bias ? sbias : nullptr, t0, T, E, k, scoring, o, hist);
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

size_t tail_smem(int E) {
  return sizeof(float) * (static_cast<size_t>(kTokTile) * (E + 1) + E) +
         sizeof(int) * E;
}

size_t fused_smem(int E) {
  return sizeof(float) * (static_cast<size_t>(route_ksplit(E)) * kTokTile * (E + 1) + E) +
         sizeof(int) * E;
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
  route_from_logits_kernel<<<blocks, kTailThreads, tail_smem(E), s>>>(logits, sel_bias, T, E, k,
                                                                      scoring, o);
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
  route_fused_bf16_kernel<<<blocks, kFusedThreads, fused_smem(E), s>>>(x, wr, rb, sel_bias, T, d,
                                                                       E, k, scoring, logits_out,
                                                                       o);
  return hipGetLastError();
}

hipError_t launch_logits_bf16(const uint16_t* x, const uint16_t* wr, const float* rb, int T,
                              int d, int E, float* logits, hipStream_t s) {
  RouteOut none{};
  return launch_route_fused_bf16(x, wr, rb, nullptr, T, d, E, 1, kSoftmax, logits, none, s);
}

}  // namespace moe
