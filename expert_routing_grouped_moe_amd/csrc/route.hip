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
// Layout of the work: a block of 256 threads owns 16 tokens; 16 lanes per token each scan every
// 16th expert, and the per-token best is found with xor-shuffles inside the 16-lane group.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kTokTile = 16;   // tokens per block
constexpr int kQ = 16;         // lanes per token
constexpr int kRouteThreads = kTokTile * kQ;

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

// Shared tail of both routing kernels: selection on the LDS logit tile, outputs, histogram,
// optional clearing of the token rows of y.
__device__ void route_tail(const float* tile, int ld, const float* sbias, int t0, int T, int E,
                           int k, int scoring, int32_t* __restrict__ ids_out,
                           float* __restrict__ w_out, int32_t* __restrict__ counts, int* hist,
                           float* __restrict__ zero_y, int d) {
  const int tl = threadIdx.x / kQ;
  const int q = threadIdx.x % kQ;
  const int t = t0 + tl;
  int ids[kMaxK];
  float w[kMaxK];
  select_and_weigh(tile + tl * ld, sbias, E, k, scoring, q, ids, w);
  if (t < T && q == 0) {
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (j < k) {
        ids_out[static_cast<long long>(t) * k + j] = ids[j];
        w_out[static_cast<long long>(t) * k + j] = w[j];
        if (counts) atomicAdd(&hist[ids[j]], 1);
      }
    }
  }
  __syncthreads();
  if (counts) {
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
      if (gridDim.x == 1) counts[e] = hist[e];
      else if (hist[e]) atomicAdd(&counts[e], hist[e]);
    }
  }
  if (zero_y) {
    const int rows = min(kTokTile, T - t0);
    const int vec = d / 4;
    float4* base = reinterpret_cast<float4*>(zero_y + static_cast<long long>(t0) * d);
    for (int i = threadIdx.x; i < rows * vec; i += blockDim.x) base[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

__global__ __launch_bounds__(kRouteThreads) void route_from_logits_kernel(
    const float* __restrict__ logits, const float* __restrict__ sel_bias, int T, int E, int k,
    int scoring, int32_t* __restrict__ ids, float* __restrict__ w, int32_t* __restrict__ counts,
    float* __restrict__ zero_y, int d) {
  extern __shared__ float smem[];
  const int ld = E + 1;
  float* tile = smem;                      // [kTokTile][E+1]
  float* sbias = tile + kTokTile * ld;     // [E]
  int* hist = reinterpret_cast<int*>(sbias + E);  // [E]
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
  route_tail(tile, ld, sel_bias ? sbias : nullptr, t0, T, E, k, scoring, ids, w, counts, hist,
             zero_y, d);
}

// Router logits for 16 tokens on the matrix cores, then selection. The four waves split the
// d-long dot products four ways; the partial 16 x E tiles are added in wave order (fixed, so the
// logits are the same on every call).
__global__ __launch_bounds__(kRouteThreads) void route_fused_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, const float* __restrict__ rb,
    const float* __restrict__ sel_bias, int T, int d, int E, int k, int scoring,
    float* __restrict__ logits_out, int32_t* __restrict__ ids, float* __restrict__ w,
    float* __restrict__ zero_y) {
  extern __shared__ float smem[];
  const int ld = E + 1;
  float* tile = smem;                      // [16][E+1]
  float* sbias = tile + kTokTile * ld;
  int* hist = reinterpret_cast<int*>(sbias + E);
  const int t0 = blockIdx.x * kTokTile;
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int neb = (E + 15) / 16;
  const int kslice = d / 4;        // d % 128 == 0 is not required; d % 64 == 0 -> kslice % 16
  const int kbeg = wave * kslice;
  const int r16 = lane & 15;
  const int kq = (lane >> 4) * 8;

  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    if (sel_bias) sbias[e] = sel_bias[e];
    hist[e] = 0;
  }

  f32x4 acc[16];
#pragma unroll
  for (int b = 0; b < 16; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int t = t0 + r16;
  const uint16_t* xrow = x + static_cast<long long>(min(t, T - 1)) * d;
  const bool tok_ok = t < T;
  // kslice is a multiple of 16 (d % 64 == 0); MFMA steps consume 32 k. A slice whose length is
  // an odd multiple of 16 ends with a half step whose upper k lanes read zeros.
  for (int k0 = kbeg; k0 < kbeg + kslice; k0 += 32) {
    const int kk = k0 + kq;
    const bool k_ok = kk < kbeg + kslice;
    u32x4 a = u32x4{0u, 0u, 0u, 0u};
    if (tok_ok && k_ok) a = load16(xrow + kk);
#pragma unroll
    for (int b = 0; b < 16; ++b) {
      if (b < neb) {
        const int e = b * 16 + r16;
        u32x4 bv = u32x4{0u, 0u, 0u, 0u};
        if (e < E && k_ok) bv = load16(wr + static_cast<long long>(e) * d + kk);
        acc[b] = mfma16x16x32(a, bv, acc[b]);
      }
    }
  }
  // ordered reduction of the four partial tiles into LDS
  for (int src = 0; src < 4; ++src) {
    if (wave == src) {
#pragma unroll
      for (int b = 0; b < 16; ++b) {
        if (b < neb) {
          const int e = b * 16 + r16;
          if (e < E) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int row = (lane >> 4) * 4 + r;
              float* dst = tile + row * ld + e;
              *dst = (src == 0) ? acc[b][r] : (*dst + acc[b][r]);
            }
          }
        }
      }
    }
    __syncthreads();
  }
  if (rb) {
    for (int i = threadIdx.x; i < kTokTile * E; i += blockDim.x) {
      const int tl = i / E, e = i % E;
      tile[tl * ld + e] = tile[tl * ld + e] + rb[e];
    }
    __syncthreads();
  }
  if (logits_out) {
    for (int i = threadIdx.x; i < kTokTile * E; i += blockDim.x) {
      const int tl = i / E, e = i % E;
      if (t0 + tl < T) logits_out[static_cast<long long>(t0 + tl) * E + e] = tile[tl * ld + e];
    }
  }
  if (ids == nullptr) return;  // logits only
  route_tail(tile, ld, sel_bias ? sbias : nullptr, t0, T, E, k, scoring, ids, w, nullptr, hist,
             zero_y, d);
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

size_t route_smem(int E) {
  return sizeof(float) * (static_cast<size_t>(kTokTile) * (E + 1) + E) + sizeof(int) * E;
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
                                    int k, int scoring, int32_t* ids, float* w, int32_t* counts,
                                    float* zero_y, int d, hipStream_t s) {
  const int blocks = (T + kTokTile - 1) / kTokTile;
  if (counts && blocks > 1) {
    hipError_t err = launch_zero_i32(counts, E, s);
    if (err != hipSuccess) return err;
  }
  route_from_logits_kernel<<<blocks, kRouteThreads, route_smem(E), s>>>(
      logits, sel_bias, T, E, k, scoring, ids, w, counts, zero_y, d);
  return hipGetLastError();
}

hipError_t launch_route_fused_bf16(const uint16_t* x, const uint16_t* wr, const float* rb,
                                   const float* sel_bias, int T, int d, int E, int k, int scoring,
                                   float* logits_out, int32_t* ids, float* w, float* zero_y,
                                   hipStream_t s) {
  const int blocks = (T + kTokTile - 1) / kTokTile;
  route_fused_bf16_kernel<<<blocks, kRouteThreads, route_smem(E), s>>>(
      x, wr, rb, sel_bias, T, d, E, k, scoring, logits_out, ids, w, zero_y);
  return hipGetLastError();
}

hipError_t launch_logits_bf16(const uint16_t* x, const uint16_t* wr, const float* rb, int T,
                              int d, int E, float* logits, hipStream_t s) {
  return launch_route_fused_bf16(x, wr, rb, nullptr, T, d, E, 1, kSoftmax, logits, nullptr,
                                 nullptr, nullptr, s);
}

}  // namespace moe
