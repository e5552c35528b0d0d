// fp32 expert FFN (steps 5-6) for layers kept in full precision: plain fp32 FMA, no reduced
// precision anywhere. SwiGLU as in audio.cpp PR #1271, "Summary", over the gate/up/down expert
// stacks of zonos2.cpp INTERNALS, "Recommended: F16 spine + K-quant experts".
//
// Tiles: 16 grouped rows x 64 output features per block of 256 threads (a 1-D grid, feature
// tile fastest: block b covers row tile b / ntn and feature tile b % ntn), K staged through LDS in
// chunks of 64 (float4 copies, all of a chunk's loads issued together, the next chunk loading
// while the current one is used). Thread (row = tid / 16, c = tid % 16) owns features c, c+16,
// c+32, c+48.
#include "common.hpp"
#include "down_epilogue.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kBM = 16;
constexpr int kBN = 64;
constexpr int kBK = 64;
constexpr int kLd = kBK + 4;  // pitch in floats; keeps rows 16-byte aligned

__device__ __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }

template <bool GATEUP>
__global__ __launch_bounds__(256) void ffn_f32_kernel(
    const float* __restrict__ a_src,   // x [T, d] (gate/up) or h [T*k, H] (down)
    const float* __restrict__ w0,      // w_gate [E, H, d] or w_down [E, d, H]
    const float* __restrict__ w1,      // w_up [E, H, d] (gate/up only)
    int K, int N, int E, int k, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_rows, float* __restrict__ h_out, DownArgs down) {
  __shared__ int sh_tiles[2 * (kMaxE + 1)];
  __shared__ __attribute__((aligned(16))) float As[kBM * kLd];
  __shared__ __attribute__((aligned(16))) float B0[kBN * kLd];
  __shared__ __attribute__((aligned(16))) float B1[(GATEUP ? kBN : 1) * kLd];
  const int ntn = (N + kBN - 1) / kBN;
  const TileInfo ti = find_tile(offsets, E, kBM, static_cast<int>(blockIdx.x / ntn), sh_tiles);
  if (ti.e < 0) return;
  const int n0 = static_cast<int>(blockIdx.x % ntn) * kBN;
  const int tid = threadIdx.x;
  const int row = tid / 16;
  const int c = tid % 16;

  // copy assignment: A row tid / 16, float4 column tid % 16; B rows tid / 16 + 16 i
  const long long wbase = static_cast<long long>(ti.e) * N * K;
  const float* arow = nullptr;
  if (row < ti.rows) {
    const int p = ti.row0 + row;
    const long long src = GATEUP ? static_cast<long long>(sorted_rows[p] / k) : p;
    arow = a_src + src * K;
  }
  const float* brow0[4];
  const float* brow1[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int n = n0 + row + 16 * i;
    brow0[i] = n < N ? w0 + wbase + static_cast<long long>(n) * K : nullptr;
    brow1[i] = (GATEUP && n < N) ? w1 + wbase + static_cast<long long>(n) * K : nullptr;
  }
  const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
  float4 ra, rb0[4], rb1[4];
  auto load = [&](int k0) {
    const int kk = k0 + c * 4;  // K % 4 == 0: a float4 is either whole or past the end
    const bool ok = kk < K;
    ra = (arow && ok) ? ld4(arow + kk) : z4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      rb0[i] = (brow0[i] && ok) ? ld4(brow0[i] + kk) : z4;
      if constexpr (GATEUP) rb1[i] = (brow1[i] && ok) ? ld4(brow1[i] + kk) : z4;
    }
  };

  float acc0[4] = {0.f, 0.f, 0.f, 0.f};
  float acc1[4] = {0.f, 0.f, 0.f, 0.f};
  load(0);
  for (int k0 = 0; k0 < K; k0 += kBK) {
    *reinterpret_cast<float4*>(&As[row * kLd + c * 4]) = ra;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<float4*>(&B0[(row + 16 * i) * kLd + c * 4]) = rb0[i];
      if constexpr (GATEUP) *reinterpret_cast<float4*>(&B1[(row + 16 * i) * kLd + c * 4]) = rb1[i];
    }
    __syncthreads();
    if (k0 + kBK < K) load(k0 + kBK);  // next chunk in flight during the products
#pragma unroll 16
    for (int kk = 0; kk < kBK; ++kk) {
      const float a = As[row * kLd + kk];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc0[i] = fmaf(a, B0[(c + 16 * i) * kLd + kk], acc0[i]);
        if constexpr (GATEUP) acc1[i] = fmaf(a, B1[(c + 16 * i) * kLd + kk], acc1[i]);
      }
    }
    __syncthreads();
  }
  if (row >= ti.rows) return;
  const int p = ti.row0 + row;
  if constexpr (GATEUP) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int n = n0 + c + 16 * i;
      if (n < N) h_out[static_cast<long long>(p) * N + n] = silu_precise(acc0[i]) * acc1[i];
    }
  } else {
    const DownRow dr = down_row(down, sorted_rows[p], p, N);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int n = n0 + c + 16 * i;
      if (n < N) down_put(down, dr, n, acc0[i]);
    }
  }
}

}  // namespace

hipError_t launch_ffn_f32(const float* x, const float* wg, const float* wu, const float* wd,
                          int T, int d, int E, int H, int k, const int32_t* offsets,
                          const int32_t* sorted_rows, float* h, const DownArgs& down,
                          hipStream_t s, const StageMarks& gu) {
  const int rows = T * k;
  const int tiles = max_tiles(rows, E, kBM);
  if (tiles == 0) return hipSuccess;
  DownArgs none{};
  // one row tile per ntn consecutive blocks; the contract's size limits (T * k * max(d, H) < 2^31,
  // T <= 2^24, widths <= 65536) keep this below 2^24 blocks, a single grid dimension
  const dim3 g1(static_cast<unsigned>(tiles) * static_cast<unsigned>((H + kBN - 1) / kBN));
  hipError_t err = launch_marked(ffn_f32_kernel<true>, g1, dim3(256), s, gu, x, wg, wu, d, H, E,
                                 k, offsets, sorted_rows, h, none);
  if (err != hipSuccess) return err;
  const dim3 g2(static_cast<unsigned>(tiles) * static_cast<unsigned>((d + kBN - 1) / kBN));
  ffn_f32_kernel<false><<<g2, 256, 0, s>>>(h, wd, nullptr, H, d, E, k, offsets, sorted_rows,
                                           nullptr, down);
  return hipGetLastError();
}

}  // namespace moe
