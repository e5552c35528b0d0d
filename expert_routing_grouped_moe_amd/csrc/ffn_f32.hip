// fp32 expert FFN (steps 5-6) for layers kept in full precision: plain fp32 FMA, no reduced
// precision anywhere. SwiGLU as in audio.cpp PR #1271, "Summary", over the gate/up/down expert
// stacks of zonos2.cpp INTERNALS, "Recommended: F16 spine + K-quant experts".
//
// Tiles: 16 grouped rows x 64 output features per block of 256 threads, K staged through LDS in
// chunks of 32. Thread (row = tid / 16, c = tid % 16) owns features c, c+16, c+32, c+48.
#include "common.hpp"
#include "down_epilogue.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kBM = 16;
constexpr int kBN = 64;
constexpr int kBK = 32;

template <bool GATEUP>
__global__ __launch_bounds__(256) void ffn_f32_kernel(
    const float* __restrict__ a_src,   // x [T, d] (gate/up) or h [T*k, H] (down)
    const float* __restrict__ w0,      // w_gate [E, H, d] or w_down [E, d, H]
    const float* __restrict__ w1,      // w_up [E, H, d] (gate/up only)
    int K, int N, int E, int k, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_rows, float* __restrict__ h_out, DownArgs down) {
  __shared__ int sh_tiles[2 * (kMaxE + 1)];
  __shared__ float As[kBM][kBK + 1];
  __shared__ float B0[kBN][kBK + 1];
  __shared__ float B1[GATEUP ? kBN : 1][kBK + 1];
  const TileInfo ti = find_tile(offsets, E, kBM, blockIdx.y, sh_tiles);
  if (ti.e < 0) return;
  const int n0 = blockIdx.x * kBN;
  const int tid = threadIdx.x;
  const int row = tid / 16;
  const int c = tid % 16;

  // source row of A for each of the 16 tile rows (loaded by threads 0..15 of each pass)
  const float* w0e = w0 + static_cast<long long>(ti.e) * N * K;
  const float* w1e = GATEUP ? w1 + static_cast<long long>(ti.e) * N * K : nullptr;

  float acc0[4] = {0.f, 0.f, 0.f, 0.f};
  float acc1[4] = {0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < K; k0 += kBK) {
    for (int i = tid; i < kBM * kBK; i += 256) {
      const int r = i / kBK, kk = i % kBK;
      float v = 0.f;
      if (r < ti.rows && k0 + kk < K) {
        const int p = ti.row0 + r;
        const long long src = GATEUP ? static_cast<long long>(sorted_rows[p] / k) : p;
        v = a_src[src * K + k0 + kk];
      }
      As[r][kk] = v;
    }
    for (int i = tid; i < kBN * kBK; i += 256) {
      const int r = i / kBK, kk = i % kBK;
      const bool ok = (n0 + r < N) && (k0 + kk < K);
      B0[r][kk] = ok ? w0e[static_cast<long long>(n0 + r) * K + k0 + kk] : 0.f;
      if constexpr (GATEUP) B1[r][kk] = ok ? w1e[static_cast<long long>(n0 + r) * K + k0 + kk] : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < kBK; ++kk) {
      const float a = As[row][kk];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc0[i] = fmaf(a, B0[c + 16 * i][kk], acc0[i]);
        if constexpr (GATEUP) acc1[i] = fmaf(a, B1[c + 16 * i][kk], acc1[i]);
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
                          hipStream_t s, void* mid_event) {
  const int rows = T * k;
  const int tiles = max_tiles(rows, E, kBM);
  if (tiles == 0) return hipSuccess;
  DownArgs none{};
  dim3 g1((H + kBN - 1) / kBN, tiles);
  ffn_f32_kernel<true><<<g1, 256, 0, s>>>(x, wg, wu, d, H, E, k, offsets, sorted_rows, h, none);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (mid_event) {
    err = record_stage_event(mid_event, s);
    if (err != hipSuccess) return err;
  }
  dim3 g2((d + kBN - 1) / kBN, tiles);
  ffn_f32_kernel<false><<<g2, 256, 0, s>>>(h, wd, nullptr, H, d, E, k, offsets, sorted_rows,
                                           nullptr, down);
  return hipGetLastError();
}

}  // namespace moe
