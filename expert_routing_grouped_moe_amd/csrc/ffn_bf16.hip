// bf16 expert FFN (steps 5-6) on the CDNA4 matrix cores, fp32 accumulation.
//   gate/up:  h[p, n] = silu(x[t] . Wg[e, n]) * (x[t] . Wu[e, n])      (SwiGLU; audio.cpp PR #1271,
//             "Summary"), t = sorted_rows[p] / k, h rounded to bf16
//   down:     o[p, n] = h[p] . Wd[e, n]  -> expert_out, or weighted into y
// Both are "NT" products: every operand row (token row, weight row) is contiguous along the
// reduction index, as the 3-D expert stacks of zonos2.cpp INTERNALS ("Recommended: F16 spine +
// K-quant experts") are stored.
//
// Two kernels, chosen on the host from the static shape (average rows per expert):
//  * decode (few rows per expert): the layer is a read of the touched experts' weights (the
//    single-stream regime of the ZONOS2-4bit MLX card, "Performance notes"). Weight rows stream
//    from HBM straight into registers, 64 contiguous bytes per lane per 128-k block, double
//    buffered; the 16 (or 32) gathered token rows sit in LDS and are reused by every wave.
//  * prefill (many rows per expert): a grouped GEMM with 128 x 128 block tiles, A (gathered rows)
//    and B (weights) staged through double-buffered LDS, 2 x 2 waves of 64 x 64 each.
#include "common.hpp"
#include "down_epilogue.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

// ------------------------------------------------------------------------------------ prefill

constexpr int kPfBM = 128;
constexpr int kPfBN = 128;          // weight rows per tile (gate/up: 64 gate + 64 up)
constexpr int kPfBK = 64;
constexpr int kPfLD = kPfBK + 8;    // LDS row pitch in bf16 (144 B: 16-lane b128 reads hit all 64 banks once)

template <bool GATEUP>
__global__ __launch_bounds__(256) void gemm_prefill_kernel(
    const uint16_t* __restrict__ A,    // x [T, d] (gate/up) or h [T*k, H] (down)
    const uint16_t* __restrict__ W0,   // w_gate [E, H, d] or w_down [E, d, H]
    const uint16_t* __restrict__ W1,   // w_up [E, H, d]
    int K, int N, int E, int k, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_rows, uint16_t* __restrict__ h_out, DownArgs down) {
  __shared__ int sh_tiles[2 * (kMaxE + 1)];
  __shared__ __attribute__((aligned(16))) uint16_t As[2][kPfBM * kPfLD];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][kPfBN * kPfLD];

  const TileInfo ti = find_tile(offsets, E, kPfBM, blockIdx.y, sh_tiles);
  if (ti.e < 0) return;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid / kWave;
  const int wm = wave & 1, wn = wave >> 1;
  const int n0 = blockIdx.x * (GATEUP ? kPfBN / 2 : kPfBN);

  // global -> LDS copy assignment: 16-byte chunk (tid & 7) of rows (tid >> 3) + 32 i
  const int chunk = tid & 7;
  const int rbase = tid >> 3;
  const uint16_t* aptr[4];
  const uint16_t* bptr[4];
  const long long wstride = static_cast<long long>(N) * K;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = rbase + 32 * i;
    aptr[i] = nullptr;
    if (r < ti.rows) {
      const int p = ti.row0 + r;
      const long long src = GATEUP ? static_cast<long long>(sorted_rows[p] / k) : p;
      aptr[i] = A + src * K + chunk * 8;
    }
    bptr[i] = nullptr;
    if (GATEUP) {
      const int f = n0 + (r & 63);
      if (f < N) bptr[i] = (r < 64 ? W0 : W1) + ti.e * wstride + static_cast<long long>(f) * K + chunk * 8;
    } else {
      const int f = n0 + r;
      if (f < N) bptr[i] = W0 + ti.e * wstride + static_cast<long long>(f) * K + chunk * 8;
    }
  }

  u32x4 ra[4], rb[4];
  auto load_global = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = aptr[i] ? load16(aptr[i] + k0) : u32x4{0u, 0u, 0u, 0u};
      rb[i] = bptr[i] ? load16(bptr[i] + k0) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store_lds = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      store16(&As[buf][(rbase + 32 * i) * kPfLD + chunk * 8], ra[i]);
      store16(&Bs[buf][(rbase + 32 * i) * kPfLD + chunk * 8], rb[i]);
    }
  };

  // B rows read by this wave for column block cb (gate/up: cb 0,1 gate; cb 2,3 the matching up)
  int brow[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
    if (GATEUP) brow[cb] = (cb < 2 ? 0 : 64) + wn * 32 + (cb & 1) * 16;
    else brow[cb] = wn * 64 + cb * 16;
  }

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int l16 = lane & 15;
  const int kq = (lane >> 4) * 8;
  const int nk = K / kPfBK;
  load_global(0);
  store_lds(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load_global((kt + 1) * kPfBK);
#pragma unroll
    for (int kk = 0; kk < kPfBK; kk += 32) {
      u32x4 af[4], bf[4];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        af[mb] = load16(&As[cur][(wm * 64 + mb * 16 + l16) * kPfLD + kk + kq]);
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
        bf[cb] = load16(&Bs[cur][(brow[cb] + l16) * kPfLD + kk + kq]);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) acc[mb][cb] = mfma16x16x32(af[mb], bf[cb], acc[mb][cb]);
    }
    if (kt + 1 < nk) store_lds(cur ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds rows 4 * (lane / 16) + r of each 16-row block, column lane % 16
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = wm * 64 + mb * 16 + (lane >> 4) * 4 + r;
      if (row >= ti.rows) continue;
      const int p = ti.row0 + row;
      if (GATEUP) {
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          const int f = n0 + wn * 32 + cb * 16 + l16;
          if (f < N) {
            const float hv = silu(acc[mb][cb][r]) * acc[mb][cb + 2][r];
            h_out[static_cast<long long>(p) * N + f] = f32_to_bf16_bits(hv);
          }
        }
      } else {
        const DownRow dr = down_row(down, p, N);
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          const int f = n0 + wn * 64 + cb * 16 + l16;
          if (f < N) down_put(down, dr, f, acc[mb][cb][r]);
        }
      }
    }
  }
}

// ------------------------------------------------------------------------------------- decode

constexpr int kDcFeat = 16;                 // output features per wave
constexpr int kDcBlockFeat = 4 * kDcFeat;   // per block of 4 waves

template <bool GATEUP, int MT>
__global__ __launch_bounds__(256) void gemm_decode_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ W0,
    const uint16_t* __restrict__ W1, int K, int N, int E, int k,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_rows,
    uint16_t* __restrict__ h_out, DownArgs down) {
  constexpr int BM = 16 * MT;
  constexpr int KC = 1024 / MT;             // k staged in LDS per chunk
  constexpr int LD = KC + 8;                // pitch in bf16; 16 rows land on distinct bank groups
  __shared__ int sh_tiles[2 * (kMaxE + 1)];
  __shared__ __attribute__((aligned(16))) uint16_t As[BM * LD];

  const TileInfo ti = find_tile(offsets, E, BM, blockIdx.y, sh_tiles);
  if (ti.e < 0) return;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid / kWave;
  const int l16 = lane & 15;
  const int kg = (lane >> 4) * 32;          // this lane's 32-wide k group inside a 128-k block
  const int f = blockIdx.x * kDcBlockFeat + wave * kDcFeat + l16;   // weight row (feature)
  const bool f_ok = f < N;
  const long long wstride = static_cast<long long>(N) * K;
  const uint16_t* pg = W0 + ti.e * wstride + static_cast<long long>(min(f, N - 1)) * K + kg;
  const uint16_t* pu = GATEUP ? W1 + ti.e * wstride + static_cast<long long>(min(f, N - 1)) * K + kg : nullptr;

  // gathered A row sources for the LDS staging loop
  auto stage_a = [&](int k0) {
    const int kc = min(KC, K - k0);
    const int chunks = kc / 8;
    __syncthreads();
    for (int i = tid; i < BM * chunks; i += 256) {
      const int r = i / chunks, c = i % chunks;
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (r < ti.rows) {
        const int p = ti.row0 + r;
        const long long src = GATEUP ? static_cast<long long>(sorted_rows[p] / k) : p;
        v = load16(A + src * K + k0 + c * 8);
      }
      store16(&As[r * LD + c * 8], v);
    }
    __syncthreads();
  };

  u32x4 bg0[4], bg1[4], bu0[4], bu1[4];
  auto load_b = [&](u32x4* bg, u32x4* bu, int kb) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      bg[c] = load16(pg + kb + c * 8);
      if constexpr (GATEUP) bu[c] = load16(pu + kb + c * 8);
    }
  };

  f32x4 accg[MT], accu[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    accg[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    accu[m] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  auto compute = [&](const u32x4* bg, const u32x4* bu, int kloc) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const u32x4 a = load16(&As[(m * 16 + l16) * LD + kloc + kg + c * 8]);
        accg[m] = mfma16x16x32(a, bg[c], accg[m]);
        if constexpr (GATEUP) accu[m] = mfma16x16x32(a, bu[c], accu[m]);
      }
    }
  };

  const int nb = K / 128;                   // K % 128 == 0 on this path
  constexpr int kBlocksPerChunk = KC / 128; // even, so odd blocks never start a chunk
  load_b(bg0, bu0, 0);
  int chunk0 = 0;
  for (int b = 0; b < nb; b += 2) {
    if (b % kBlocksPerChunk == 0) {
      chunk0 = b * 128;
      stage_a(chunk0);
    }
    if (b + 1 < nb) load_b(bg1, bu1, (b + 1) * 128);
    compute(bg0, bu0, b * 128 - chunk0);
    if (b + 1 < nb) {
      if (b + 2 < nb) load_b(bg0, bu0, (b + 2) * 128);
      compute(bg1, bu1, (b + 1) * 128 - chunk0);
    }
  }

  if (!f_ok) return;
#pragma unroll
  for (int m = 0; m < MT; ++m) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = m * 16 + (lane >> 4) * 4 + r;
      if (row >= ti.rows) continue;
      const int p = ti.row0 + row;
      if constexpr (GATEUP) {
        const float hv = silu(accg[m][r]) * accu[m][r];
        h_out[static_cast<long long>(p) * N + f] = f32_to_bf16_bits(hv);
      } else {
        const DownRow dr = down_row(down, p, N);
        down_put(down, dr, f, accg[m][r]);
      }
    }
  }
}

template <int MT>
hipError_t launch_decode(const uint16_t* x, const uint16_t* wg, const uint16_t* wu,
                         const uint16_t* wd, int T, int d, int E, int H, int k,
                         const int32_t* offsets, const int32_t* sorted_rows, uint16_t* h,
                         const DownArgs& down, hipStream_t s, void* mid_event) {
  const int tiles = max_tiles(T * k, E, 16 * MT);
  DownArgs none{};
  dim3 g1((H + kDcBlockFeat - 1) / kDcBlockFeat, tiles);
  gemm_decode_kernel<true, MT><<<g1, 256, 0, s>>>(x, wg, wu, d, H, E, k, offsets, sorted_rows, h,
                                                  none);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (mid_event) {
    err = record_stage_event(mid_event, s);
    if (err != hipSuccess) return err;
  }
  dim3 g2((d + kDcBlockFeat - 1) / kDcBlockFeat, tiles);
  gemm_decode_kernel<false, MT><<<g2, 256, 0, s>>>(h, wd, nullptr, H, d, E, k, offsets,
                                                   sorted_rows, nullptr, down);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ffn_bf16(const uint16_t* x, const uint16_t* wg, const uint16_t* wu,
                           const uint16_t* wd, int T, int d, int E, int H, int k,
                           const int32_t* offsets, const int32_t* sorted_rows, uint16_t* h,
                           const DownArgs& down, hipStream_t s, void* mid_event) {
  const int rows = T * k;
  if (rows <= 0) return hipSuccess;
  const bool k128 = (d % 128 == 0) && (H % 128 == 0);
  const double avg = static_cast<double>(rows) / E;
  if (k128 && avg <= 12.0) {
    return launch_decode<1>(x, wg, wu, wd, T, d, E, H, k, offsets, sorted_rows, h, down, s,
                            mid_event);
  }
  if (k128 && avg <= 32.0) {
    return launch_decode<2>(x, wg, wu, wd, T, d, E, H, k, offsets, sorted_rows, h, down, s,
                            mid_event);
  }
  const int tiles = max_tiles(rows, E, kPfBM);
  DownArgs none{};
  dim3 g1((H + kPfBN / 2 - 1) / (kPfBN / 2), tiles);
  gemm_prefill_kernel<true><<<g1, 256, 0, s>>>(x, wg, wu, d, H, E, k, offsets, sorted_rows, h,
                                               none);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (mid_event) {
    err = record_stage_event(mid_event, s);
    if (err != hipSuccess) return err;
  }
  dim3 g2((d + kPfBN - 1) / kPfBN, tiles);
  gemm_prefill_kernel<false><<<g2, 256, 0, s>>>(h, wd, nullptr, H, d, E, k, offsets, sorted_rows,
                                                nullptr, down);
  return hipGetLastError();
}

}  // namespace moe
