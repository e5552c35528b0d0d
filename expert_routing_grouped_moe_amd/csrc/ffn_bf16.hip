// bf16 expert FFN (steps 5-6) on the CDNA4 matrix cores, fp32 accumulation.
//   gate/up:  h[p, n] = silu(x[t] . Wg[e, n]) * (x[t] . Wu[e, n])      (SwiGLU; audio.cpp PR #1271,
//             "Summary"), t = sorted_rows[p] / k, h rounded to bf16
//   down:     o[p, n] = h[p] . Wd[e, n]  -> expert_out, or weighted into y
// Both are "NT" products: every operand row (token row, weight row) is contiguous along the
// reduction index, as the 3-D expert stacks of zonos2.cpp INTERNALS ("Recommended: F16 spine +
// K-quant experts") are stored.
//
// Two kernels, chosen on the host from the static shape (average rows per expert):
//  * streaming (few rows per expert, decode): the layer is a read of the touched experts'
//    weights (the single-stream regime of the ZONOS2-4bit MLX card, "Performance notes"). One
//    one-wave block per (16-feature slab, expert); weight rows stream from HBM straight into
//    registers (each load instruction covers 64 contiguous bytes of 16 rows), two 128-k blocks in
//    flight, with the expert's token rows read alongside from L2. The block finds its expert's
//    rows itself (from the dispatch order, or by scanning the expert ids), so the decode layer
//    needs no dispatch kernel.
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

// Block -> tile: column tiles fastest, then row tiles. `tiles` is the exact number of row tiles
// (computed on the device from the offsets), so the idle blocks of the worst-case grid are the
// highest block ids.
constexpr int kXcds = 8;

__device__ __forceinline__ bool prefill_tile_of_block(int ntn, int tiles, int* m, int* n) {
  const long long total = static_cast<long long>(ntn) * tiles;
  const long long L = blockIdx.x;
  if (L >= total) return false;
  *m = static_cast<int>(L / ntn);
  *n = static_cast<int>(L % ntn);
  return true;
}

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

  const int ntn = (N + (GATEUP ? kPfBN / 2 : kPfBN) - 1) / (GATEUP ? kPfBN / 2 : kPfBN);
  const int tiles = tile_scan(offsets, E, kPfBM, sh_tiles);
  int mt, nt;
  if (!prefill_tile_of_block(ntn, tiles, &mt, &nt)) return;
  const TileInfo ti = tile_lookup(E, kPfBM, mt, sh_tiles);
  if (ti.e < 0) return;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid / kWave;
  const int wm = wave & 1, wn = wave >> 1;
  const int n0 = nt * (GATEUP ? kPfBN / 2 : kPfBN);

  // global -> LDS copy assignment: 16-byte chunk (tid & 7) of rows (tid >> 3) + 32 i. Rows past
  // the tile's rows read row 0 of the tile and weight rows past N read row N - 1: the products
  // they feed land in rows/columns that are never stored (row i of the product depends only on
  // A row i, column j only on B row j), and the loads stay unconditional.
  const int chunk = tid & 7;
  const int rbase = tid >> 3;
  const uint16_t* aptr[4];
  const uint16_t* bptr[4];
  const long long wstride = static_cast<long long>(N) * K;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = rbase + 32 * i;
    const int p = ti.row0 + (r < ti.rows ? r : 0);
    const long long src = GATEUP ? static_cast<long long>(sorted_rows[p] / k) : p;
    aptr[i] = A + src * K + chunk * 8;
    const int f = min(n0 + (GATEUP ? (r & 63) : r), N - 1);
    const uint16_t* wsrc = (GATEUP && r >= 64) ? W1 : W0;
    bptr[i] = wsrc + ti.e * wstride + static_cast<long long>(f) * K + chunk * 8;
  }

  // two register stages: the loads of K tile kt + 2 are in flight while tile kt is multiplied
  // out of LDS and tile kt + 1 (loaded one step earlier) is written to the other LDS buffer
  u32x4 ra0[4], rb0[4], ra1[4], rb1[4];
  const int nk = K / kPfBK;
  auto load_global = [&](u32x4* ra, u32x4* rb, int kt) {
    const int k0 = min(kt, nk - 1) * kPfBK;  // past the end: re-read the last tile (unused)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = load16(aptr[i] + k0);
      rb[i] = load16(bptr[i] + k0);
    }
  };
  auto store_lds = [&](const u32x4* ra, const u32x4* rb, int buf) {
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
  // 16-row blocks of this wave that hold rows of the tile (a wave-uniform count)
  const int live_mb = min(4, max(0, (ti.rows - wm * 64 + 15) / 16));

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int l16 = lane & 15;
  const int kq = (lane >> 4) * 8;
  auto compute = [&](int buf) {
#pragma unroll
    for (int kk = 0; kk < kPfBK; kk += 32) {
      u32x4 bf[4];
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
        bf[cb] = load16(&Bs[buf][(brow[cb] + l16) * kPfLD + kk + kq]);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        if (mb < live_mb) {
          const u32x4 af = load16(&As[buf][(wm * 64 + mb * 16 + l16) * kPfLD + kk + kq]);
#pragma unroll
          for (int cb = 0; cb < 4; ++cb) acc[mb][cb] = mfma16x16x32(af, bf[cb], acc[mb][cb]);
        }
      }
    }
  };

  load_global(ra0, rb0, 0);
  load_global(ra1, rb1, 1);
  store_lds(ra0, rb0, 0);
  __syncthreads();
  int kt = 0;
  for (; kt + 2 <= nk; kt += 2) {
    // step kt: LDS buffer 0 holds tile kt, ra1/rb1 tile kt + 1
    load_global(ra0, rb0, kt + 2);
    compute(0);
    store_lds(ra1, rb1, 1);
    __syncthreads();
    // step kt + 1: LDS buffer 1 holds tile kt + 1, ra0/rb0 tile kt + 2
    load_global(ra1, rb1, kt + 3);
    compute(1);
    store_lds(ra0, rb0, 0);
    __syncthreads();
  }
  if (kt < nk) compute(0);  // odd tile count: the last tile sits in buffer 0

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
        const DownRow dr = down_row(down, sorted_rows[p], p, N);
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          const int f = n0 + wn * 64 + cb * 16 + l16;
          if (f < N) down_put(down, dr, f, acc[mb][cb][r]);
        }
      }
    }
  }
}

// ------------------------------------------------------------------------------ streaming

constexpr int kStFeat = 16;  // output features per block (one wave)

// Rows r (ascending) of expert e, from the expert ids, by one wave: a ballot per 64 ids.
__device__ int scan_rows(const int32_t* __restrict__ ids, int n, int e, int* lr) {
  const int lane = lane_id();
  const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  int total = 0;
  for (int base = 0; base < n; base += kWave) {
    const int r = base + lane;
    const bool m = r < n && ids[r] == e;
    const unsigned long long mask = __ballot(m);
    if (m) lr[total + __popcll(mask & lt)] = r;
    total += __popcll(mask);
  }
  __syncthreads();
  return total;
}

// One group of up to 16 rows (entries m0 .. of the expert's row list) against this wave's 16
// features over the whole reduction length K, with no barrier and no LDS staging:
//  * per 128-k block a lane loads four 16-byte pieces of its weight row (and of its up row for the
//    gate/up product) at k = 32 c + 8 (lane / 16), the MFMA operand layout, so that each load
//    instruction reads 64 contiguous bytes of each of 16 rows, and the same pieces of its A row
//    (a token row of x or a row of h, both L2-resident);
//  * two blocks are in flight ahead of use;
//  * waves start at different blocks of the reduction (a rotation by the wave's global index) so
//    that concurrent waves spread over the HBM channels instead of reading the same offset of
//    their rows. The sum order is fixed per wave, so results repeat exactly.
template <bool GATEUP>
__device__ __forceinline__ void stream_tile(const uint16_t* __restrict__ A,
                                            const uint16_t* __restrict__ W0,
                                            const uint16_t* __restrict__ W1, int K, int N, int k,
                                            int e, const int* lr, int m0, int rows, int hbase,
                                            uint16_t* __restrict__ h_out, const DownArgs& down) {
  const int lane = lane_id();
  const int l16 = lane & 15;
  const int kq = (lane >> 4) * 8;
  const int f = blockIdx.x * kStFeat + l16;  // weight row (N % 16 == 0)
  const long long wofs = static_cast<long long>(e) * N * K + static_cast<long long>(f) * K + kq;
  const uint16_t* pg = W0 + wofs;
  const uint16_t* pu = GATEUP ? W1 + wofs : nullptr;
  // lanes past the group's rows read row 0 of the group: their output rows are never stored
  // (row i of the product depends only on A row i), and the duplicate reads coalesce
  const int li_a = m0 + (l16 < rows ? l16 : 0);
  const long long arow = GATEUP ? lr[li_a] / k : (hbase >= 0 ? hbase + li_a : lr[li_a]);
  const uint16_t* pa = A + arow * K + kq;
  const int nb = K / 128;                     // even: K % 256 == 0 on this path
  const int rot = ((blockIdx.y * gridDim.x + blockIdx.x) * 5) % nb;

  u32x4 a0[4], bg0[4], bu0[4], a1[4], bg1[4], bu1[4];
  auto load = [&](u32x4* a, u32x4* bg, u32x4* bu, int sq) {
    const int kb = ((min(sq, nb - 1) + rot) % nb) * 128;  // past the end: re-read the last block
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      bg[c] = load16(pg + kb + c * 32);
      if constexpr (GATEUP) bu[c] = load16(pu + kb + c * 32);
      a[c] = load16(pa + kb + c * 32);
    }
  };
  f32x4 accg = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 accu = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const u32x4* a, const u32x4* bg, const u32x4* bu) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      accg = mfma16x16x32(a[c], bg[c], accg);
      if constexpr (GATEUP) accu = mfma16x16x32(a[c], bu[c], accu);
    }
  };
  load(a0, bg0, bu0, 0);
  load(a1, bg1, bu1, 1);
  for (int sq = 0; sq < nb; sq += 2) {
    // sched_barrier keeps the scheduler from sinking the prefetches below the next compute
    compute(a0, bg0, bu0);
    __builtin_amdgcn_sched_barrier(0);
    load(a0, bg0, bu0, sq + 2);
    __builtin_amdgcn_sched_barrier(0);
    compute(a1, bg1, bu1);
    __builtin_amdgcn_sched_barrier(0);
    load(a1, bg1, bu1, sq + 3);
    __builtin_amdgcn_sched_barrier(0);
  }

#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = (lane >> 4) * 4 + r;  // row of this group
    if (i >= rows) continue;
    const int li = m0 + i;              // entry of the expert's row list
    const int hrow = hbase >= 0 ? hbase + li : lr[li];
    if constexpr (GATEUP) {
      const float hv = silu(accg[r]) * accu[r];
      h_out[static_cast<long long>(hrow) * N + f] = f32_to_bf16_bits(hv);
    } else {
      const DownRow dr = down_row(down, lr[li], hrow, N);
      down_put(down, dr, f, accg[r]);
    }
  }
}

// Grid (N / 16, E), one wave per block: block (x, e) computes features [16 x, 16 x + 16) of
// expert e for all of the expert's rows, 16 rows per pass (a second pass over the same weights
// mostly hits the caches).
template <bool GATEUP>
__global__ __launch_bounds__(kWave) void ffn_stream_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ W0,
    const uint16_t* __restrict__ W1, int K, int N, int k, RowSource rs,
    uint16_t* __restrict__ h_out, DownArgs down) {
  __shared__ int lr[kMaxScanRows];
  const int e = blockIdx.y;
  int count, hbase;
  if (rs.ids) {
    count = scan_rows(rs.ids, rs.n_rows, e, lr);
    hbase = -1;
    if (rs.counts_out && blockIdx.x == 0 && threadIdx.x == 0) rs.counts_out[e] = count;
  } else {
    hbase = rs.offsets[e];
    count = rs.offsets[e + 1] - hbase;
    for (int i = threadIdx.x; i < count; i += blockDim.x) lr[i] = rs.sorted_rows[hbase + i];
    __syncthreads();
  }
  for (int m0 = 0; m0 < count; m0 += 16)
    stream_tile<GATEUP>(A, W0, W1, K, N, k, e, lr, m0, min(16, count - m0), hbase, h_out, down);
}

}  // namespace

bool ffn_bf16_streaming(int T, int d, int E, int H, int k) {
  const long long rows = static_cast<long long>(T) * k;
  return rows <= kMaxScanRows && d % 256 == 0 && H % 256 == 0 && rows <= 32ll * E;
}

hipError_t launch_ffn_bf16(const uint16_t* x, const uint16_t* wg, const uint16_t* wu,
                           const uint16_t* wd, int T, int d, int E, int H, int k,
                           const RowSource& rs, uint16_t* h, const DownArgs& down, hipStream_t s,
                           void* mid_event) {
  const int rows = T * k;
  if (rows <= 0) return hipSuccess;
  DownArgs none{};
  hipError_t err;
  if (ffn_bf16_streaming(T, d, E, H, k)) {
    ffn_stream_kernel<true><<<dim3(H / kStFeat, E), kWave, 0, s>>>(x, wg, wu, d, H, k, rs, h,
                                                                    none);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (mid_event && (err = record_stage_event(mid_event, s)) != hipSuccess) return err;
    RowSource rs2 = rs;
    rs2.counts_out = nullptr;
    ffn_stream_kernel<false><<<dim3(d / kStFeat, E), kWave, 0, s>>>(h, wd, nullptr, H, d, k,
                                                                     rs2, nullptr, down);
    return hipGetLastError();
  }
  // grouped GEMM over the dispatch order (rs.offsets / rs.sorted_rows); a 1-D grid sized for
  // the worst-case tile count, rounded up to whole XCD rounds
  const long long tiles = max_tiles(rows, E, kPfBM);
  auto grid_for = [&](int ntn) {
    const long long total = tiles * ntn;
    return static_cast<unsigned>((total + kXcds - 1) / kXcds * kXcds);
  };
  const int ntn1 = (H + kPfBN / 2 - 1) / (kPfBN / 2);
  gemm_prefill_kernel<true><<<grid_for(ntn1), 256, 0, s>>>(x, wg, wu, d, H, E, k, rs.offsets,
                                                           rs.sorted_rows, h, none);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (mid_event && (err = record_stage_event(mid_event, s)) != hipSuccess) return err;
  const int ntn2 = (d + kPfBN - 1) / kPfBN;
  gemm_prefill_kernel<false><<<grid_for(ntn2), 256, 0, s>>>(h, wd, nullptr, H, d, E, k,
                                                            rs.offsets, rs.sorted_rows, nullptr,
                                                            down);
  return hipGetLastError();
}

}  // namespace moe
