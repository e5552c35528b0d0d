// Dispatch (step 4): group the T*k assignment rows by expert, stably.
//
// The pages run the experts as one grouped matmul over the expert stacks (zonos2.cpp INTERNALS,
// "Performance": mul_mat_id over Q8_0 experts, replayed in a captured graph); the bookkeeping
// that feeds such a grouped matmul is fixed here:
//   offsets[e]      exclusive prefix sum of the per-expert counts, offsets[E] = T*k
//   sorted_rows[p]  the assignment rows r = t*k + j of expert e in ascending r, at
//                   p in [offsets[e], offsets[e+1])
//   row_pos[r]      inverse of sorted_rows
//
// Two phases, no atomics, the same result on every call:
//  1. per block of 16 tokens (16*k rows): the expert histogram of the block and the rank of each
//     row among the block's earlier rows of the same expert (written by the routing kernel, or by
//     block_hist_kernel when only the ids are given);
//  2. one block of 1024 threads scans the histograms in expert-major order (expert e, then block
//     b), which yields offsets[e] and the base position of every (block, expert) pair, and then
//     scatters: row r of block b with expert e lands at base[b][e] + rank[r].
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kScanThreads = 1024;
constexpr int kScanWaves = kScanThreads / kWave;

size_t up256(size_t v) { return (v + 255) / 256 * 256; }

__global__ __launch_bounds__(256) void block_hist_kernel(const int32_t* __restrict__ ids, int T,
                                                         int k, int E,
                                                         int32_t* __restrict__ block_hist,
                                                         int32_t* __restrict__ lrank) {
  __shared__ int sids[kTokTile * kMaxK];
  const int t0 = blockIdx.x * kTokTile;
  const int nrows = min(kTokTile, T - t0) * k;
  const int row0 = t0 * k;
  for (int i = threadIdx.x; i < nrows; i += blockDim.x)
    sids[i] = min(max(ids[row0 + i], 0), E - 1);  // out-of-range ids are outside the contract
  __syncthreads();
  block_hist_rank(sids, nrows, E, row0, block_hist, lrank);
}

__global__ __launch_bounds__(kScanThreads) void scan_scatter_kernel(
    const int32_t* __restrict__ ids, const int32_t* __restrict__ block_hist,
    const int32_t* __restrict__ lrank, int n, int k, int nb, int E, int32_t* __restrict__ base,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_rows,
    int32_t* __restrict__ row_pos, int32_t* __restrict__ counts_out) {
  __shared__ int wsum[kScanWaves];
  __shared__ int soff[kMaxE + 1];
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid / kWave;
  const int total = nb * E;
  const int per = (total + kScanThreads - 1) / kScanThreads;
  const int beg = min(tid * per, total);
  const int end = min(beg + per, total);

  // expert-major element i is (e = i / nb, b = i % nb), stored at block_hist[b * E + e]
  int s = 0;
  for (int i = beg; i < end; ++i) s += block_hist[(i % nb) * E + i / nb];
  int incl = s;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int v = __shfl_up(incl, o);
    if (lane >= o) incl += v;
  }
  if (lane == kWave - 1) wsum[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    int v = lane < kScanWaves ? wsum[lane] : 0;
    const int own = v;
#pragma unroll
    for (int o = 1; o < kScanWaves; o <<= 1) {
      const int u = __shfl_up(v, o);
      if (lane >= o) v += u;
    }
    if (lane < kScanWaves) wsum[lane] = v - own;  // exclusive prefix of the wave totals
  }
  __syncthreads();
  int run = wsum[wave] + incl - s;
  for (int i = beg; i < end; ++i) {
    const int e = i / nb, b = i % nb;
    const int h = block_hist[b * E + e];
    base[b * E + e] = run;
    if (b == 0) soff[e] = run;
    run += h;
  }
  if (tid == 0) soff[E] = n;
  __threadfence();
  __syncthreads();
  for (int e = tid; e <= E; e += kScanThreads) {
    offsets[e] = soff[e];
    if (e < E && counts_out) counts_out[e] = soff[e + 1] - soff[e];
  }
  const int rows_per_block = kTokTile * k;
  for (int r = tid; r < n; r += kScanThreads) {
    const int e = min(max(ids[r], 0), E - 1);
    const int b = r / rows_per_block;
    const int p = base[b * E + e] + lrank[r];
    sorted_rows[p] = r;
    row_pos[r] = p;
  }
}

}  // namespace

size_t dispatch_scratch_bytes(int T, int E, int k) {
  const size_t nb = (static_cast<size_t>(T) + kTokTile - 1) / kTokTile;
  return up256(nb * E * 4) * 2 + up256(static_cast<size_t>(T) * k * 4);
}

hipError_t launch_scan_scatter(const int32_t* ids, const int32_t* block_hist,
                               const int32_t* lrank, int T, int E, int k, int32_t* offsets,
                               int32_t* sorted_rows, int32_t* row_pos, int32_t* counts_out,
                               int32_t* base_scratch, hipStream_t s) {
  const int nb = (T + kTokTile - 1) / kTokTile;
  scan_scatter_kernel<<<1, kScanThreads, 0, s>>>(ids, block_hist, lrank, T * k, k, nb, E,
                                                 base_scratch, offsets, sorted_rows, row_pos,
                                                 counts_out);
  return hipGetLastError();
}

hipError_t launch_permute(const int32_t* ids, int T, int E, int k, int32_t* offsets,
                          int32_t* sorted_rows, int32_t* row_pos, int32_t* counts_out,
                          void* scratch, hipStream_t s) {
  const int nb = (T + kTokTile - 1) / kTokTile;
  char* p = static_cast<char*>(scratch);
  int32_t* hist = reinterpret_cast<int32_t*>(p);
  int32_t* base = reinterpret_cast<int32_t*>(p + up256(static_cast<size_t>(nb) * E * 4));
  int32_t* lrank = reinterpret_cast<int32_t*>(p + 2 * up256(static_cast<size_t>(nb) * E * 4));
  block_hist_kernel<<<nb, 256, 0, s>>>(ids, T, k, E, hist, lrank);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch_scan_scatter(ids, hist, lrank, T, E, k, offsets, sorted_rows, row_pos,
                             counts_out, base, s);
}

}  // namespace moe
