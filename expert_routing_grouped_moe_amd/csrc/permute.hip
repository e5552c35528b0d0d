// Dispatch (step 4): group the T*k assignment rows by expert, stably.
//
// The pages run the experts as one grouped matmul over the expert stacks (zonos2.cpp internals,
// "Performance": mul_mat_id over Q8_0 experts, replayed in a captured graph); the bookkeeping
// that feeds such a grouped matmul is fixed here:
//   offsets[e]      exclusive prefix sum of the per-expert counts, offsets[E] = T*k
//   sorted_rows[p]  the assignment rows r = t*k + j of expert e in ascending r, at
//                   p in [offsets[e], offsets[e+1])
//   row_pos[r]      inverse of sorted_rows
//
// One block per expert, no inter-block communication, the same result on every call:
//  pass 1  every block counts, over all T*k ids, those below its expert (= offsets[e]) and those
//          equal to it (= counts[e]): plain compares and a block reduction, no atomics;
//  pass 2  thread i owns a contiguous run of rows (runs in thread order = rows in ascending
//          order); a block-wide exclusive scan of the per-thread match counts places each of the
//          block's rows, which it writes to sorted_rows and row_pos.
// Rows are read 8 per thread per round with all 8 loads issued before use. With T*k <= 8192 one
// round does both passes, each thread owning two runs of four rows (one in each half of the ids)
// read with whole-line 16-byte loads.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kDispThreads = 1024;
constexpr int kDispWaves = kDispThreads / kWave;
constexpr int kPer = 8;                         // rows per thread per round
constexpr int kRound = kDispThreads * kPer;

__device__ __forceinline__ int clamp_id(int e, int E) { return min(max(e, 0), E - 1); }

__global__ __launch_bounds__(kDispThreads) void dispatch_kernel(
    const int32_t* __restrict__ ids, int n, int E, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_rows, int32_t* __restrict__ row_pos,
    int32_t* __restrict__ counts_out) {
  __shared__ int wsum[kDispWaves];
  __shared__ int wless[kDispWaves];
  __shared__ int s_base;
  const int e = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid / kWave;

  if (n <= kRound) {
    // one round: the ids are read once, and one barrier serves both the counts and the scan.
    // Thread t owns two runs of four rows, 4 t .. 4 t + 3 and kRound / 2 + 4 t .. + 3, so that
    // each wave's 16-byte loads cover whole lines (eight rows per thread in one run would leave
    // every load instruction with half of each line, and took about twice as long); the counts
    // of the two runs are scanned together, packed in one integer (each below 2^16).
    constexpr int kHalf = kRound / 2;
    int v[kPer];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r0 = h * kHalf + 4 * tid;
      if (r0 + 3 < n) {
        const int4 q = *reinterpret_cast<const int4*>(ids + r0);
        v[4 * h + 0] = clamp_id(q.x, E);
        v[4 * h + 1] = clamp_id(q.y, E);
        v[4 * h + 2] = clamp_id(q.z, E);
        v[4 * h + 3] = clamp_id(q.w, E);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[4 * h + i] = r0 + i < n ? clamp_id(ids[r0 + i], E) : E;
      }
    }
    int less = 0, mine0 = 0, mine1 = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) less += v[i] < e;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      mine0 += v[i] == e;
      mine1 += v[4 + i] == e;
    }
    const int mine = mine0 | (mine1 << 16);
    int incl = mine;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int u = __shfl_up(incl, o);
      if (lane >= o) incl += u;
    }
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) less += __shfl_xor(less, o);
    if (lane == kWave - 1) wsum[wave] = incl;
    if (lane == 0) wless[wave] = less;
    __syncthreads();
    int base = 0, before = 0, total = 0;
    for (int w = 0; w < kDispWaves; ++w) {
      const int t = wsum[w];
      base += wless[w];
      if (w < wave) before += t;
      total += t;
    }
    const int total0 = total & 0xffff, total1 = total >> 16;
    if (tid == 0) {
      offsets[e] = base;
      if (counts_out) counts_out[e] = total0 + total1;
      if (e == E - 1) offsets[E] = n;
    }
    const int excl = before + incl - mine;    // packed: earlier rows of run 0 | of run 1 << 16
    int p0 = base + (excl & 0xffff);
    int p1 = base + total0 + (excl >> 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (v[i] == e) {
        const int r = 4 * tid + i;
        sorted_rows[p0] = r;
        row_pos[r] = p0;
        ++p0;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (v[4 + i] == e) {
        const int r = kHalf + 4 * tid + i;
        sorted_rows[p1] = r;
        row_pos[r] = p1;
        ++p1;
      }
    }
    return;
  }

  // pass 1: rows with a smaller expert id, and rows of this expert
  int less = 0, mine_all = 0;
  for (int base = 0; base < n; base += kRound) {
    int v[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int r = base + tid * kPer + i;
      v[i] = r < n ? clamp_id(ids[r], E) : E;   // past the end: counts nowhere
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      less += v[i] < e;
      mine_all += v[i] == e;
    }
  }
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) {
    less += __shfl_xor(less, o);
    mine_all += __shfl_xor(mine_all, o);
  }
  if (lane == 0) {
    wless[wave] = less;
    wsum[wave] = mine_all;
  }
  __syncthreads();
  if (tid == 0) {
    int tl = 0, tm = 0;
    for (int w = 0; w < kDispWaves; ++w) {
      tl += wless[w];
      tm += wsum[w];
    }
    s_base = tl;
    offsets[e] = tl;
    if (counts_out) counts_out[e] = tm;
    if (e == E - 1) offsets[E] = n;
  }
  __syncthreads();
  // pass 2: stable placement of this expert's rows
  int run = s_base;
  for (int base = 0; base < n; base += kRound) {
    int v[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int r = base + tid * kPer + i;
      v[i] = r < n ? clamp_id(ids[r], E) : -1;
    }
    int mine = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) mine += v[i] == e;
    int incl = mine;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int u = __shfl_up(incl, o);
      if (lane >= o) incl += u;
    }
    if (lane == kWave - 1) wsum[wave] = incl;
    __syncthreads();
    int before = 0, total = 0;
    for (int w = 0; w < kDispWaves; ++w) {
      const int t = wsum[w];
      if (w < wave) before += t;
      total += t;
    }
    int p = run + before + incl - mine;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      if (v[i] == e) {
        const int r = base + tid * kPer + i;
        sorted_rows[p] = r;
        row_pos[r] = p;
        ++p;
      }
    }
    run += total;
    __syncthreads();
  }
}

// counts[e] = number of ids equal to e among ids[0..n): one block, an LDS histogram.
__global__ __launch_bounds__(kDispThreads) void counts_kernel(const int32_t* __restrict__ ids,
                                                              int n, int E,
                                                              int32_t* __restrict__ counts) {
  __shared__ int hist[kMaxE];
  for (int e = threadIdx.x; e < E; e += kDispThreads) hist[e] = 0;
  __syncthreads();
  for (int r = threadIdx.x; r < n; r += kDispThreads) atomicAdd(&hist[clamp_id(ids[r], E)], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kDispThreads) counts[e] = hist[e];
}

}  // namespace

hipError_t launch_counts(const int32_t* ids, int n_rows, int E, int32_t* counts, hipStream_t s) {
  counts_kernel<<<1, kDispThreads, 0, s>>>(ids, n_rows, E, counts);
  return hipGetLastError();
}

hipError_t launch_dispatch(const int32_t* ids, int n_rows, int E, int32_t* offsets,
                           int32_t* sorted_rows, int32_t* row_pos, int32_t* counts_out,
                           hipStream_t s) {
  dispatch_kernel<<<E, kDispThreads, 0, s>>>(ids, n_rows, E, offsets, sorted_rows, row_pos,
                                             counts_out);
  return hipGetLastError();
}

}  // namespace moe
