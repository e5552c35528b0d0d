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
// One block of 1024 threads (16 wave64s) does everything, so the result needs no inter-block
// ordering and is identical on every call. Pass 1 builds the histogram with LDS atomics (integer,
// order-free). Pass 2 walks the rows in chunks of 1024: inside a wave, lanes with the same expert
// get their rank from a ballot (lanes below with the same id), across waves a per-wave count
// table in LDS gives each wave its base, and a running per-expert base carries across chunks.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kPermThreads = 1024;
constexpr int kPermWaves = kPermThreads / kWave;

__global__ __launch_bounds__(kPermThreads) void permute_kernel(
    const int32_t* __restrict__ ids, int n, int E, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_rows, int32_t* __restrict__ row_pos,
    int32_t* __restrict__ counts_out) {
  __shared__ int cnt[kMaxE];
  __shared__ int base[kMaxE];
  __shared__ int wcnt[kPermWaves][kMaxE];
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = lane_id();

  for (int e = tid; e < E; e += kPermThreads) cnt[e] = 0;
  __syncthreads();
  for (int r = tid; r < n; r += kPermThreads) {
    const int e = min(max(ids[r], 0), E - 1);  // out-of-range ids are outside the contract
    atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  // exclusive scan over E <= 256 by wave 0, four experts per lane
  if (wave == 0) {
    int c[4];
    int run = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane * 4 + q;
      c[q] = e < E ? cnt[e] : 0;
      run += c[q];
    }
    int incl = run;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int v = __shfl_up(incl, o);
      if (lane >= o) incl += v;
    }
    int ex = incl - run;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane * 4 + q;
      if (e < E) {
        base[e] = ex;
        offsets[e] = ex;
        if (counts_out) counts_out[e] = c[q];
      }
      ex += c[q];
    }
    if (lane == kWave - 1) offsets[E] = incl;
  }
  __syncthreads();

  const unsigned long long lt_mask = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  for (int c0 = 0; c0 < n; c0 += kPermThreads) {
    for (int i = tid; i < kPermWaves * E; i += kPermThreads) wcnt[i / E][i % E] = 0;
    __syncthreads();
    const int r = c0 + tid;
    const int e = r < n ? min(max(ids[r], 0), E - 1) : -1;
    int rank = 0;
    unsigned long long pending = __ballot(e >= 0);
    while (pending) {
      const int leader = __ffsll(static_cast<long long>(pending)) - 1;
      const int le = __shfl(e, leader);
      const unsigned long long same = __ballot(e == le);
      if (e == le) {
        rank = __popcll(same & lt_mask);
        if (lane == leader) wcnt[wave][le] = __popcll(same);
      }
      pending &= ~same;
    }
    __syncthreads();
    if (e >= 0) {
      int pos = base[e] + rank;
      for (int w = 0; w < wave; ++w) pos += wcnt[w][e];
      sorted_rows[pos] = r;
      row_pos[r] = pos;
    }
    __syncthreads();
    for (int x = tid; x < E; x += kPermThreads) {
      int add = 0;
      for (int w = 0; w < kPermWaves; ++w) add += wcnt[w][x];
      base[x] += add;
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_permute(const int32_t* ids, const int32_t* /*counts_in*/, int n_rows, int E,
                          int32_t* offsets, int32_t* sorted_rows, int32_t* row_pos,
                          int32_t* counts_out, hipStream_t s) {
  permute_kernel<<<1, kPermThreads, 0, s>>>(ids, n_rows, E, offsets, sorted_rows, row_pos,
                                            counts_out);
  return hipGetLastError();
}

}  // namespace moe
