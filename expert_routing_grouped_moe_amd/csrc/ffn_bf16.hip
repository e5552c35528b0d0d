// bf16 expert FFN (steps 5-6) on the CDNA4 matrix cores, fp32 accumulation.
//   gate/up:  h[p, n] = silu(x[t] . Wg[e, n]) * (x[t] . Wu[e, n])      (SwiGLU; audio.cpp PR #1271,
//             "Summary"), t = sorted_rows[p] / k, h rounded to fp16 (saturated at +-65504)
//   down:     o[p, n] = h[p] . Wd[e, n]  -> expert_out, or weighted into y; fp16 operands (int8
//             codes convert exactly, bf16 weights exactly for magnitudes 2^-17..65504, smaller
//             ones toward zero; 4-bit weights s * q + b are formed with one fp16 fused
//             multiply-add), fp32 accumulation. fp16's 11
//             significant bits keep the rounding of h from dominating the error: rounded to bf16,
//             h alone put the skewed prefill's largest output error at 0.0203 x output RMS.
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
//  * prefill (many rows per expert): a grouped GEMM over the dispatch order, operands copied
//    from global memory straight into an LDS ring (no register staging), waves of 64 x 64: 128 x
//    256 tiles with 32-wide K steps at two blocks per CU while the experts average less than a
//    256-row tile; beyond that the tiles are ordered per XCD for L2 reuse, gate/up on 256 x 256
//    tiles with 64-wide K steps (one block of 16 waves per CU) and down on 256 x 128 tiles.
#include <type_traits>

#include "common.hpp"
#include "down_epilogue.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

// ------------------------------------------------------------------------------------ prefill

// Block -> tile. `tiles` is the exact number of row tiles (computed on the device from the
// offsets); blocks past the last tile exit. XCD-aware order: the hardware hands block b to XCD
// b % kXcds (kXcds L2 domains of 4 MB); XCD x takes a contiguous range of the tile order, and that
// order runs through groups of kXcdGroup row tiles with the row tile fastest, so the blocks sharing
// an XCD's L2 at one time also share most of their A and B tiles. Lines that miss the L2 come from
// the Infinity Fabric at little more than HBM speed (~7 TB/s measured even for data resident in
// the Infinity Cache). Against column tiles fastest over the whole grid: skewed prefill ~40 % fewer
// bytes fetched and ~8 % less time; ZONOS3-Mini prefill (about one row tile per expert) ~2 % less
// time per step.
constexpr int kXcds = 8;
constexpr int kXcdGroup = 4;

__device__ __forceinline__ bool prefill_tile_of_block(int ntn, int tiles, int* m, int* n) {
  const long long total = static_cast<long long>(ntn) * tiles;
  const long long b = blockIdx.x;
  const long long per = (total + kXcds - 1) / kXcds;
  const long long j = b / kXcds;
  if (j >= per) return false;
  const long long L = (b % kXcds) * per + j;
  if (L >= total) return false;
  const long long gsz = static_cast<long long>(kXcdGroup) * ntn;
  const long long group = L / gsz;
  const long long r = L - group * gsz;
  const int first = static_cast<int>(group) * kXcdGroup;
  const int gs = min(kXcdGroup, tiles - first);
  *m = first + static_cast<int>(r % gs);
  *n = static_cast<int>(r / gs);
  return true;
}

// Blocks a launch needs for up to `max_row_tiles` row tiles: tile L sits at block
// (L % per) * kXcds + L / per, which reaches up to kXcds * per - 1 >= total - 1.
inline long long prefill_grid(long long max_row_tiles, int ntn) {
  const long long total = max_row_tiles * ntn;
  return (total + kXcds - 1) / kXcds * kXcds;
}

// The wide tiles once the experts average a full 256-row tile or more.
inline bool prefill_wide_tiles(int rows, int E, int bm) {
  return rows >= static_cast<long long>(bm) * E;
}

// Grouped GEMM with loads straight from global memory into LDS (global_load_lds_dwordx4: each
// lane's 16 bytes land at base + 16 * lane, so one wave instruction fills 1 KB: 16 rows of a
// 32-wide K step or 8 rows of a 64-wide one). A ring of RING K steps lives in LDS; the loads of
// step kt + RING - 1 are issued right after the barrier that retires step kt - 1, so RING - 1
// steps are in flight behind the products. One barrier per K step. Waves of WROWS x 64 outputs,
// (BM / WROWS) x (BN / 64) of them per block.
// An LDS row holds one K step of one operand row: 64 bytes for BK = 32, whose four 16-byte pieces
// sit at position piece ^ (((r >> 1) ^ (r >> 2)) & 3), or 128 bytes for BK = 64, whose eight
// pieces sit at piece ^ ((r >> 1) & 7); either way a fragment read (16 consecutive rows, one
// piece) touches 16 distinct 16-byte bank groups.
// Three slots of 32-wide steps of a 256 x 128 or 128 x 256 tile take 72 KB, so two blocks
// (16 waves, <= 128 VGPRs each) share a CU and one block's barrier wait is covered by the other's
// products; the 256 x 256 tile with 64-wide steps (two slots, 128 KB) runs one block per CU.

template <int BK>
__device__ __forceinline__ int swz(int r) {
  static_assert(BK == 32 || BK == 64, "K step");
  if constexpr (BK == 32) return ((r >> 1) ^ (r >> 2)) & 3;
  else return (r >> 1) & 7;
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// wait until at most `behind` steps of CPW loads each are outstanding (behind <= B)
template <int B, int CPW>
__device__ __forceinline__ void wait_steps_behind(int behind) {
  if constexpr (B == 0) {
    wait_vmcnt<0>();
  } else {
    if (behind >= B) wait_vmcnt<B * CPW>();
    else wait_steps_behind<B - 1, CPW>(behind);
  }
}

__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// BFRAG: the weight stacks (B) are stored fragment-major (moe_pack_weights_frag): each 16-row x
// 32-k fragment is one contiguous kilobyte, lane l's piece (row l % 16, k 8 (l / 16) .. + 7) at
// 16 l. Such a fragment is copied as one of the step's 1 KB chunks and lands in LDS already in the
// order the MFMA reads it (lane l's piece at 16 l), so those reads need no swizzle; the products
// and their order are the same as with row-major weights.
template <bool GATEUP, int BM, int BN, int RING, int WROWS, int BK, bool BFRAG>
__global__ __launch_bounds__(BM / WROWS * (BN / 64) * kWave)
__attribute__((amdgpu_waves_per_eu(2))) void gemm_dma_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ W0,
    const uint16_t* __restrict__ W1, int K, int N, int E, int k,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_rows,
    uint16_t* __restrict__ h_out, DownArgs down) {
  constexpr int WMW = BM / WROWS;           // waves along M (WROWS rows each)
  constexpr int WNW = BN / 64;              // waves along N (64 columns each)
  constexpr int NW = WMW * WNW;             // waves per block
  constexpr int WN = BN / WNW;              // columns per wave
  constexpr int MB = WROWS / 16;            // 16-row blocks per wave
  constexpr int NBK = WN / 16;              // 16-column blocks per wave
  constexpr int RPC = 1024 / (2 * BK);            // rows per 1 KB chunk
  constexpr int PCS = BK / 8;                     // 16-byte pieces per row
  constexpr int CHA = BM / RPC, CHB = BN / RPC;   // 1 KB chunks per K step
  constexpr int CPW = (CHA + CHB) / NW;           // chunks per wave per K step
  static_assert((CHA + CHB) % NW == 0, "chunks split over the waves");
  static_assert(RING >= 2 && (RING - 2) * CPW < 64, "ring depth within the wait counter");
  constexpr int STAGE = (BM + BN) * BK;           // bf16 elements per ring slot
  constexpr int FEAT = GATEUP ? BN / 2 : BN;
  __shared__ __attribute__((aligned(1024))) uint16_t ring[RING * STAGE];
  static_assert(2 * (kMaxE + 1) * 4 <= STAGE * 2, "tile table fits one slot");
  int* sh_tiles = reinterpret_cast<int*>(&ring[(RING - 1) * STAGE]);

  const int ntn = (N + FEAT - 1) / FEAT;
  const int tiles = tile_scan(offsets, E, BM, sh_tiles);
  int mt, nt;
  if (!prefill_tile_of_block(ntn, tiles, &mt, &nt)) return;
  const TileInfo ti = tile_lookup(E, BM, mt, sh_tiles);
  if (ti.e < 0) return;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid / kWave;
  // wave w runs on SIMD w % 4; bands of 64 rows go to wave pairs (w / WNW), so a tile whose rows
  // end within its first half still keeps every SIMD busy with one wave (the others skip)
  const int wm = wave / WNW, wn = wave % WNW;
  const int n0 = nt * FEAT;
  const long long wstride = static_cast<long long>(N) * K;

  // this lane's source rows: chunk j = wave + NW c covers LDS rows RPC j .. RPC j + RPC - 1 of
  // the step (A rows first, then B rows); lane i fills row RPC j + i / PCS, position i % PCS
  const uint16_t* src[CPW];
  int ldsoff[CPW];
  bool fragc[CPW];                          // a fragment-major weight chunk (16 k per K step)
#pragma unroll
  for (int c = 0; c < CPW; ++c) {
    const int j = wave + NW * c;
    const int r = RPC * j + lane / PCS;     // row of the step tile (A: < BM)
    const int pos = lane % PCS;
    fragc[c] = BFRAG && j >= CHA;
    if (j < CHA) {
      const int pr = ti.row0 + (r < ti.rows ? r : 0);
      const long long arow = GATEUP ? static_cast<long long>(sorted_rows[pr] / k) : pr;
      src[c] = A + arow * K + ((pos ^ swz<BK>(r)) * 8);
    } else if constexpr (BFRAG) {
      // chunk jb of the step's weight rows: 16-row block jb / (BK / 32), its fragment jb % (BK /
      // 32) of the step; N % 16 == 0, so a block past the last row reads the last block
      const int jb = j - CHA;
      const int rb16 = 16 * (jb / (BK / 32));
      const int f0 = min(n0 + (GATEUP ? (rb16 % FEAT) : rb16), N - 16);
      const uint16_t* wsrc = (GATEUP && rb16 >= FEAT) ? W1 : W0;
      const long long blk = (static_cast<long long>(ti.e) * N + f0) / 16;
      src[c] = wsrc + (blk * (K / 32) + jb % (BK / 32)) * 512 + 8 * lane;
    } else {
      const int rb = r - BM;
      const int f = min(n0 + (GATEUP ? (rb % FEAT) : rb), N - 1);
      const uint16_t* wsrc = (GATEUP && rb >= FEAT) ? W1 : W0;
      src[c] = wsrc + ti.e * wstride + static_cast<long long>(f) * K + ((pos ^ swz<BK>(rb)) * 8);
    }
    ldsoff[c] = RPC * j * BK;               // element offset of the chunk inside a slot
  }
  const int nk = K / BK;
  const uint32_t ring0 = lds_addr(ring);
  auto issue = [&](int kt) {
    const int slot = kt % RING;
    const int k0 = min(kt, nk - 1) * BK;    // prologue past the end: re-read the last step
#pragma unroll
    for (int c = 0; c < CPW; ++c)   // a fragment-major chunk advances 512 elements per 32 k
      dma16(src[c] + (fragc[c] ? 16 * k0 : k0),
            ring0 + 2u * static_cast<uint32_t>(slot * STAGE + ldsoff[c]));
  };

  int brow[NBK];
#pragma unroll
  for (int cb = 0; cb < NBK; ++cb) {
    if (GATEUP) brow[cb] = (cb < NBK / 2 ? 0 : FEAT) + wn * (WN / 2) + (cb % (NBK / 2)) * 16;
    else brow[cb] = wn * WN + cb * 16;
  }
  const int live_mb = min(MB, max(0, (ti.rows - wm * WROWS + 15) / 16));
  const bool wave_live = live_mb > 0;
  const int l16 = lane & 15;
  const int q = lane >> 4;                  // 16-byte piece (k 8q .. 8q+7) of the MFMA step
  // fragment offsets of the first 32-wide MFMA step of a slot; with BK = 64 the second step's
  // pieces 4 + q sit at offset ^ 32 (the piece index's bit 2)
  int aoff[MB], boff[NBK];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int r = wm * WROWS + mb * 16 + l16;
    aoff[mb] = r * BK + ((q ^ swz<BK>(r)) * 8);
  }
#pragma unroll
  for (int cb = 0; cb < NBK; ++cb) {
    const int r = brow[cb] + l16;
    boff[cb] = BFRAG ? BM * BK + (brow[cb] / 16) * (BK / 32) * 512 + 8 * lane
                     : BM * BK + r * BK + ((q ^ swz<BK>(r)) * 8);
  }

  f32x4 acc[MB][NBK];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NBK; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int slot) {
    const uint16_t* st = &ring[slot * STAGE];
#pragma unroll
    for (int sub = 0; sub < BK / 32; ++sub) {
      const int x = 32 * sub;               // XOR on the element offset
      u32x4 bf[NBK], af[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) af[mb] = load16(st + (aoff[mb] ^ x));
#pragma unroll
      for (int cb = 0; cb < NBK; ++cb)
        bf[cb] = load16(st + (BFRAG ? boff[cb] + 16 * x : (boff[cb] ^ x)));
      if constexpr (!GATEUP) {              // h is fp16: the bf16 weights go to fp16
#pragma unroll
        for (int cb = 0; cb < NBK; ++cb) bf[cb] = bf16x8_to_f16x8(bf[cb]);
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int cb = 0; cb < NBK; ++cb)
          acc[mb][cb] = GATEUP ? mfma16x16x32(af[mb], bf[cb], acc[mb][cb])
                               : mfma16x16x32_f16(af[mb], bf[cb], acc[mb][cb]);
    }
  };

  // issue order = step order; step kt is complete once at most (issued after it) * CPW of this
  // wave's loads are outstanding, and visible to the block after the barrier that follows
#pragma unroll
  for (int s = 0; s < RING - 1; ++s) issue(s);
  int kt = 0;
  for (; kt + RING - 1 < nk; ++kt) {
    wait_vmcnt<(RING - 2) * CPW>();
    block_barrier();                        // slot (kt - 1) % RING is free in every wave
    issue(kt + RING - 1);
    if (wave_live) compute(kt % RING);
  }
  for (; kt < nk; ++kt) {                   // nothing more to issue; nk - 1 - kt steps behind
    wait_steps_behind<RING - 2, CPW>(nk - 1 - kt);
    block_barrier();
    if (wave_live) compute(kt % RING);
  }
  wait_vmcnt<0>();                          // prologue re-reads (K < 3 steps) have landed too
  block_barrier();                          // every wave is done with the ring: reuse it below

  // Epilogue through LDS: each wave stages one 16-row block of its results at a time in a private
  // part of the ring, then writes whole 16-byte pieces of output rows (gate/up: 8 fp16 h values;
  // down: 4 fp32 values), so that every store instruction covers 4 rows x 64 (h) or 256 (y) bytes.
  if (!wave_live) return;
  constexpr int CW = GATEUP ? WN / 2 : WN;             // output columns per wave
  constexpr int EB = GATEUP ? 2 : 4;                   // bytes per output element
  constexpr int PITCH = CW * EB + 16;                  // staging row pitch in bytes (padded)
  char* stage = reinterpret_cast<char*>(ring) + wave * 16 * PITCH;
  const int c0 = n0 + wn * CW;                         // first output column of this wave
  constexpr int PR = CW * EB / 16;                     // 16-byte pieces per staged row
  static_assert(PR >= 1 && 64 % PR == 0, "pieces per row");
  constexpr int RPI = 64 / PR;                         // staged rows covered per instruction
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    if (mb >= live_mb) break;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int sr = (lane >> 4) * 4 + r;              // staged row (0..15)
      if constexpr (GATEUP) {
#pragma unroll
        for (int cb = 0; cb < NBK / 2; ++cb) {
          const float hv = silu(acc[mb][cb][r]) * acc[mb][cb + NBK / 2][r];
          *reinterpret_cast<uint16_t*>(stage + sr * PITCH + (cb * 16 + l16) * 2) = f32_to_f16_bits_sat(hv);
        }
      } else {
#pragma unroll
        for (int cb = 0; cb < NBK; ++cb)
          *reinterpret_cast<float*>(stage + sr * PITCH + (cb * 16 + l16) * 4) = acc[mb][cb][r];
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's staging is in LDS
#pragma unroll
    for (int it = 0; it < 16 / RPI; ++it) {
      const int sr = it * RPI + lane / PR;             // staged row this lane writes
      const int pc = lane % PR;                        // its 16-byte piece
      const int row = wm * WROWS + mb * 16 + sr;
      const int col = c0 + pc * (16 / EB);
      const u32x4 v = *reinterpret_cast<const u32x4*>(stage + sr * PITCH + pc * 16);
      if (row < ti.rows && col < N) {
        const int p = ti.row0 + row;
        if constexpr (GATEUP) {
          store16(h_out + static_cast<long long>(p) * N + col, v);
        } else {
          const DownRow dr = down_row(down, sorted_rows[p], p, N);
          down_put4(down, dr, col, v);
        }
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // read back before the next block's writes
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

// The same from ids already in registers (id[i] = ids[lane + 64 i], -1 past n; n <= 64 R).
template <int R>
__device__ int scan_rows_regs(const int (&id)[R], int e, int* lr) {
  const int lane = lane_id();
  const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  int total = 0;
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const bool m = id[i] == e;
    const unsigned long long mask = __ballot(m);
    if (m) lr[total + __popcll(mask & lt)] = kWave * i + lane;
    total += __popcll(mask);
  }
  __syncthreads();
  return total;
}

// 8 int8 codes (two dwords, lowest k first) as 8 bf16 values (exact: |code| <= 127 needs 7
// significand bits): sign-extend, convert to fp32, keep the upper halves.
__device__ __forceinline__ uint32_t i8pair_to_bf16x2(uint32_t v, int sh) {
  const float lo = static_cast<float>(static_cast<int8_t>(v >> sh));
  const float hi = static_cast<float>(static_cast<int8_t>(v >> (sh + 8)));
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}
__device__ __forceinline__ u32x4 i8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  return u32x4{i8pair_to_bf16x2(w0, 0), i8pair_to_bf16x2(w0, 16), i8pair_to_bf16x2(w1, 0),
               i8pair_to_bf16x2(w1, 16)};
}
// The same codes as 8 fp16 values (exact), for products against the fp16 h.
__device__ __forceinline__ uint32_t i8pair_to_f16x2(uint32_t v, int sh) {
  const float lo = static_cast<float>(static_cast<int8_t>(v >> sh));
  const float hi = static_cast<float>(static_cast<int8_t>(v >> (sh + 8)));
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
}
__device__ __forceinline__ u32x4 i8x8_to_f16x8(uint32_t w0, uint32_t w1) {
  return u32x4{i8pair_to_f16x2(w0, 0), i8pair_to_f16x2(w0, 16), i8pair_to_f16x2(w1, 0),
               i8pair_to_f16x2(w1, 16)};
}

// 8 packed 4-bit codes (see moe_quantize_groups_q4: element 2 j is the nibble at bits 4 j, element
// 2 j + 1 the one at bits 16 + 4 j, so both halves of a dword belong to one group) dequantised as
// w = s * q + b with the group's bf16 scale s (low half of `pair`) and bias b (high half): one
// packed fp16 fused multiply-add per pair, rounded once to nearest fp16 (s and b convert to fp16
// exactly for magnitudes 2^-14..65504). 11 significant bits: rounded to bf16 instead, the
// weights' rounding put zonos2 decode's largest output error at 0.0175 x output RMS, near the
// 2e-2 bound.
__device__ __forceinline__ u32x4 q4x8_dequant(uint32_t v, uint32_t pair) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  const float sc = __uint_as_float(pair << 16);
  const float bs = __uint_as_float(pair & 0xffff0000u);
  const f16x2 s2 = __builtin_convertvector(f32x2{sc, sc}, f16x2);
  const f16x2 b2 = __builtin_convertvector(f32x2{bs, bs}, f16x2);
  const f16x2 base{static_cast<_Float16>(1024.f), static_cast<_Float16>(1024.f)};
  u32x4 out;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // the pair's codes as the fp16 values 1024 + q (exact), less 1024 (exact), then s * q + b
    // with one rounding
    const uint32_t m = ((v >> (4 * j)) & 0x000F000Fu) | 0x64006400u;
    const f16x2 q = __builtin_bit_cast(f16x2, m) - base;
    out[j] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(q, s2, b2));
  }
  return out;
}

// Up to NG groups of 16 rows (entries m0 .. of the expert's row list) against this wave's 16
// features over the whole reduction length K, with no barrier and no LDS staging; the groups
// share every weight load, so an expert with up to 16 NG rows reads its weights once:
//  * per 128-k block, MFMA step c (c = 0..3) and lane group g = lane / 16 cover 8 consecutive k;
//    bf16 weights: k = 32 c + 8 g, so each load instruction reads 64 contiguous bytes of each of
//    16 rows; int8 weights (W8): k = 32 g + 8 c, so a lane's 32 code bytes of the block are
//    contiguous (two 16-byte loads), converted to bf16 right before the MFMA and scaled per row
//    in the epilogue; 4-bit weights (W4): the bf16 k layout, a lane's 16 code bytes of the block
//    in one load plus the (scale, bias) pairs of the block's two groups of 64, each weight formed
//    as s * q + b in fp16 right before the MFMA (q4x8_dequant), the gate/up's
//    bf16 token rows converted to fp16 for these products. Fragment-major storage of any of the
//    three (WFR): the same bytes reach the same lanes, but each load instruction's 64 lanes x 16
//    bytes are one contiguous kilobyte (eight whole 128-byte lines, where a row-major instruction
//    covers half of each of 16 lines). The A rows (a token row of x or a row of h, both
//    L2-resident) are read with the same k layout, one piece per step, for every group;
//  * two blocks are in flight ahead of use;
//  * waves start at different blocks of the reduction (a rotation by the wave's global index) so
//    that concurrent waves spread over the HBM channels instead of reading the same offset of
//    their rows. The sum order is fixed per wave, so results repeat exactly.
template <bool GATEUP, int NG, int WF, int NB>
__device__ __forceinline__ void stream_tile(const uint16_t* __restrict__ A,
                                            const void* __restrict__ W0,
                                            const void* __restrict__ W1,
                                            const void* __restrict__ S0,
                                            const void* __restrict__ S1, int K, int N, int k,
                                            int e, int slab, const int* lr, int m0, int rows,
                                            int hbase, uint16_t* __restrict__ h_out,
                                            const DownArgs& down) {
  constexpr int BASE = WF & ~kWFragMajor;
  constexpr bool W8 = BASE == kWI8, W4 = BASE == kWQ4, WFR = (WF & kWFragMajor) != 0;
  constexpr int WR = W8 ? 2 : (W4 ? 1 : 4);   // weight registers (u32x4) per matrix per block
  const int lane = lane_id();
  const int l16 = lane & 15;
  const int grp = lane >> 4;
  const int kq = W8 ? 32 * grp : 8 * grp;     // lane's first k inside a 128-k block
  const int f = slab * kStFeat + l16;        // weight row (N % 16 == 0)
  const long long row0 = static_cast<long long>(e) * N + f;
  // bytes: bf16 2 per weight, int8 1, 4-bit one half (a lane's 16 bytes of a block hold the
  // codes of its k = 32 c + 8 g runs, as packed by moe_quantize_groups_q4)
  // fragment-major: the wave's 16 rows are one run of 1024-byte chunks, one per load instruction
  // (WR per block), lane l's 16 bytes at 16 l in each: the same bytes as in the row-major layout
  const long long wofs = WFR ? (row0 >> 4) * 16 * (W4 ? K / 2 : (W8 ? K : 2 * K)) + 16 * lane
                             : (W4 ? row0 * (K / 2) + 16 * grp
                                   : (W8 ? row0 * K + kq : 2 * (row0 * K + kq)));
  const char* pg = static_cast<const char*>(W0) + wofs;
  const char* pu = GATEUP ? static_cast<const char*>(W1) + wofs : nullptr;
  float sg = 1.f, su = 1.f;
  if constexpr (W8) {
    sg = static_cast<const float*>(S0)[row0];
    if constexpr (GATEUP) su = static_cast<const float*>(S1)[row0];
  }
  // 4-bit: the (scale, bias) pairs of a block's two groups of 64, per row
  const uint32_t* qg = W4 ? static_cast<const uint32_t*>(S0) + row0 * (K / 64) : nullptr;
  const uint32_t* qu = (W4 && GATEUP) ? static_cast<const uint32_t*>(S1) + row0 * (K / 64) : nullptr;
  // lanes past a group's rows read row 0 of that group (never stored: row i of the product
  // depends only on A row i; the duplicate reads coalesce); a group past all rows repeats group 0
  const uint16_t* pa[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int gr = rows - 16 * g;           // rows of group g (may be <= 0 for NG > 1)
    const int li_a = m0 + (gr > 0 ? 16 * g + (l16 < gr ? l16 : 0) : 0);
    const long long arow = GATEUP ? lr[li_a] / k : (hbase >= 0 ? hbase + li_a : lr[li_a]);
    pa[g] = A + arow * K + kq;
  }
  const int nb = NB > 0 ? NB : K / 128;       // even: K % 256 == 0 on this path
  // the same for the whole wave; without the explicit broadcast the compiler keeps the rotated
  // block indices in vector registers and the kernel's register use doubles
  const int rot = __builtin_amdgcn_readfirstlane(((e * (N / kStFeat) + slab) * 5) % nb);

  u32x4 a[2][NG][4], bg[2][WR], bu[2][WR];     // two blocks in flight, slot = block % 2
  uint2 pgs[2], pus[2];                        // 4-bit: the block's (scale, bias) pairs
  auto load = [&](int j, int sq) {
    const int blk = (min(sq, nb - 1) + rot) % nb;  // past the end: re-read the last block
    const int kb = blk * 128;
#pragma unroll
    for (int c = 0; c < WR; ++c) {
      const int off = WFR ? 1024 * (WR * blk + c)
                          : (W4 ? 64 * blk : (W8 ? kb + 16 * c : 2 * (kb + 32 * c)));  // bytes
      bg[j][c] = load16(pg + off);
      if constexpr (GATEUP) bu[j][c] = load16(pu + off);
    }
    if constexpr (W4) {
      pgs[j] = *reinterpret_cast<const uint2*>(qg + 2 * blk);
      if constexpr (GATEUP) pus[j] = *reinterpret_cast<const uint2*>(qu + 2 * blk);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int g = 0; g < NG; ++g) a[j][g][c] = load16(pa[g] + kb + (W8 ? 8 * c : 32 * c));
  };
  auto wop = [&](const u32x4* b, int c, uint2 pr) -> u32x4 {
    if constexpr (W4) {
      return q4x8_dequant(b[0][c], c < 2 ? pr.x : pr.y);
    } else if constexpr (W8) {
      const u32x4 v = b[c >> 1];
      const uint32_t w0 = (c & 1) ? v[2] : v[0], w1 = (c & 1) ? v[3] : v[1];
      return GATEUP ? i8x8_to_bf16x8(w0, w1) : i8x8_to_f16x8(w0, w1);
    } else {
      return b[c];
    }
  };
  f32x4 accg[NG], accu[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    accg[g] = f32x4{0.f, 0.f, 0.f, 0.f};
    accu[g] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // h is fp16, so the down product runs on fp16 operands, its weights converted to fp16 (bf16
  // weights here, int8 codes in wop)
  constexpr bool kF16Down = !GATEUP;
  auto compute = [&](int j) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      u32x4 wg = wop(bg[j], c, pgs[j]);
      u32x4 wu = wg;
      if constexpr (GATEUP) wu = wop(bu[j], c, pus[j]);
      if constexpr (kF16Down && BASE == kWBf16) wg = bf16x8_to_f16x8(wg);
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        if constexpr (kF16Down) {
          accg[g] = mfma16x16x32_f16(a[j][g][c], wg, accg[g]);
        } else if constexpr (W4) {          // fp16 weights: the bf16 token rows go to fp16
          const u32x4 av = bf16x8_to_f16x8(a[j][g][c]);
          accg[g] = mfma16x16x32_f16(av, wg, accg[g]);
          accu[g] = mfma16x16x32_f16(av, wu, accu[g]);
        } else {
          accg[g] = mfma16x16x32(a[j][g][c], wg, accg[g]);
          if constexpr (GATEUP) accu[g] = mfma16x16x32(a[j][g][c], wu, accu[g]);
        }
      }
    }
  };
  load(0, 0);
  load(1, 1);
  // unrolled completely when NB is known: in straight-line code the compiler's wait counts leave
  // the next block in flight, while a loop back edge makes it wait for every outstanding load
  constexpr int kUnroll = NB > 0 ? NB / 2 : 1;
#pragma unroll kUnroll
  for (int sq = 0; sq < nb; sq += 2) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      // sched_barrier keeps the scheduler from sinking the prefetch below the next compute
      compute(j);
      __builtin_amdgcn_sched_barrier(0);
      load(j, sq + j + 2);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

#pragma unroll
  for (int g = 0; g < NG; ++g) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * g + (lane >> 4) * 4 + r;  // row of this pass
      if (i >= rows) continue;
      const int li = m0 + i;                     // entry of the expert's row list
      const int hrow = hbase >= 0 ? hbase + li : lr[li];
      if constexpr (GATEUP) {
        const float hv = silu(sg * accg[g][r]) * (su * accu[g][r]);
        h_out[static_cast<long long>(hrow) * N + f] = f32_to_f16_bits_sat(hv);
      } else {
        const DownRow dr = down_row(down, lr[li], hrow, N);
        down_put(down, dr, f, sg * accg[g][r]);
      }
    }
  }
}

// Grid (N / 16, E), one wave per block. Each block computes 16 features of one expert for all of
// the expert's rows, up to 16 MAXG rows per pass over the weights (a further pass mostly hits the
// caches). MAXG = 2 lets an expert with 17..32 rows, common under a selection bias, read its
// weights once, at the cost of registers (fewer resident waves). WF (WeightFormat): bf16 weights,
// row-major or fragment-major; int8 codes with fp32 row scales S0 (gate or down) and S1 (up); or
// packed 4-bit codes with (scale, bias) pairs S0 and S1.
// Block to (expert, slab): with fewer than kStCompactMinE experts, block (x, y) takes slab x of
// expert y. With more, most experts have no rows on a decode step, and a CU whose blocks all fell
// on routed experts carried about twice the average load and set the kernel's end (ZONOS3-Mini
// decode: the median wave ended ~15 us after the start, the last ~22 us). There the blocks are
// work items over the experts that have rows: item i = y (N / 16) + x takes slab i % (N / 16) of
// the (i / (N / 16))-th such expert, and items past the last one exit at once, so the active items
// sit at the start of the grid and spread evenly over the CUs (blocks are dispatched in order,
// round robin over the XCDs). Gate/up 21.3 -> 19.9 us on that workload; with 16 experts, all of
// them routed on a decode step, the extra count pass only cost time.
constexpr int kStCompactMinE = 32;

template <bool GATEUP, int MAXG, int WF>
__global__ __launch_bounds__(kWave) void ffn_stream_kernel(
    const uint16_t* __restrict__ A, const void* __restrict__ W0, const void* __restrict__ W1,
    const void* __restrict__ S0, const void* __restrict__ S1, int K, int N, int k,
    RowSource rs, uint16_t* __restrict__ h_out, DownArgs down) {
  __shared__ int lr[kMaxScanRows];
  __shared__ int cnt[kMaxE];
  const int lane = lane_id();
  const int E = gridDim.y;
  int e = blockIdx.y, slab = blockIdx.x;
  // with few ids the count pass keeps them in registers and the row scan reuses them (one read
  // of the ids per block instead of two)
  constexpr int kRegIds = 4;
  int idr[kRegIds];
  const bool ids_in_regs = E >= kStCompactMinE && rs.ids && rs.n_rows <= kRegIds * kWave;
  if (E >= kStCompactMinE) {
    const int slabs = gridDim.x;
    const int item = blockIdx.y * slabs + blockIdx.x;
    // rows per expert: from the ids (one LDS add per id) or from the dispatch offsets
    for (int i = lane; i < E; i += kWave) cnt[i] = rs.ids ? 0 : rs.offsets[i + 1] - rs.offsets[i];
    if (ids_in_regs) {
#pragma unroll
      for (int i = 0; i < kRegIds; ++i) {
        const int r = kWave * i + lane;
        idr[i] = r < rs.n_rows ? rs.ids[r] : -1;
      }
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int i = 0; i < kRegIds; ++i)
        if (kWave * i + lane < rs.n_rows) atomicAdd(&cnt[min(max(idr[i], 0), E - 1)], 1);
    } else if (rs.ids) {
      __builtin_amdgcn_wave_barrier();
      for (int r = lane; r < rs.n_rows; r += kWave)
        atomicAdd(&cnt[min(max(rs.ids[r], 0), E - 1)], 1);
    }
    __syncthreads();
    if (rs.counts_out && item < E && lane == 0) rs.counts_out[item] = cnt[item];
    // the (item / slabs)-th expert with rows
    int a = item / slabs;
    e = -1;
    for (int c0 = 0; c0 < E; c0 += kWave) {
      const unsigned long long m = __ballot(c0 + lane < E && cnt[c0 + lane] > 0);
      const int pc = __popcll(m);
      if (a < pc) {
        unsigned long long mm = m;
        for (int i = 0; i < a; ++i) mm &= mm - 1;     // drop the a lowest set bits
        e = c0 + __ffsll(static_cast<long long>(mm)) - 1;
        break;
      }
      a -= pc;
    }
    if (e < 0) return;                                // past the last expert with rows
    slab = item % slabs;
  }
  int count, hbase;
  if (rs.ids) {
    count = ids_in_regs ? scan_rows_regs(idr, e, lr) : scan_rows(rs.ids, rs.n_rows, e, lr);
    hbase = -1;
    if (E < kStCompactMinE && rs.counts_out && blockIdx.x == 0 && lane == 0)
      rs.counts_out[e] = count;
  } else {
    hbase = rs.offsets[e];
    count = rs.offsets[e + 1] - hbase;
    for (int i = threadIdx.x; i < count; i += blockDim.x) lr[i] = rs.sorted_rows[hbase + i];
    __syncthreads();
  }
  // passes of up to 16 MAXG rows: the 16-row groups of a pass share each weight load
  for (int m0 = 0; m0 < count; m0 += 16 * MAXG) {
    const int rows = min(16 * MAXG, count - m0);
    // the reduction loop fully unrolled for the expert widths of the two models (nb blocks of
    // 128)
    auto tile = [&](auto nb_const) {
      constexpr int NB = decltype(nb_const)::value;
      if (MAXG > 1 && rows > 16)
        stream_tile<GATEUP, MAXG, WF, NB>(A, W0, W1, S0, S1, K, N, k, e, slab, lr, m0, rows,
                                          hbase, h_out, down);
      else
        stream_tile<GATEUP, 1, WF, NB>(A, W0, W1, S0, S1, K, N, k, e, slab, lr, m0, rows, hbase,
                                       h_out, down);
    };
    switch (K) {
      case 512: tile(std::integral_constant<int, 4>{}); break;
      case 1024: tile(std::integral_constant<int, 8>{}); break;
      case 2048: tile(std::integral_constant<int, 16>{}); break;
      case 2816: tile(std::integral_constant<int, 22>{}); break;
      default: tile(std::integral_constant<int, 0>{}); break;
    }
  }
}

}  // namespace

// Prefill tile configurations, chosen from the shape (eight or sixteen waves of 64 x 64, 3-slot
// rings of 32-wide K steps at two blocks per CU unless stated otherwise; XCD-aware tile order):
//  * fewer rows than a full 256-row tile per expert on average (zonos3mini prefill): 128 x 256
//    tiles for both products (gate/up: 128 gate + 128 up features). Against
//    256 x 128 tiles the grid shrinks from 632 to ~440 blocks (one round of the block slots),
//    small experts pad half as many rows, and each weight fragment of the down product is
//    converted to fp16 by two waves instead of four: gate/up 55 -> 48 us, down 55 -> 47 us.
//  * a full row tile per expert or more (zonos2 skewed prefill): gate/up on
//    256 x 256 tiles with 64-wide K steps in a 2-slot ring (128 KB, one block per CU): 128-byte row
//    segments copy from L2 at twice the rate of 64-byte ones and the wider tile copies a third
//    less per product (gate/up 215 against 233 us). The down product keeps 256 x 128 tiles
//    (128 x 256: 185 against 166 us; 256 x 256 with one block per CU: 159 against 152 us).
// Also measured slower on the skewed prefill: waves of 128 x 64 or 32 x 64, deeper rings, and
// 64-wide K steps at 256 x 128 (one block per CU).
constexpr int kTileM = 256;
constexpr int kTileWaveRows = 64;

bool ffn_bf16_streaming(int T, int d, int E, int H, int k) {
  const long long rows = static_cast<long long>(T) * k;
  return rows <= kMaxScanRows && d % 256 == 0 && H % 256 == 0 && rows <= 32ll * E;
}

namespace {

// Gate/up and down weight-streaming launches for one weight format. Two-group passes where every
// block of the grid stays resident at their lower occupancy (gate/up: at most 2048 blocks;
// down: at most 4096).
template <int WF>
hipError_t launch_streaming(const uint16_t* x, const void* wg, const void* wu, const void* wd,
                            int d, int E, int H, int k, const RowSource& rs, uint16_t* h,
                            const DownArgs& down, hipStream_t s, const StageMarks& gu,
                            const QuantWeights& qw) {
  const DownArgs none{};
  const dim3 g_gu(H / kStFeat, E), g_dn(d / kStFeat, E);
  const bool g2 = (H / kStFeat) * E <= 2048;
  const hipError_t err =
      g2 ? launch_marked(ffn_stream_kernel<true, 2, WF>, g_gu, dim3(kWave), s, gu, x, wg, wu,
                         qw.gate, qw.up, d, H, k, rs, h, none)
         : launch_marked(ffn_stream_kernel<true, 1, WF>, g_gu, dim3(kWave), s, gu, x, wg, wu,
                         qw.gate, qw.up, d, H, k, rs, h, none);
  if (err != hipSuccess) return err;
  RowSource rs2 = rs;
  rs2.counts_out = nullptr;
  if ((d / kStFeat) * E <= 4096)
    ffn_stream_kernel<false, 2, WF><<<g_dn, kWave, 0, s>>>(h, wd, nullptr, qw.down, nullptr, H, d,
                                                           k, rs2, nullptr, down);
  else
    ffn_stream_kernel<false, 1, WF><<<g_dn, kWave, 0, s>>>(h, wd, nullptr, qw.down, nullptr, H, d,
                                                           k, rs2, nullptr, down);
  return hipGetLastError();
}

// One grouped-GEMM launch: BM x BN tiles (gate/up: BN / 2 gate and BN / 2 up features) with
// BK-wide K steps in a RING-slot ring, 64 x 64 waves.
template <bool GATEUP, int BM, int BN, int RING, int BK>
hipError_t launch_gemm(int rows, int E, hipStream_t s, const StageMarks& marks,
                       const uint16_t* A, const void* W0, const void* W1, int K, int N, int k,
                       const RowSource& rs, uint16_t* h, const DownArgs& down, bool bfrag) {
  constexpr int NT = BM / kTileWaveRows * (BN / 64) * kWave;
  constexpr int FEAT = GATEUP ? BN / 2 : BN;
  const int ntn = (N + FEAT - 1) / FEAT;
  const long long grid = prefill_grid(max_tiles(rows, E, BM), ntn);
  if (bfrag)
    return launch_marked(gemm_dma_kernel<GATEUP, BM, BN, RING, kTileWaveRows, BK, true>,
                         dim3(static_cast<unsigned>(grid)), dim3(NT), s, marks, A,
                         static_cast<const uint16_t*>(W0), static_cast<const uint16_t*>(W1), K,
                         N, E, k, rs.offsets, rs.sorted_rows, h, down);
  return launch_marked(gemm_dma_kernel<GATEUP, BM, BN, RING, kTileWaveRows, BK, false>,
                       dim3(static_cast<unsigned>(grid)), dim3(NT), s, marks, A,
                       static_cast<const uint16_t*>(W0), static_cast<const uint16_t*>(W1), K, N,
                       E, k, rs.offsets, rs.sorted_rows, h, down);
}

}  // namespace

hipError_t launch_ffn_bf16(const uint16_t* x, const void* wg, const void* wu, const void* wd,
                           int T, int d, int E, int H, int k, const RowSource& rs, uint16_t* h,
                           const DownArgs& down, hipStream_t s, const StageMarks& gu,
                           const QuantWeights& qw) {
  const int rows = T * k;
  if (rows <= 0) return hipSuccess;
  DownArgs none{};
  hipError_t err;
  if (ffn_bf16_streaming(T, d, E, H, k)) {
    switch (qw.fmt) {
      case kWBf16: return launch_streaming<kWBf16>(x, wg, wu, wd, d, E, H, k, rs, h, down, s, gu, qw);
      case kWI8: return launch_streaming<kWI8>(x, wg, wu, wd, d, E, H, k, rs, h, down, s, gu, qw);
      case kWQ4: return launch_streaming<kWQ4>(x, wg, wu, wd, d, E, H, k, rs, h, down, s, gu, qw);
      case kWBf16 | kWFragMajor:
        return launch_streaming<kWBf16 | kWFragMajor>(x, wg, wu, wd, d, E, H, k, rs, h, down, s,
                                                      gu, qw);
      case kWI8 | kWFragMajor:
        return launch_streaming<kWI8 | kWFragMajor>(x, wg, wu, wd, d, E, H, k, rs, h, down, s, gu,
                                                    qw);
      case kWQ4 | kWFragMajor:
        return launch_streaming<kWQ4 | kWFragMajor>(x, wg, wu, wd, d, E, H, k, rs, h, down, s, gu,
                                                    qw);
      default: return hipErrorInvalidValue;
    }
  }
  // quantised weights: weight-streaming shapes only (checked by the callers); bf16 weights
  // row-major or fragment-major
  if (qw.fmt != kWBf16 && qw.fmt != (kWBf16 | kWFragMajor)) return hipErrorInvalidValue;
  const bool bfrag = qw.fmt != kWBf16;
  // grouped GEMM over the dispatch order; 1-D grids sized for the worst-case tile count
  const StageMarks no_marks{};
  if (prefill_wide_tiles(rows, E, kTileM)) {
    err = launch_gemm<true, 256, 256, 2, 64>(rows, E, s, gu, x, wg, wu, d, H, k, rs, h, none,
                                             bfrag);
    if (err != hipSuccess) return err;
    return launch_gemm<false, 256, 128, 3, 32>(rows, E, s, no_marks, h, wd, nullptr, H, d, k, rs,
                                               nullptr, down, bfrag);
  }
  err = launch_gemm<true, 128, 256, 3, 32>(rows, E, s, gu, x, wg, wu, d, H, k, rs, h, none,
                                           bfrag);
  if (err != hipSuccess) return err;
  return launch_gemm<false, 128, 256, 3, 32>(rows, E, s, no_marks, h, wd, nullptr, H, d, k, rs,
                                             nullptr, down, bfrag);
}

}  // namespace moe
