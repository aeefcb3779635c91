// LDS access helpers shared by the MFMA kernels (gfx950, wave64).
//
// Operand layouts of v_mfma_f32_32x32x16_bf16 (C = A.B + C, A 32x16, B 16x32):
//   A: lane l holds A[l % 32][8 * (l / 32) + 0..7]
//   B: lane l holds B[8 * (l / 32) + 0..7][l % 32]
//   C: lane l holds C[8 * (v / 4) + 4 * (l / 32) + (v % 4)][l % 32], v = 0..15
// so a row-major tile read 16 bytes per lane (row = lane % 32) serves as A or
// as B alike, and a C accumulator feeds the next product as B with its 16
// values split into two k-steps of 8 (v = 0..7 and 8..15).  The k index of
// those steps is then the permuted row order {4h + 0..3, 8 + 4h + 0..3} + 16 st
// (h = l / 32); the matching A operand is read from LDS with the transposing
// read below, which produces exactly that order.
#pragma once

#include "ra_common.cuh"

namespace ra {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;

__device__ __forceinline__ bf16x8 lds_read_b128(const __bf16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

// Transposed read: within each 16-lane group, lane j receives element (j % 4) of
// the 4-element chunks addressed by lanes 4e + j/4 for e = 0..3.
__device__ __forceinline__ i16x4 lds_read_tr(const __bf16* p) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

// A operand holding the transpose of a row-major LDS tile X (rows = the k index
// of the product, columns = the A rows): lane l gets
//   A[l % 32][i] = X[r0 + 16 st + 4 (l / 32) + i][c0 + l % 32]        i = 0..3
//   A[l % 32][i] = X[r0 + 16 st + 8 + 4 (l / 32) + i - 4][c0 + l % 32] i = 4..7
// i.e. the k order of a C accumulator's k-step st (see above).  SROW is the
// tile's row stride in elements.
template <int SROW>
__device__ __forceinline__ bf16x8 lds_read_a_transposed(const __bf16* tile, int r0, int st, int c0, int lane) {
  const int g = lane >> 4, gi = lane & 15, hh = lane >> 5;
  const int row = r0 + st * 16 + 4 * hh + (gi >> 2);
  const int col = c0 + 16 * (g & 1) + 4 * (gi & 3);
  const i16x4 lo = lds_read_tr(tile + row * SROW + col);
  const i16x4 hi = lds_read_tr(tile + (row + 8) * SROW + col);
  bf16x8 a;
  __builtin_memcpy(&a, &lo, 8);
  __builtin_memcpy(reinterpret_cast<char*>(&a) + 8, &hi, 8);
  return a;
}

// ---- swizzled unpadded tiles.  A row of D bf16 holds D / 8 chunks of 16 bytes, and
// chunk c of row r is stored at chunk position c ^ swz_key<D>(r).  gfx950's LDS has 64
// banks of 4 bytes (256 bytes per cycle), so
//   - a 16-byte operand read (lds_read_swz) is served 16 lanes at a time: 16 consecutive
//     rows (aligned to 16), one chunk each;
//   - a transposing 8-byte read is served 32 lanes at a time: 4 consecutive rows (aligned to
//     4), 4 consecutive chunks (aligned to 4), both halves of each.
// Each group must cover the 256-byte bank period exactly once.  At D = 64 two rows share a
// period (row parity picks the half), so the key must map the 8 rows of one parity among 16
// to 8 distinct values and give rows r and r + 2 of an aligned 4 different bit 2: key = (bit 1,
// bit 2, bit 3) of r.  At D = 128 a row fills the period, so the key must be a bijection over 16
// rows whose bits 3..2 differ within an aligned 4: key = (bits 1..0, bits 3..2) of r.
// (r & 7, the usual key for 32 banks, leaves every such read two-way conflicted here.)  Direct global -> LDS copies write 16 consecutive bytes
// per lane and fetch the global chunk that belongs there, so they are conflict-free for any key.
template <int D>
__device__ __forceinline__ int swz_key(int row) {
  static_assert(D == 64 || D == 128, "head_dim 64 or 128");
  if constexpr (D == 64) return (((row >> 1) & 1) << 2) | (((row >> 2) & 1) << 1) | ((row >> 3) & 1);
  else return ((row & 3) << 2) | ((row >> 2) & 3);
}

template <int D>
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * D + ((chunk ^ swz_key<D>(row)) << 3);
}

// 16-byte operand read of row `row`, chunk `chunk` of a swizzled tile.
template <int D>
__device__ __forceinline__ bf16x8 lds_read_swz(const __bf16* tile, int row, int chunk) {
  return *reinterpret_cast<const bf16x8*>(tile + swz<D>(row, chunk));
}

// lds_read_a_transposed for a swizzled tile (same result layout).
template <int D>
__device__ __forceinline__ bf16x8 lds_read_a_transposed_swz(const __bf16* tile, int r0, int st, int c0, int lane) {
  const int g = lane >> 4, gi = lane & 15, hh = lane >> 5;
  const int row = r0 + st * 16 + 4 * hh + (gi >> 2);
  const int col = c0 + 16 * (g & 1) + 4 * (gi & 3);      // element column; 4 elements = 8 bytes
  const int within = col & 7;                             // 0 or 4
  const i16x4 lo = lds_read_tr(tile + swz<D>(row, col >> 3) + within);
  const i16x4 hi = lds_read_tr(tile + swz<D>(row + 8, col >> 3) + within);
  bf16x8 a;
  __builtin_memcpy(&a, &lo, 8);
  __builtin_memcpy(reinterpret_cast<char*>(&a) + 8, &hi, 8);
  return a;
}

// Direct global -> LDS copy of 16 bytes per lane: lane l's bytes land at lds + 16 l
// (lds must be wave-uniform).  Completion is counted by vmcnt only, and the copy is
// issued through inline assembly so that the compiler does not treat it as an LDS
// store: it would otherwise wait for every copy in flight before any LDS read and at
// every barrier.  Callers wait with RA_WAIT_VMCNT and a barrier before the data is read.
// The copy's LDS address goes through M0, which the statement writes and declares clobbered.  The
// compiler treats M0 as reserved and would not restore a value of its own there; these kernels rely
// on it keeping none (tests/test_device_asm.py checks the generated code for any other M0 use).
__device__ __forceinline__ void dma16(const void* g, __bf16* lds) {
  const unsigned dst = static_cast<unsigned>(
      reinterpret_cast<size_t>((__attribute__((address_space(3))) void*)lds));
  // (one wait state between the M0 write and the copy that reads it)
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" : : "s"(dst), "v"(g) : "memory", "m0");
}

// The same copy from a wave-uniform base address held in SGPRs plus a 32-bit per-lane byte
// offset (the instruction's saddr form): the per-lane part stays loop-invariant, so a tile's
// copies need no 64-bit address arithmetic on the vector unit.
// (base must be wave-uniform; the compiler cannot always prove it, so it is read from lane 0,
// which folds away where the value already sits in SGPRs)
__device__ __forceinline__ void dma16_sb(const void* base, unsigned off_bytes, __bf16* lds) {
  const unsigned dst = static_cast<unsigned>(
      reinterpret_cast<size_t>((__attribute__((address_space(3))) void*)lds));
  const unsigned long long a = reinterpret_cast<unsigned long long>(base);
  const unsigned lo = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(a));
  const unsigned hi = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(a >> 32));
  const unsigned long long sbase = (static_cast<unsigned long long>(hi) << 32) | lo;
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" : : "s"(dst), "v"(off_bytes), "s"(sbase)
               : "memory", "m0");
}

// s_waitcnt vmcnt(N) leaving the other counters unconstrained (gfx9 encoding).
#define RA_WAIT_VMCNT(N) __builtin_amdgcn_s_waitcnt(((N) & 15) | (((N) >> 4) << 14) | (7 << 4) | (15 << 8))

// Pack values v = 8 st .. 8 st + 7 of a C accumulator (already in float) as a
// bf16 B operand (round to nearest even).
__device__ __forceinline__ bf16x8 pack_bf16x8(const float* e) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16x2 pr = __builtin_convertvector((f32x2){e[2 * i], e[2 * i + 1]}, bf16x2);
    r[2 * i] = pr[0];
    r[2 * i + 1] = pr[1];
  }
  return r;
}

// c * x for eight bfloat16 values, rounded to nearest even: folds a constant factor
// into an operand that stays in registers.
__device__ __forceinline__ bf16x8 scale_bf16x8(bf16x8 x, float c) {
  float e[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) e[i] = c * static_cast<float>(x[i]);
  return pack_bf16x8(e);
}

// Reductions over the lane pair (l, l ^ 32) that shares one column of a C
// accumulator: v_permlane32_swap exchanges the two halves of the wave, and
// both results of the swap hold one value of each pair.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Minimum / maximum over the 64 lanes of a wave (result in every lane).
__device__ __forceinline__ int wave_min_i32(int x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = min(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ int wave_max_i32(int x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = max(x, __shfl_xor(x, o));
  return x;
}

// Smallest and largest id over the workgroup (each lane passes the range of its own ids,
// INT32_MAX / INT32_MIN for none); every wave gets the same result.  Contains a barrier.
template <int NW>
__device__ __forceinline__ void wg_id_range(int lo, int hi, int (&s)[NW][2], int wave, int lane, int& glo, int& ghi) {
  lo = wave_min_i32(lo);
  hi = wave_max_i32(hi);
  if (lane == 0) {
    s[wave][0] = lo;
    s[wave][1] = hi;
  }
  __syncthreads();
  glo = s[0][0];
  ghi = s[0][1];
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    glo = min(glo, s[w][0]);
    ghi = max(ghi, s[w][1]);
  }
}

// Tile filter for segment ids: bit t of the result is set iff some position q in
// [start + 64 t, start + 64 t + 64) with q < end has lo <= ids[q] <= hi.  Each of the 64
// tiles costs one coalesced load of 64 ids and one ballot; the result is wave-uniform.
__device__ __forceinline__ uint64_t seg_window_mask(const int* __restrict__ ids, int start, int end, int lo, int hi,
                                                    int lane) {
  constexpr int STEP = 32;   // loads issued before their ballots (two round trips per window)
  uint64_t m = 0;
#pragma unroll
  for (int g = 0; g < 64; g += STEP) {
    int id[STEP];
#pragma unroll
    for (int i = 0; i < STEP; ++i) {
      const int q = start + (g + i) * 64 + lane;
      id[i] = q < end ? ids[q] : 0;
    }
#pragma unroll
    for (int i = 0; i < STEP; ++i) {
      const bool inside = start + (g + i) * 64 + lane < end;
      if (__ballot(inside && id[i] >= lo && id[i] <= hi) != 0) m |= uint64_t(1) << (g + i);
    }
  }
  return m;
}

// Lookahead filter over a tile walk (tiles of 64 positions): passes over the tiles whose
// bit is clear.  The window [win, wend) of at most 64 tiles never extends past the end of
// the block or rank it was scanned in, so a window scanned for one block is never used
// for another.
struct SegTileFilter {
  uint64_t mask = 0;
  int win = 0, wend = 0;
  // pos: first position of the walk's current tile; end: end of its block; ids: id of
  // position q at ids[q].  Returns 0 if the tile is to be visited, else how many tiles to
  // advance (past the window when none of its remaining tiles matches).
  __device__ __forceinline__ int skip(const int* __restrict__ ids, int pos, int end, int lo, int hi, int lane) {
    if (pos < win || pos >= wend) {
      win = pos;
      wend = min(pos + 64 * 64, end);
      mask = seg_window_mask(ids, pos, end, lo, hi, lane);
    }
    const int bit = (pos - win) >> 6;
    const uint64_t rest = mask >> bit;
    if (rest & 1) return 0;
    return rest ? __builtin_ctzll(rest) : 64 - bit;
  }
};

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Host side of the backward launchers: calls CALL(causal mode, has bias, has segment ids) with the
// template flags that match the parameters.
#define RA_SELECT_FLAGS(CALL)                                                      \
  do {                                                                             \
    const bool b_ = p.bias != nullptr, s_ = p.seg != nullptr;                     \
    if (p.causal == 1) {                                                           \
      if (b_) { if (s_) CALL(1, true, true); else CALL(1, true, false); }          \
      else { if (s_) CALL(1, false, true); else CALL(1, false, false); }           \
    } else if (p.causal > 1) {                                                     \
      if (b_) { if (s_) CALL(2, true, true); else CALL(2, true, false); }          \
      else { if (s_) CALL(2, false, true); else CALL(2, false, false); }           \
    } else {                                                                       \
      if (b_) { if (s_) CALL(0, true, true); else CALL(0, true, false); }          \
      else { if (s_) CALL(0, false, true); else CALL(0, false, false); }           \
    }                                                                              \
  } while (0)

}  // namespace ra
