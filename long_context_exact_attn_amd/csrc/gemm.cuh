// bfloat16 GEMM on the matrix cores of gfx950 for the blockwise feed-forward: C = A B with float32
// accumulation (v_mfma_f32_32x32x16_bf16) and an epilogue chosen at compile time.
//
// Workgroup tile BM x BN = 256 x 256, eight waves in a 2 x 4 grid (two per SIMD), each wave 128 x 64
// (4 x 2 blocks of 32 x 32: 128 accumulator registers).  K advances BK = 64 at a time through a
// two-stage LDS ring (128 KiB) filled by direct global -> LDS copies one tile ahead.  Either operand
// may be stored with K contiguous ("K-major": A as [M][K], B as [N][K]) or with M / N contiguous
// ([K][M], [K][N]); K-major tiles are read with 16-byte LDS reads, the others with transposing reads,
// both giving the operand in the MFMA's natural k order.
//
// Copies: every lane's byte offset inside a tile is fixed for the whole kernel, and each copy
// instruction takes a wave-uniform base (the instruction's saddr form), so interior tiles cost no
// vector address arithmetic.  Tiles that reach past the matrix (ragged M, N or K) take a checked
// path in which chunks outside the matrix are copied from a zero chunk.  The contiguous dimension of
// every operand must be a multiple of 8 (so a 16-byte chunk is wholly inside or outside).
#pragma once

#include "mfma_util.cuh"

namespace ra {
namespace gemm {

#ifndef RA_GEMM_BK
#define RA_GEMM_BK 64
#endif
#ifndef RA_GEMM_NS
#define RA_GEMM_NS 2
#endif
constexpr int BM = 256, BN = 256, BK = RA_GEMM_BK, NS = RA_GEMM_NS;
static_assert(BK == 32 || BK == 64, "k tile of 32 or 64");
constexpr int kWavesG = 8;
constexpr int kThreadsG = 64 * kWavesG;

// 16 zero bytes: the source of every copy chunk that lies outside its matrix
__device__ __attribute__((aligned(16))) const __bf16 kZeroChunk[8] = {};

// Operand description: element (r, k) of the operand (r = row of A or column of B) lives at
// base[r * ld + k] when stored K-major, else at base[k * ld + r].  For a K-major operand, rows at or
// past `split` come from base2 (row r - split); for the other layout, k rows at or past `split` do
// (this is how [W1; W3] is used without stacking it).  rows / kdim bound the valid region.
struct Operand {
  const __bf16* base;
  const __bf16* base2;
  int64_t ld;
  int64_t split;   // INT64_MAX: none
  int64_t rows, kdim;
};

// ---- LDS layouts (element offsets).  K-major tile: rows of BK = 64 elements (8 chunks of 16 bytes),
// chunk c of row r stored at chunk position c ^ ((r >> 1) & 7): the 16 rows a 16-byte read serves in
// one pass cover the 64 banks once (two rows share a 256-byte bank period).  Transposed tile: BK rows
// of W elements, chunk c of row k stored at c ^ (4 (k & 3)): the 4 rows x 4 chunks a transposing
// read serves per pass cover the banks once too.
// (BK = 32: rows of 64 bytes, four per period, key (r >> 2) & 3)
__device__ __forceinline__ int kmaj_key(int r) { return BK == 64 ? ((r >> 1) & 7) : ((r >> 2) & 3); }
__device__ __forceinline__ int kmaj_off(int r, int c) { return r * BK + ((c ^ kmaj_key(r)) << 3); }
template <int W>
__device__ __forceinline__ int tr_off(int k, int c) { return k * W + ((c ^ (4 * (k & 3))) << 3); }

// operand fragment for k-step kk of a K-major tile: lane l gets X[r0 + l % 32][16 kk + 8 (l / 32) + 0..7]
__device__ __forceinline__ bf16x8 frag_kmaj(const __bf16* t, int r0, int kk, int lane) {
  return *reinterpret_cast<const bf16x8*>(t + kmaj_off(r0 + (lane & 31), 2 * kk + (lane >> 5)));
}

// the same from a transposed tile (rows = k, W elements each), by two transposing reads: within a
// 16-lane group lane j receives element j % 4 of the 4-element pieces that lanes 4 e + j / 4 address,
// so lane 4 e + j' addresses row 8 (l / 32) + e (+ 4 for the second read) at column 16 (g & 1) + 4 j'.
template <int W>
__device__ __forceinline__ bf16x8 frag_tr(const __bf16* t, int r0, int kk, int lane) {
  const int g = lane >> 4, gi = lane & 15, hh = lane >> 5;
  const int k = 16 * kk + 8 * hh + (gi >> 2);
  const int col = r0 + 16 * (g & 1) + 4 * (gi & 3);
  const int c = col >> 3, within = col & 7;
  const i16x4 lo = lds_read_tr(t + tr_off<W>(k, c) + within);
  const i16x4 hi = lds_read_tr(t + tr_off<W>(k + 4, c) + within);
  bf16x8 a;
  __builtin_memcpy(&a, &lo, 8);
  __builtin_memcpy(reinterpret_cast<char*>(&a) + 8, &hi, 8);
  return a;
}

// B-row maps: the operand row of row r (0..BN-1) of the workgroup's B tile that starts at column n0.
// A map must be affine with slope 1 within each aligned group of 16 rows (one copy instruction's).
struct LinearRows {
  __device__ int64_t operator()(int64_t n0, int r) const { return n0 + r; }
};

// The copy schedule of one operand tile (R operand rows x BK): the chunk at LDS chunk position
// p = (wave * PER + i) * 64 + lane holds logical chunk (row, k) of the operand.
template <bool KMAJ, int R>
struct TileCopy {
  static constexpr int CHUNKS = R * BK / 8;
  static constexpr int PER = CHUNKS / kThreadsG;
  static_assert(PER * kThreadsG == CHUNKS, "tile must split evenly over the workgroup");
  static constexpr int CPR = KMAJ ? BK / 8 : R / 8;   // chunks per LDS row
  static_assert(KMAJ ? (64 % CPR == 0) : (CPR % 64 == 0 || 64 % CPR == 0), "whole rows per instruction");
  // the tile-relative (row, k) of the chunk at position p
  __device__ static void at(int p, int& row, int& k) {
    if constexpr (KMAJ) {
      const int r = p / CPR, slot = p % CPR;
      row = r;
      k = 8 * (slot ^ kmaj_key(r));
    } else {
      const int kr = p / CPR, slot = p % CPR;
      k = kr;
      row = 8 * (slot ^ (4 * (kr & 3)));
    }
  }
};

// each lane's fixed byte offsets of the fast path: its chunk of instruction i relative to the
// instruction's uniform base (its first row, or its first k row)
template <bool KMAJ, int R, typename RowMap>
__device__ __forceinline__ void copy_offsets(const Operand& o, int wave, int lane, RowMap rowmap,
                                             unsigned (&off)[TileCopy<KMAJ, R>::PER]) {
  using TC = TileCopy<KMAJ, R>;
#pragma unroll
  for (int i = 0; i < TC::PER; ++i) {
    const int p0 = (wave * TC::PER + i) * 64;
    int r0, kq, r, k;
    TC::at(p0, r0, kq);
    TC::at(p0 + lane, r, k);
    int64_t e;
    if constexpr (KMAJ) {
      e = (rowmap(r) - rowmap(r0)) * o.ld + k;
    } else {
      e = static_cast<int64_t>(k - kq) * o.ld + (rowmap(r) - rowmap(0));
    }
    off[i] = static_cast<unsigned>(2 * e);
  }
}

// Copies of the tile at k0 into dst.  fast (the whole tile lies inside the operand and this split's K
// range): per-lane constant offsets from a wave-uniform base.  Otherwise each chunk is checked, and a
// chunk outside comes from the zero chunk.  rowmap: tile row -> operand row.
template <bool KMAJ, int R, typename RowMap>
__device__ __forceinline__ void copy_tile(const Operand& o, int64_t k0, int64_t kend, __bf16* dst, int wave, int lane,
                                          const unsigned (&off)[TileCopy<KMAJ, R>::PER], bool fast, RowMap rowmap) {
  using TC = TileCopy<KMAJ, R>;
#pragma unroll
  for (int i = 0; i < TC::PER; ++i) {
    __bf16* d = dst + (wave * TC::PER + i) * 512;
    const int p0 = (wave * TC::PER + i) * 64;   // the instruction's first chunk (wave-uniform)
    int r0, kq;
    TC::at(p0, r0, kq);
    if (fast) {
      const __bf16* base;
      if constexpr (KMAJ) {
        const int64_t row = rowmap(r0);
        base = row < o.split ? o.base + row * o.ld + k0 : o.base2 + (row - o.split) * o.ld + k0;
      } else {
        const int64_t k = k0 + kq;
        const int64_t row = rowmap(0);
        base = k < o.split ? o.base + k * o.ld + row : o.base2 + (k - o.split) * o.ld + row;
      }
      dma16_sb(base, off[i], d);
    } else {
      int r, kk;
      TC::at(p0 + lane, r, kk);
      const int64_t row = rowmap(r), k = k0 + kk;
      const bool ok = row < o.rows && k < kend;
      const __bf16* b;
      int64_t e;
      if constexpr (KMAJ) {
        b = row < o.split ? o.base : o.base2;
        e = (row < o.split ? row : row - o.split) * o.ld + k;
      } else {
        b = k < o.split ? o.base : o.base2;
        e = (k < o.split ? k : k - o.split) * o.ld + row;
      }
      dma16(ok ? b + e : kZeroChunk, d);
    }
  }
}

// Epilogue interface: epi(acc, mb0, nb0, split, l32, hh, M, N) is called once per wave with its tile,
//   acc[a][b][4 g + e] = C[mb0 + 32 a + l32][nb0 + 32 b + 8 g + 4 hh + e]    (g, e = 0..3)
// The products take B's fragment as their first operand, which gives the transposed accumulator
// layout: each lane holds four consecutive columns of one row, so an epilogue stores four elements
// per instruction (the operand fragments of a 32 x 32 x 16 product have the same form on both sides).
// b_valid: the B tile is inside its operand when n0 + BN <= b_valid.
template <bool A_KMAJ, bool B_KMAJ, typename BRowMap, typename Epi>
__global__ __launch_bounds__(kThreadsG) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_kernel(
    Operand A, Operand B, int64_t M, int64_t N, int64_t K, int tiles_m, int tiles_n, int splits, int64_t k_per_split,
    int64_t b_valid, BRowMap browmap, Epi epi) {
  __shared__ __attribute__((aligned(16))) __bf16 sA[NS][BM * BK];
  __shared__ __attribute__((aligned(16))) __bf16 sB[NS][BN * BK];
  using TA = TileCopy<A_KMAJ, BM>;
  using TB = TileCopy<B_KMAJ, BN>;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int wm = wave >> 2, wn = wave & 3;

  // workgroup -> tile: consecutive workgroups go to different XCDs, so each XCD gets a contiguous
  // range of tiles.  Inside it the tiles go in groups of GM tile rows, the row fastest: the 32
  // workgroups an XCD runs at once cover about 8 x 4 tiles and share 8 A and 4 B panels in that
  // XCD's L2 (one tile column at a time would need 32 A panels per k step).
  constexpr int GM = 8;
  const int total = tiles_m * tiles_n * splits;
  const int w = blockIdx.x, x = w & 7, i = w >> 3;
  const int q = total >> 3, rr = total & 7;
  const int t = x * q + (x < rr ? x : rr) + i;
  const int split = t / (tiles_m * tiles_n);
  const int tt = t % (tiles_m * tiles_n);
  const int group = tt / (GM * tiles_n);
  const int first_m = group * GM;
  const int gm = tiles_m - first_m < GM ? tiles_m - first_m : GM;   // rows in this (possibly last) group
  const int rg = tt - group * GM * tiles_n;
  const int tm = first_m + rg % gm, tn = rg / gm;
  const int64_t m0 = static_cast<int64_t>(tm) * BM, n0 = static_cast<int64_t>(tn) * BN;
  const int64_t kbeg = static_cast<int64_t>(split) * k_per_split;
  const int64_t kend = kbeg + k_per_split < K ? kbeg + k_per_split : K;
  const int nk = kend > kbeg ? static_cast<int>((kend - kbeg + BK - 1) / BK) : 0;

  auto arow = [m0](int r) -> int64_t { return m0 + r; };
  auto brow = [&browmap, n0](int r) -> int64_t { return browmap(n0, r); };
  unsigned offA[TA::PER], offB[TB::PER];
  copy_offsets<A_KMAJ, BM>(A, wave, lane, arow, offA);
  copy_offsets<B_KMAJ, BN>(B, wave, lane, brow, offB);
  const bool rows_in = m0 + BM <= A.rows && n0 + BN <= b_valid;

  f32x16 acc[4][2];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x16{};

  // one wave-uniform branch per tile between the all-fast and the checked copies: with the choice made
  // inside the unrolled per-copy loop the compiler kept a pair of branches around every copy
  auto issue = [&](int kt, int slot) {
    const int64_t k0 = kbeg + static_cast<int64_t>(kt) * BK;
    if (rows_in && k0 + BK <= kend) {
      copy_tile<A_KMAJ, BM>(A, k0, kend, sA[slot], wave, lane, offA, true, arow);
      copy_tile<B_KMAJ, BN>(B, k0, kend, sB[slot], wave, lane, offB, true, brow);
    } else {
      copy_tile<A_KMAJ, BM>(A, k0, kend, sA[slot], wave, lane, offA, false, arow);
      copy_tile<B_KMAJ, BN>(B, k0, kend, sB[slot], wave, lane, offB, false, brow);
    }
  };

  constexpr int PER_TILE = TA::PER + TB::PER;   // copies per lane and tile
#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < nk) issue(s, s);
  RA_WAIT_VMCNT(0);
  __syncthreads();

  int slot = 0;
  for (int kt = 0; kt < nk; ++kt) {
    const bool more = kt + NS - 1 < nk;
    if (more) issue(kt + NS - 1, slot == 0 ? NS - 1 : slot - 1);
    const __bf16* ta = sA[slot];
    const __bf16* tb = sB[slot];
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8 af[4], bf[2];
#pragma unroll
      for (int a = 0; a < 4; ++a)
        af[a] = A_KMAJ ? frag_kmaj(ta, 128 * wm + 32 * a, kk, lane) : frag_tr<BM>(ta, 128 * wm + 32 * a, kk, lane);
#pragma unroll
      for (int b = 0; b < 2; ++b)
        bf[b] = B_KMAJ ? frag_kmaj(tb, 64 * wn + 32 * b, kk, lane) : frag_tr<BN>(tb, 64 * wn + 32 * b, kk, lane);
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = mfma32(bf[b], af[a], acc[a][b]);
    }
    // the next tile's copies must have landed before anyone reads them (those issued in this iteration
    // may stay in flight), and every wave must be done with this tile's stage before copies overwrite it
    if (more) {
      RA_WAIT_VMCNT((NS - 2) * PER_TILE);
    } else {
      RA_WAIT_VMCNT(0);
    }
    __syncthreads();
    slot = slot + 1 == NS ? 0 : slot + 1;
  }

  epi(acc, m0 + 128 * wm, n0 + 64 * wn, split, l32, hh, M, N);
}

}  // namespace gemm
}  // namespace ra
