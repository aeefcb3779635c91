// Forward blockwise ring attention, bfloat16 in / float32 accumulate, MFMA on gfx950.
//
// One workgroup = 4 wavefronts = one query tile of BQ = 4 * 32 * NQB rows of one
// (batch, head); the tile stays resident (Q in VGPRs) while the K/V tiles of the
// ring walk stream through LDS: direct global -> LDS copies into a ring of stages,
// issued ahead of use (no staging registers).  Per K/V tile of BK = 64 keys each
// wave computes
//   S^T = K . Q^T           v_mfma_f32_32x32x16_bf16, rows = keys, columns = queries
//   online-softmax update   every lane owns one query column, so row max / row sum are
//                           in-lane plus one exchange with lane^32
//   O^T += V^T . P^T        P^T comes straight from the S^T accumulator registers;
//                           V^T is read from the row-major LDS tile with ds_read_b64_tr_b16
// and the epilogue writes out = O / l and lse = m + log l.
//
// The merge rule is the online softmax: a running row maximum m (log2 units), a
// running sum l and an unnormalised accumulator O; a new tile rescales them by
// exp2(m_old - m_new).  The rescale is deferred while the new maximum exceeds the
// stored one by at most kTau (P then stays <= 2^kTau), which is exact because O
// and l always share the same reference m.
#include <type_traits>

#include "mfma_util.cuh"

namespace ra {
namespace {

constexpr int BK = 64;            // keys per K/V tile
constexpr float kTau = 8.0f;      // lazy-rescale threshold, log2 units
constexpr float kSumMax = 256.0f; // 2^kTau

// LDS stages of the K/V ring (two: one tile in flight while one is computed; a third
// stage measured slower at head_dim 64).
template <int D>
struct FwdLds {
#ifndef RA_FWD_NS
#define RA_FWD_NS 2
#endif
  static constexpr int NS = D == 64 ? RA_FWD_NS : 2;
  static constexpr int TILE = BK * D;          // unpadded, swizzled (see swz)
  static constexpr int NSEG = TILE * 2 / 1024 / kWaves;   // 1 KiB direct-load segments per wave per tile
};

// OCC: waves per SIMD the register allocation must allow (2 lets one wave's softmax
// arithmetic run while the other's matrix products do).
// STEP: one ring step (see ra_blockwise_attn_fwd_step): the keys held are one block at global
// positions kv_pos0 + j, the running state is read from and written back to caller memory.
// CM: causal mode, 0 none, 1 token level, 2 causal blocks of p.causal > 1 tokens (a mode of its own,
// so that the common modes compile exactly as they would without block sizes).
template <int D, int NQB, int CM, bool HAS_BIAS, bool HAS_SEG, int OCC, bool STEP>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(OCC, OCC))) void fwd_mfma_kernel(Params p) {
  constexpr bool CAUSAL = CM != 0;
  constexpr bool CBLK = CM == 2;
  constexpr int QW = 32 * NQB;         // queries per wave
  constexpr int BQ = kWaves * QW;      // queries per workgroup
  constexpr int KK = D / 16;           // k-steps of S^T (head_dim / 16)
  constexpr int DB = D / 32;           // 32-row blocks of O^T
  constexpr int NS = FwdLds<D>::NS;
  constexpr int TILE = FwdLds<D>::TILE;
  constexpr int NSEG = FwdLds<D>::NSEG;
  static_assert(NSEG * 1024 * kWaves == TILE * 2, "tile must split into 1 KiB segments");

  __shared__ __attribute__((aligned(16))) __bf16 sK[NS][TILE];
  __shared__ __attribute__((aligned(16))) __bf16 sV[NS][TILE];
  __shared__ float sBias[NS][BK];
  __shared__ __attribute__((aligned(16))) int sSeg[NS][BK];
  __shared__ int sSegRange[NS][2];   // smallest and largest segment id among the tile's keys
  __shared__ int sWaveSeg[kWaves][2];  // each wave's range of query segment ids

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: wave-derived values stay scalar
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  // ---- which query tile (grid = B * H * n_qt): one (batch, head) per XCD at a time where B * H
  // allows it; within a head the heaviest (latest) query tiles go first
  const int64_t n_qt_blk = (p.Lb + BQ - 1) / BQ;
  const int64_t n_qt = (p.ring_rank < 0 ? p.n_ring : 1) * n_qt_blk;
  const HeadTile ht = head_tile(blockIdx.x, p.B * p.H, n_qt, true);
  const int hb = ht.hb;
  const int64_t t = n_qt - 1 - ht.t;
  const int b = hb / p.H, h = hb % p.H;
  const int r_local = static_cast<int>(t / n_qt_blk);
  const int64_t qa = (t % n_qt_blk) * BQ;                  // first row of the tile inside its block
  const int r = p.ring_rank < 0 ? r_local : p.ring_rank;
  const int64_t qrow_base = static_cast<int64_t>(r_local) * p.Lb;   // local row of the block's row 0
  // position of the tile's row 0 in the coordinates of the keys held (global positions minus
  // kv_pos0, which is 0 outside a single ring step)
  const int64_t pos0 = (STEP ? p.q_pos0 - p.kv_pos0 : static_cast<int64_t>(r) * p.Lb) + qa;
  const int64_t nrows = (p.Lb - qa) < BQ ? (p.Lb - qa) : BQ;

  const __bf16* __restrict__ qp = static_cast<const __bf16*>(p.q);
  const __bf16* __restrict__ kp = static_cast<const __bf16*>(p.k);
  const __bf16* __restrict__ vp = static_cast<const __bf16*>(p.v);

  // Without a bias or segment ids the score accumulators start from a held register copy of
  // -m (the row's reference maximum; 0 while it is -inf) and Q is held pre-multiplied by
  // c = scale * log2e (rounded to bfloat16), so the matrix unit delivers the exponent
  // c s - m directly and the vector unit is left with the exponential.  The other variants
  // have no registers to spare for the held copy: they keep raw Q and form c s - m per score.
  constexpr bool kFold = !HAS_BIAS && !HAS_SEG;
  const float c = p.scale * kLog2e;   // raw score -> log2 units
  // ---- the wave's queries, as the B operand of S^T = K . Q^T
  const int64_t wrow0 = qa + wave * QW;                      // first row of the wave inside the block
  const int64_t wpos0 = pos0 + wave * QW;
  const int64_t wvalid = p.Lb - wrow0;                       // rows of this wave that exist (may be <= 0)
  bf16x8 Qf[NQB][KK];
#pragma unroll
  for (int nb = 0; nb < NQB; ++nb) {
    const int64_t row = wrow0 + nb * 32 + l32;
    const bool ok = row < p.Lb;
    const __bf16* src = qp + row_offset(b, qrow_base + (ok ? row : 0), h, p.Lq, p.H, D);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      bf16x8 x = *reinterpret_cast<const bf16x8*>(src + 16 * kk + 8 * hh);
      Qf[nb][kk] = !ok ? bf16x8{} : (kFold ? scale_bf16x8(x, c) : x);
    }
  }
  int qseg[NQB];
  int qseg_lo = 0, qseg_hi = 0;   // range of the wave's query segment ids
  if constexpr (HAS_SEG) {
    int lo = INT32_MAX, hi = INT32_MIN;
#pragma unroll
    for (int nb = 0; nb < NQB; ++nb) {
      int64_t pos = wpos0 + nb * 32 + l32;
      const bool ok = wrow0 + nb * 32 + l32 < p.Lb;
      qseg[nb] = ok ? p.seg[static_cast<int64_t>(b) * p.seg_len + p.kv_pos0 + pos] : 0;
      lo = ok ? min(lo, qseg[nb]) : lo;
      hi = ok ? max(hi, qseg[nb]) : hi;
    }
    qseg_lo = __builtin_amdgcn_readfirstlane(wave_min_i32(lo));
    qseg_hi = __builtin_amdgcn_readfirstlane(wave_max_i32(hi));
  }
  // the workgroup's range of query segment ids: a K/V tile none of whose keys carries an id
  // in it has no visible pair with any of the workgroup's queries, and is neither loaded
  // nor computed (exact for any ids)
  int gseg_lo = 0, gseg_hi = 0;
  if constexpr (HAS_SEG) wg_id_range(qseg_lo, qseg_hi, sWaveSeg, wave, lane, gseg_lo, gseg_hi);

  float m[NQB], lsum[NQB];
  f32x16 minit[NQB];
  f32x16 O[DB][NQB];
#pragma unroll
  for (int nb = 0; nb < NQB; ++nb) {
    m[nb] = -INFINITY;
    lsum[nb] = 0.f;
    minit[nb] = f32x16{};
#pragma unroll
    for (int db = 0; db < DB; ++db) O[db][nb] = f32x16{};
  }

  if constexpr (STEP) {
    if (!p.step_init) {
      // the running state of an earlier ring step: O^T fragments as stored by the epilogue,
      // m (log2 units) in both lanes of a column, l in the lower one (the pair sums to it)
#pragma unroll
      for (int nb = 0; nb < NQB; ++nb) {
        const int64_t row = wrow0 + nb * 32 + l32;
        if (row >= p.Lb) continue;
        const float* src = p.o_state + row_offset(b, row, h, p.Lq, p.H, D);
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int v4 = 0; v4 < 4; ++v4) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(src + db * 32 + 8 * v4 + 4 * hh);
#pragma unroll
            for (int i = 0; i < 4; ++i) O[db][nb][4 * v4 + i] = x[i];
          }
        const int64_t si = (static_cast<int64_t>(b) * p.H + h) * p.Lq + row;
        m[nb] = p.m_state[si];
        lsum[nb] = hh == 0 ? p.l_state[si] : 0.f;
      }
    }
#pragma unroll
    for (int nb = 0; nb < NQB; ++nb) {
      const float ms = m[nb] == -INFINITY ? 0.f : -m[nb];
#pragma unroll
      for (int v = 0; v < 16; ++v) minit[nb][v] = ms;
    }
  }

  // ---- K/V tile staging: direct global -> LDS copies into a ring of NS stages, issued
  // NS - 1 tiles ahead.  Each wave copies NSEG 1 KiB segments of K and of V per tile; the
  // lane that lands at segment byte 16 l fetches the chunk the swizzle puts there.  The
  // tile's base address is wave-uniform; rows past the end of a ragged tile fetch row 0
  // instead (finite values that the masks give zero weight).
  const int64_t kv_bh = (static_cast<int64_t>(b) * p.Lk * p.H + h) * D;   // (b, key 0, h)
  const int64_t kstride = static_cast<int64_t>(p.H) * D;                 // elements per key
  int grow_[NSEG], goff[NSEG], goff0[NSEG];
#pragma unroll
  for (int j = 0; j < NSEG; ++j) {
    const int byte = (wave * NSEG + j) * 1024 + lane * 16;
    const int row = byte / (2 * D);
    const int chunk = ((byte % (2 * D)) >> 4) ^ swz_key<D>(row);
    grow_[j] = row;
    goff[j] = row * static_cast<int>(kstride) + chunk * 8;   // < 64 * H * D, checked on the host
    goff0[j] = chunk * 8;
  }
  // For head_dim 64 without bias or segment ids the copies take the tile's base from SGPRs and a
  // 32-bit per-lane byte offset (2 goff < 2^32, which the host ensures) as their only per-lane
  // operand; the other variants form 64-bit addresses, since the SGPR bases push them into spills.
  constexpr bool kUniformCopies = D == 64 && !HAS_BIAS && !HAS_SEG;
  // bias / segment ids of the tile (plain loads; the raw values are kept until store_small,
  // before the barrier, so that the wait for these loads lands there)
  float breg = 0.f;
  int sreg = 0;
  bool kok = false;
  auto load_small = [&](int key0, int kend) {
    if (tid < BK) {
      kok = key0 + tid < kend;
      const int key = kok ? key0 + tid : key0;
      if constexpr (HAS_BIAS)
        breg = p.bias[static_cast<int64_t>(h) * p.bias_len +
                      static_cast<unsigned>(static_cast<int>(p.kv_pos0) + key) % static_cast<unsigned>(p.bias_len)];
      if constexpr (HAS_SEG) sreg = p.seg[static_cast<int64_t>(b) * p.seg_len + p.kv_pos0 + key];
    }
  };
  auto store_small = [&](int slot) {
    if (tid < BK) {
      if constexpr (HAS_BIAS) sBias[slot][tid] = kok ? breg * kLog2e : 0.f;
      if constexpr (HAS_SEG) {
        const int sid = kok ? sreg : 0;
        sSeg[slot][tid] = sid;
        // the tile's id range lets a wave skip a tile that shares no segment with its queries
        const int lo = wave_min_i32(kok ? sid : INT32_MAX);
        const int hi = wave_max_i32(kok ? sid : INT32_MIN);
        if (tid == 0) {
          sSegRange[slot][0] = lo;
          sSegRange[slot][1] = hi;
        }
      }
    }
  };
  auto issue_kv = [&](int key0, int kend, int slot) {
    const __bf16* kb = kp + kv_bh + static_cast<int64_t>(key0) * kstride;
    const __bf16* vb = vp + kv_bh + static_cast<int64_t>(key0) * kstride;
    if constexpr (kUniformCopies) {
      // full tiles (all but a block's ragged last one) take a branch of their own, so their copies
      // need no per-chunk selects (-1.6% on the 1M-token share; the dQ kernel does the same)
      if (key0 + BK <= kend) {
#pragma unroll
        for (int j = 0; j < NSEG; ++j) {
          const unsigned off = 2u * static_cast<unsigned>(goff[j]);
          dma16_sb(kb, off, &sK[slot][(wave * NSEG + j) * 512]);
          dma16_sb(vb, off, &sV[slot][(wave * NSEG + j) * 512]);
        }
      } else {
        const int nvalid = kend - key0;
#pragma unroll
        for (int j = 0; j < NSEG; ++j) {
          const unsigned off = 2u * static_cast<unsigned>(grow_[j] < nvalid ? goff[j] : goff0[j]);
          dma16_sb(kb, off, &sK[slot][(wave * NSEG + j) * 512]);
          dma16_sb(vb, off, &sV[slot][(wave * NSEG + j) * 512]);
        }
      }
    } else {
      const bool full = key0 + BK <= kend;
      const int nvalid = kend - key0;
#pragma unroll
      for (int j = 0; j < NSEG; ++j) {
        const int off = (full || grow_[j] < nvalid) ? goff[j] : goff0[j];
        dma16(kb + off, &sK[slot][(wave * NSEG + j) * 512]);
        dma16(vb + off, &sV[slot][(wave * NSEG + j) * 512]);
      }
    }
  };

  // ring walk with NS - 1 tiles of lookahead: T[0] is being computed, T[NS-1] is issued
  // causal limits: relative positions have their origin at global position kv_pos0 (0 outside a
  // ring step); the walk stops after the last key the workgroup's last query can see
  const int coff = static_cast<int>(p.kv_pos0);
  RingWalk walk;
  walk.begin(p.n_ring, r, p.Lb, CAUSAL,
             CBLK && nrows > 0 ? causal_last_key(static_cast<int>(pos0 + nrows - 1), coff, p.causal) : pos0 + nrows - 1);
  // With segment ids the walk passes over tiles that share no id with the workgroup's
  // queries (windows of 64 tiles, see SegTileFilter).
  SegTileFilter filt;
  const int* __restrict__ kv_ids = HAS_SEG ? p.seg + static_cast<int64_t>(b) * p.seg_len + p.kv_pos0 : nullptr;
  auto next_tile = [&]() -> bool {
    while (walk.next<BK>()) {
      if constexpr (!HAS_SEG) return true;
      static_assert(BK == 64, "the segment filter works in 64-key tiles");
      const int skip = filt.skip(kv_ids, walk.key0, walk.kend, gseg_lo, gseg_hi, lane);
      if (skip == 0) return true;
      walk.key0 += (skip - 1) * BK;   // next() adds the last BK
    }
    return false;
  };
  int tk0[NS], tke[NS];
  bool tok[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    tok[i] = nrows > 0 && next_tile();
    tk0[i] = walk.key0;
    tke[i] = walk.kend;
  }
  // prologue: the first NS - 1 tiles
#pragma unroll
  for (int i = 0; i < NS - 1; ++i)
    if (tok[i]) {
      load_small(tk0[i], tke[i]);
      issue_kv(tk0[i], tke[i], i);
      store_small(i);
    }
  RA_WAIT_VMCNT(0);
  __syncthreads();

  // the wave's first query position and last existing row as 32-bit values (token positions
  // are below 2^30, checked on the host), so that per-tile tests stay on the scalar unit
  const int wpos = static_cast<int>(wpos0);
  const int wlast = static_cast<int>(wvalid < QW ? wvalid : QW) - 1;
  // the last key the wave's first and last query can see, and each lane's own limits
  int wlim_first = 0, wlim_last = 0;
  int qlim[NQB];
#pragma unroll
  for (int nb = 0; nb < NQB; ++nb) qlim[nb] = 0;
  if constexpr (CBLK) {
    wlim_first = causal_last_key(wpos, coff, p.causal);
    wlim_last = wlast >= 0 ? causal_last_key(wpos + wlast, coff, p.causal) : -1;
#pragma unroll
    for (int nb = 0; nb < NQB; ++nb) qlim[nb] = causal_last_key(wpos + nb * 32 + l32, coff, p.causal);
  }
  // one step of the walk per ring stage.  For head_dim 64 without bias or segment ids the walk
  // is unrolled over the stages, so that each stage's LDS addresses are compile-time offsets (no
  // per-tile address arithmetic on the vector unit); the other variants keep a runtime stage,
  // since the unrolled bodies push them into spills.
  constexpr bool kUnrollWalk = D == 64 && !HAS_BIAS && !HAS_SEG;
  auto step = [&](auto slot_c) {
    const int slot = slot_c;   // a compile-time constant when the walk is unrolled
    const int key0 = tk0[0], kend = tke[0];
    const int ahead = slot + NS - 1 >= NS ? slot - 1 : slot + NS - 1;   // (slot + NS - 1) % NS
    const bool issue = tok[NS - 1];
    if (issue) {
      load_small(tk0[NS - 1], tke[NS - 1]);   // before the copies: its wait then spares them
      issue_kv(tk0[NS - 1], tke[NS - 1], ahead);
    }
    const int buf = slot;
    const __bf16* Kt = sK[buf];
    const __bf16* Vt = sV[buf];
    bool wave_active = wlast >= 0 && !(CAUSAL && key0 > (CBLK ? wlim_last : wpos + wlast));
    bool seg_mask = HAS_SEG;   // some pair of the tile may lie in different segments
    if constexpr (HAS_SEG) {
      // no key of the tile shares a segment with the wave's queries: every pair is masked
      const int klo = __builtin_amdgcn_readfirstlane(sSegRange[buf][0]);
      const int khi = __builtin_amdgcn_readfirstlane(sSegRange[buf][1]);
      wave_active = wave_active && klo <= qseg_hi && khi >= qseg_lo;
      // every key and every query of the wave in one segment: the segment mask selects nothing
      seg_mask = !(klo == khi && qseg_lo == qseg_hi && klo == qseg_lo);
    }
    if (wave_active) {
      const bool need_mask = seg_mask || (key0 + BK > kend) || (CAUSAL && key0 + BK - 1 > (CBLK ? wlim_first : wpos));
      bf16x8 P[NQB][2][2];   // [query block][key block][16-key step]
      // kFold: a fast pass first.  It takes the exponentials against the held reference without
      // forming the row maximum.  If every lane's part of the tile's row sum is at most 2^kTau,
      // no score exceeds the reference by more than kTau, so the exact pass would find no row to
      // rescale and compute the very same values.  Otherwise (a row's first visible tile, or a
      // maximum that grew) the tile is done again by the exact pass: row maximum, rescale of the
      // rows whose maximum grew by more than kTau, exponentials against the new reference.
      // The other variants take the exact pass only.
      bool exact = !kFold;
      if constexpr (kFold) {
        bool fresh = false;   // a row with no reference yet
#pragma unroll
        for (int nb = 0; nb < NQB; ++nb) fresh = fresh || m[nb] == -INFINITY;
        exact = __ballot(fresh) != 0;
      }
      int zoff = 0;
      for (;;) {
        // (a second pass reads the K tile from LDS again: its offset goes through an empty asm
        // statement, so that the compiler does not hold the first pass's reads in registers)
        if constexpr (kFold) asm volatile("" : "+s"(zoff));
        const __bf16* Kp = Kt + zoff;
        // ---- S^T = K . Q^T : rows = 64 keys (two 32-row blocks), columns = the wave's queries
        // (kFold: in log2 units, minus the row's reference maximum)
        f32x16 S[2][NQB];
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
          for (int mb = 0; mb < 2; ++mb) {
            const bf16x8 a = lds_read_swz<D>(Kp, mb * 32 + l32, 2 * kk + hh);
#pragma unroll
            for (int nb = 0; nb < NQB; ++nb)
              S[mb][nb] = mfma32(a, Qf[nb][kk], kk > 0 ? S[mb][nb] : (kFold ? minit[nb] : f32x16{}));
          }
        }
        int kseg[2][16];
        if (HAS_SEG && need_mask) {
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
              const int4 x = *reinterpret_cast<const int4*>(&sSeg[buf][mb * 32 + 8 * g4 + 4 * hh]);
              kseg[mb][4 * g4 + 0] = x.x;
              kseg[mb][4 * g4 + 1] = x.y;
              kseg[mb][4 * g4 + 2] = x.z;
              kseg[mb][4 * g4 + 3] = x.w;
            }
        }
        bool ok = true;
        float part[NQB];
#pragma unroll
        for (int nb = 0; nb < NQB; ++nb) {
          // logits in log2 units when there is a bias (else, without kFold, raw scores scaled
          // inside the exponential)
          if constexpr (HAS_BIAS) {
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
              for (int v = 0; v < 16; ++v) {
                const int kr = mb * 32 + 8 * (v >> 2) + 4 * hh + (v & 3);
                S[mb][nb][v] = __builtin_fmaf(S[mb][nb][v], c, sBias[buf][kr]);
              }
          }
          if (need_mask) {
            // key kr of the tile is visible iff kr <= klim (causal and ragged end) and, with
            // segments, its id equals the query's; applied with selects, no branches
            int klim = (kend - key0 < BK ? kend - key0 : BK) - 1;
            if constexpr (CAUSAL) {
              // the query's last visible key, relative to key 0
              const int rel = CBLK ? qlim[nb] - key0 : wpos - key0 + nb * 32 + l32;
              klim = rel < klim ? (rel < -1 ? -1 : rel) : klim;
            }
            // the lane's key rows are kr0(v) + 4 * hh with kr0 a constant of v: compare kr0
            // against the shifted limit, so the row numbers never occupy registers
            const int klim4 = klim - 4 * hh;
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
              for (int v = 0; v < 16; ++v) {
                bool vis = mb * 32 + 8 * (v >> 2) + (v & 3) <= klim4;
                if constexpr (HAS_SEG) vis = vis && kseg[mb][v] == qseg[nb];
                S[mb][nb][v] = vis ? S[mb][nb][v] : -INFINITY;
              }
          }
          if (exact) {
            float mx = -INFINITY;
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
              for (int v = 0; v < 16; ++v) mx = fmaxf(mx, S[mb][nb][v]);
            mx = pair_max(mx);
            // the offset already taken off the scores (kFold), and the tile's maximum in absolute terms
            const float msub0 = (m[nb] == -INFINITY) ? 0.f : m[nb];
            const float mxa = kFold ? mx + msub0 : (HAS_BIAS ? mx : mx * c);
            // Each row decides for itself whether its maximum grew by more than kTau; the
            // multiply runs only when some row of the wave needs it, with alpha = 1 (exact)
            // for the others, so a row's result never depends on its neighbours' data.
            const bool grow = mxa > m[nb] + kTau;
            if (__ballot(grow) != 0) {
              const float mnew = grow ? mxa : m[nb];
              const float alpha = grow ? __builtin_amdgcn_exp2f(m[nb] - mnew) : 1.f;   // m = -inf gives 0
              lsum[nb] *= alpha;
#pragma unroll
              for (int db = 0; db < DB; ++db) O[db][nb] *= alpha;
              m[nb] = mnew;
              if constexpr (kFold) {
                // move the tile's scores and the held offset to the new reference
                const float shift = grow ? mnew - msub0 : 0.f;
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                  for (int v = 0; v < 16; ++v) S[mb][nb][v] -= shift;
                const float ms = m[nb] == -INFINITY ? 0.f : -m[nb];
#pragma unroll
                for (int v = 0; v < 16; ++v) minit[nb][v] = ms;
              }
            }
          }
          // exponentials against the reference, packed into P, and the lane's part of the row
          // sum in independent partial sums (no serial dependency chain)
          const float msub = kFold ? 0.f : ((m[nb] == -INFINITY) ? 0.f : m[nb]);
          float acc[2][2];
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int st = 0; st < 2; ++st) {
              float e[8];
#pragma unroll
              for (int i = 0; i < 8; ++i) {
                const float x = S[mb][nb][8 * st + i];
                e[i] = kFold      ? __builtin_amdgcn_exp2f(x)
                       : HAS_BIAS ? __builtin_amdgcn_exp2f(x - msub)
                                  : __builtin_amdgcn_exp2f(__builtin_fmaf(x, c, -msub));
              }
              P[nb][mb][st] = pack_bf16x8(e);
              acc[mb][st] = ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
            }
          part[nb] = (acc[0][0] + acc[0][1]) + (acc[1][0] + acc[1][1]);
          ok = ok && part[nb] <= kSumMax;
        }
        if (exact || __ballot(!ok) == 0) {
#pragma unroll
          for (int nb = 0; nb < NQB; ++nb) lsum[nb] += part[nb];
          break;
        }
        exact = true;
      }

      // ---- O^T += V^T . P^T ; V^T operand through transposed LDS reads
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const bf16x8 a = lds_read_a_transposed_swz<D>(Vt, mb * 32, st, db * 32, lane);
#pragma unroll
            for (int nb = 0; nb < NQB; ++nb) O[db][nb] = mfma32(a, P[nb][mb][st], O[db][nb]);
          }
    }

    // the next tile's copies (issued NS - 2 iterations ago) must have landed; the ones
    // issued this iteration may stay in flight
    if (issue) {
      store_small(ahead);
      if constexpr (NS == 3) {
        RA_WAIT_VMCNT(2 * NSEG);
      } else {
        RA_WAIT_VMCNT(0);
      }
    } else {
      RA_WAIT_VMCNT(0);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i + 1 < NS; ++i) {
      tok[i] = tok[i + 1];
      tk0[i] = tk0[i + 1];
      tke[i] = tke[i + 1];
    }
    tok[NS - 1] = next_tile();
    tk0[NS - 1] = walk.key0;
    tke[NS - 1] = walk.kend;
  };
  if constexpr (kUnrollWalk) {
    static_assert(NS == 2 || NS == 3, "the walk is unrolled over two or three stages");
    while (tok[0]) {
      step(std::integral_constant<int, 0>{});
      if (!tok[0]) break;
      step(std::integral_constant<int, 1>{});
      if constexpr (NS == 3) {
        if (!tok[0]) break;
        step(std::integral_constant<int, 2>{});
      }
    }
  } else {
    int slot = 0;
    while (tok[0]) {
      step(slot);
      slot = slot + 1 == NS ? 0 : slot + 1;
    }
  }

  if constexpr (STEP) {
    // ---- epilogue of a ring step: the running state goes back to caller memory
#pragma unroll
    for (int nb = 0; nb < NQB; ++nb) {
      const int64_t row = wrow0 + nb * 32 + l32;
      const float lt = pair_sum(lsum[nb]);
      if (row >= p.Lb) continue;
      float* dst = p.o_state + row_offset(b, row, h, p.Lq, p.H, D);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
          f32x4 x;
#pragma unroll
          for (int i = 0; i < 4; ++i) x[i] = O[db][nb][4 * v4 + i];
          *reinterpret_cast<f32x4*>(dst + db * 32 + 8 * v4 + 4 * hh) = x;
        }
      if (hh == 0) {
        const int64_t si = (static_cast<int64_t>(b) * p.H + h) * p.Lq + row;
        p.m_state[si] = m[nb];
        p.l_state[si] = lt;
      }
    }
    return;
  }
  // ---- epilogue: out = O / l, lse = m + log l (natural log)
  __bf16* __restrict__ op = static_cast<__bf16*>(p.out);
#pragma unroll
  for (int nb = 0; nb < NQB; ++nb) {
    const int64_t row = wrow0 + nb * 32 + l32;
    const float lt = pair_sum(lsum[nb]);
    if (row >= p.Lb || row < 0) continue;
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    __bf16* dst = op + row_offset(b, qrow_base + row, h, p.Lq, p.H, D);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        bf16x4 o4;
#pragma unroll
        for (int i = 0; i < 4; ++i) o4[i] = (__bf16)(O[db][nb][4 * v4 + i] * inv);
        *reinterpret_cast<bf16x4*>(dst + db * 32 + 8 * v4 + 4 * hh) = o4;
      }
    if (hh == 0)
      p.lse[(static_cast<int64_t>(b) * p.H + h) * p.Lq + qrow_base + row] =
          lt > 0.f ? (m[nb] + __builtin_amdgcn_logf(lt)) * kLn2 : -INFINITY;
  }
}

template <int D, int NQB, int CM, bool HAS_BIAS, bool HAS_SEG, bool STEP>
hipError_t launch_t(const Params& p, hipStream_t st) {
  constexpr int BQ = kWaves * 32 * NQB;
  const int64_t n_qt = (p.ring_rank < 0 ? p.n_ring : 1) * ((p.Lb + BQ - 1) / BQ);
  const int64_t grid = n_qt * p.B * p.H;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  // two waves per SIMD for every variant: the bias and segment variants spill a few registers,
  // outside the score products, which costs far less than a SIMD left with one wave (measured:
  // 44-48% less forward time with segment ids or a bias)
  constexpr int OCC = 2;
  hipLaunchKernelGGL((fwd_mfma_kernel<D, NQB, CM, HAS_BIAS, HAS_SEG, OCC, STEP>), dim3(static_cast<unsigned>(grid)),
                     dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

template <int D, int NQB, int CM, bool STEP>
hipError_t launch_m(const Params& p, hipStream_t st) {
  const bool bi = p.bias != nullptr, sg = p.seg != nullptr;
  if (bi) return sg ? launch_t<D, NQB, CM, true, true, STEP>(p, st) : launch_t<D, NQB, CM, true, false, STEP>(p, st);
  return sg ? launch_t<D, NQB, CM, false, true, STEP>(p, st) : launch_t<D, NQB, CM, false, false, STEP>(p, st);
}

template <int D, int NQB, bool STEP>
hipError_t launch_d(const Params& p, hipStream_t st) {
  if (p.causal == 0) return launch_m<D, NQB, 0, STEP>(p, st);
  if (p.causal == 1) return launch_m<D, NQB, 1, STEP>(p, st);
  return launch_m<D, NQB, 2, STEP>(p, st);
}

}  // namespace

hipError_t launch_fwd_mfma(const Params& p, hipStream_t st) {
  if (p.D == 64) return launch_d<64, 2, false>(p, st);
  if (p.D == 128) return launch_d<128, 1, false>(p, st);
  return hipErrorInvalidValue;
}

hipError_t launch_fwd_step_mfma(const Params& p, hipStream_t st) {
  if (p.D == 64) return launch_d<64, 2, true>(p, st);
  if (p.D == 128) return launch_d<128, 1, true>(p, st);
  return hipErrorInvalidValue;
}

}  // namespace ra
