// Backward blockwise ring attention, dK/dV kernel: bfloat16 in / float32 accumulate, MFMA on gfx950.
//
// The probabilities are recomputed from the saved logsumexp, P = exp(s - lse),
// so no score matrix is ever stored (the recompute policy of the pages'
// blockwise_kwargs).  Two kernels, each owning the rows it writes, so the
// result is deterministic and needs no atomics: this file's and the one in
// bwd_dq_mfma.hip (dQ).  The two kernels live in separate files so that neither's code shape can
// change how the compiler allocates the other's registers.
//
// dK/dV kernel -- one workgroup owns BKW keys of one (batch, head): each wave
//   keeps 32 * NKB keys' K and V rows in VGPRs and walks the query tiles that
//   K/V block meets on the ring (its own rank first, then the later ones);
//   query tiles (Q, dO, lse, Delta, segment ids) stream through LDS, two
//   buffers deep.  Per query tile and 32-query block:
//     S  = Q . K^T,  dP = dO . V^T     (rows = queries, columns = the lane's key)
//     P  = exp2(S * scale * log2e + bias - lse * log2e),  dS = P (dP - Delta)
//   The held K rows are stored pre-multiplied by scale * log2e (rounded to bfloat16) and the
//   score accumulators start at bias - lse * log2e, the dP accumulators at -Delta, so that the
//   matrix unit delivers the exponent and dP - Delta directly and the vector unit is left with
//   one exponential and one product per score.
//     dV^T += dO^T . P,  dK^T += Q^T . dS     (dO^T, Q^T by transposing LDS reads)
#include <type_traits>

#include "mfma_util.cuh"


namespace ra {
namespace {

// ================================================================== dK/dV (K/V tiles stationary)
#ifndef RA_KV_BQ
#define RA_KV_BQ 128
#endif
constexpr int kBqKv = RA_KV_BQ;   // queries per LDS tile at head_dim 64 without segment ids (else 64)

// STEP: one backward ring step (ra_blockwise_attn_bwd_step): the queries held are one block at
// global positions q_pos0 + i, and dK / dV are summed into float32 caller memory (unscaled).
template <int D, int NKB, int CM, bool HAS_BIAS, bool HAS_SEG, int OCC, bool STEP>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(OCC, OCC))) void dkdv_mfma_kernel(Params p) {
  constexpr bool CAUSAL = CM != 0;
  constexpr bool CBLK = CM == 2;
  constexpr int BQ = (HAS_SEG || D != 64) ? 64 : kBqKv;
  constexpr int KW = 32 * NKB;         // keys per wave
  constexpr int BKW = kWaves * KW;     // keys per workgroup
  constexpr int KK = D / 16;
  constexpr int DB = D / 32;
#ifndef RA_KV_NS
#define RA_KV_NS 2
#endif
  constexpr int NS = D == 64 ? RA_KV_NS : 2;  // LDS stages of the query-tile ring
  constexpr int TILE = BQ * D;         // unpadded, swizzled
  constexpr int NSEG = TILE * 2 / 1024 / kWaves;   // 1 KiB direct-copy segments per wave per tile
  static_assert(NSEG * 1024 * kWaves == TILE * 2, "tile must split into 1 KiB segments");
  static_assert(BQ % 32 == 0 && BQ <= kThreads, "whole 32-query blocks per tile");

  __shared__ __attribute__((aligned(16))) __bf16 sQ[NS][TILE];
  __shared__ __attribute__((aligned(16))) __bf16 sG[NS][TILE];
  __shared__ __attribute__((aligned(16))) float sL[NS][BQ];    // -lse * log2e (-inf: row contributes nothing)
  __shared__ __attribute__((aligned(16))) float sDl[NS][BQ];   // -Delta
  __shared__ __attribute__((aligned(16))) int sSg[NS][BQ];     // segment id of the query
  __shared__ int sTileSeg[NS][2];   // smallest and largest segment id among the tile's queries
  __shared__ int sWaveSeg[kWaves][2];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  // grid = B * H * n_ring * n_kt_blk: a head's key tiles of block 0 first (under a causal mask they
  // meet the most query blocks); one (batch, head) per XCD at a time for one rank's queries (or one
  // ring step), pairs fastest for the whole ring, as in the dQ kernel
  const int64_t n_kt_blk = (p.Lb + BKW - 1) / BKW;
  const HeadTile ht = head_tile(blockIdx.x, p.B * p.H, static_cast<int64_t>(p.n_ring) * n_kt_blk,
                                p.ring_rank >= 0);
  const int hb = ht.hb;
  const int64_t kt = ht.t;
  const int b = hb / p.H, h = hb % p.H;
  const int j = static_cast<int>(kt / n_kt_blk);
  const int64_t ka = (kt % n_kt_blk) * BKW;                     // first key of the tile inside block j
  const int64_t kfirst = static_cast<int64_t>(j) * p.Lb + ka;   // its global position
  const int64_t wk0 = ka + wave * KW;                           // the wave's first key inside block j
  const int64_t wkey0 = kfirst + wave * KW;                     // ... and its global position

  const __bf16* __restrict__ qp = static_cast<const __bf16*>(p.q);
  const __bf16* __restrict__ kp = static_cast<const __bf16*>(p.k);
  const __bf16* __restrict__ vp = static_cast<const __bf16*>(p.v);
  const __bf16* __restrict__ gp = static_cast<const __bf16*>(p.dout);
  // segment ids on positions relative to the keys held (kv_pos0 = 0 outside a ring step)
  const int* __restrict__ ids = HAS_SEG ? p.seg + static_cast<int64_t>(b) * p.seg_len + p.kv_pos0 : nullptr;

  // the wave's keys, as B operands of S = Q . K^T (K times scale * log2e) and dP = dO . V^T
  bf16x8 Kf[NKB][KK], Vf[NKB][KK];
  float kbias[NKB];
  int ksg[NKB];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    const int64_t krow = wk0 + kb * 32 + l32;
    const bool ok = krow < p.Lb;
    const int64_t key = static_cast<int64_t>(j) * p.Lb + (ok ? krow : 0);
    const int64_t off = row_offset(b, key, h, p.Lk, p.H, D);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const bf16x8 x = *reinterpret_cast<const bf16x8*>(kp + off + 16 * kk + 8 * hh);
      const bf16x8 y = *reinterpret_cast<const bf16x8*>(vp + off + 16 * kk + 8 * hh);
      Kf[kb][kk] = ok ? scale_bf16x8(x, p.scale * kLog2e) : bf16x8{};
      Vf[kb][kk] = ok ? y : bf16x8{};
    }
    kbias[kb] = (HAS_BIAS && ok) ? p.bias[static_cast<int64_t>(h) * p.bias_len + (p.kv_pos0 + key) % p.bias_len] * kLog2e
                                 : 0.f;
    ksg[kb] = (HAS_SEG && ok) ? ids[key] : 0;
  }
  // the wave's and the workgroup's range of key segment ids: query tiles with no id in the
  // workgroup's range are passed over, and a wave skips the products of a tile with none in its own
  int gseg_lo = 0, gseg_hi = 0, kseg_lo = 0, kseg_hi = 0;
  if constexpr (HAS_SEG) {
    int lo = INT32_MAX, hi = INT32_MIN;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
      if (wk0 + kb * 32 + l32 < p.Lb) {
        lo = min(lo, ksg[kb]);
        hi = max(hi, ksg[kb]);
      }
    kseg_lo = __builtin_amdgcn_readfirstlane(wave_min_i32(lo));
    kseg_hi = __builtin_amdgcn_readfirstlane(wave_max_i32(hi));
    wg_id_range(kseg_lo, kseg_hi, sWaveSeg, wave, lane, gseg_lo, gseg_hi);
  }

  // with a bias: the lane's part of sum_i dS_ij for its key, from which the bias gradient is formed
  // (in a ring step the sums are added to the ones the K/V block carries)
  constexpr bool KEYSUM = HAS_BIAS;
  float dsum[NKB];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) dsum[kb] = 0.f;
  f32x16 dK[DB][NKB], dV[DB][NKB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      dK[db][kb] = f32x16{};
      dV[db][kb] = f32x16{};
    }
  if constexpr (STEP) {
    if (!p.init_dkv) {
      // the sums of earlier ring steps: lane holds d = db*32 + 8*(v/4) + 4*hh + v%4 of its key
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const int64_t krow = wk0 + kb * 32 + l32;
        if (krow >= p.Lb) continue;
        const int64_t off = row_offset(b, krow, h, p.Lk, p.H, D);
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int v4 = 0; v4 < 4; ++v4) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(p.dk_acc + off + db * 32 + 8 * v4 + 4 * hh);
            const f32x4 y = *reinterpret_cast<const f32x4*>(p.dv_acc + off + db * 32 + 8 * v4 + 4 * hh);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              dK[db][kb][4 * v4 + i] = x[i];
              dV[db][kb][4 * v4 + i] = y[i];
            }
          }
      }
    }
  }

  // ---- query tile staging: direct global -> LDS copies of Q and dO into a ring of NS
  // stages, issued NS - 1 tiles ahead (rows past the rank's end fetch the tile's row 0:
  // finite values whose -inf lse gives them zero weight); lse, Delta and segment ids of
  // the tile go through registers.
  const int64_t qstride = static_cast<int64_t>(p.H) * D;
  const int64_t q_bh = (static_cast<int64_t>(b) * p.Lq * p.H + h) * D;   // (b, row 0, h)
  int grow_[NSEG], goff[NSEG], goff0[NSEG];
#pragma unroll
  for (int jj = 0; jj < NSEG; ++jj) {
    const int byte = (wave * NSEG + jj) * 1024 + lane * 16;
    const int row = byte / (2 * D);
    const int chunk = ((byte % (2 * D)) >> 4) ^ swz_key<D>(row);
    grow_[jj] = row;
    goff[jj] = row * static_cast<int>(qstride) + chunk * 8;   // < 128 * H * D, checked on the host
    goff0[jj] = chunk * 8;
  }
  // For head_dim 64 without bias or segment ids the copies take the tile's base from SGPRs and a
  // 32-bit per-lane byte offset (2 goff < 2^32, which the host ensures) as their only per-lane
  // operand; the other variants form 64-bit addresses, since the SGPR bases push them into spills.
  constexpr bool kUniformCopies = D == 64 && !HAS_BIAS && !HAS_SEG;
  // (raw values are kept until the store, so that the wait for these loads lands there and
  // not right after them)
  float lreg = 0.f, dreg = 0.f;
  int sreg = 0;
  bool lok = false;
  auto load_small = [&](int row0, int rend, int pbase) {
    if (tid < BQ) {
      const int r = row0 + tid;
      lok = r < rend;
      const int rr = lok ? r : row0;
      const int64_t li = (static_cast<int64_t>(b) * p.H + h) * p.Lq + rr;
      lreg = p.lse[li];
      dreg = p.delta[li];
      if constexpr (HAS_SEG) sreg = ids[pbase + rr];
    }
  };
  auto store_small = [&](int slot) {
    if (tid < BQ) {
      sL[slot][tid] = (lok && lreg != -INFINITY) ? -lreg * kLog2e : -INFINITY;
      sDl[slot][tid] = lok ? -dreg : 0.f;
      if constexpr (HAS_SEG) {
        static_assert(!HAS_SEG || BQ == 64, "one wave holds a segment tile's ids");
        const int sid = lok ? sreg : 0;
        sSg[slot][tid] = sid;
        const int lo = wave_min_i32(lok ? sid : INT32_MAX);
        const int hi = wave_max_i32(lok ? sid : INT32_MIN);
        if (tid == 0) {
          sTileSeg[slot][0] = lo;
          sTileSeg[slot][1] = hi;
        }
      }
    }
  };
  auto issue_qg = [&](int row0, int rend, int slot) {
    const __bf16* qb_ = qp + q_bh + static_cast<int64_t>(row0) * qstride;
    const __bf16* gb_ = gp + q_bh + static_cast<int64_t>(row0) * qstride;
    if constexpr (kUniformCopies) {
      const bool full = row0 + BQ <= rend;
      const int nvalid = rend - row0;
      if (!STEP && full) {
        // full tiles in a branch of their own, with no per-chunk selects (-0.5% on the 1M-token share);
        // the ring-step variant keeps the selects, without which it no longer fits 256 registers
#pragma unroll
        for (int jj = 0; jj < NSEG; ++jj) {
          const unsigned off = 2u * static_cast<unsigned>(goff[jj]);
          dma16_sb(qb_, off, &sQ[slot][(wave * NSEG + jj) * 512]);
          dma16_sb(gb_, off, &sG[slot][(wave * NSEG + jj) * 512]);
        }
      } else {
#pragma unroll
        for (int jj = 0; jj < NSEG; ++jj) {
          const unsigned off = 2u * static_cast<unsigned>(full ? goff[jj] : (grow_[jj] < nvalid ? goff[jj] : goff0[jj]));
          dma16_sb(qb_, off, &sQ[slot][(wave * NSEG + jj) * 512]);
          dma16_sb(gb_, off, &sG[slot][(wave * NSEG + jj) * 512]);
        }
      }
    } else {
      const bool full = row0 + BQ <= rend;
      const int nvalid = rend - row0;
#pragma unroll
      for (int jj = 0; jj < NSEG; ++jj) {
        const int off = (full || grow_[jj] < nvalid) ? goff[jj] : goff0[jj];
        dma16(qb_ + off, &sQ[slot][(wave * NSEG + jj) * 512]);
        dma16(gb_ + off, &sG[slot][(wave * NSEG + jj) * 512]);
      }
    }
  };

  // query walk with NS - 1 tiles of lookahead: entry 0 is computed, entry NS - 1 is issued
  // causal limits: positions relative to global kv_pos0 (0 outside a ring step); the walk skips
  // the query tiles that end before the first query able to see the workgroup's first key
  const int coff = static_cast<int>(p.kv_pos0);
  const int64_t qfirst = CBLK ? causal_first_query(static_cast<int>(kfirst), coff, p.causal) : kfirst;
  QueryWalk walk;
  if constexpr (STEP) walk.begin_step(p.Lq, CAUSAL, qfirst, p.q_pos0 - p.kv_pos0);
  else walk.begin(p.n_ring, j, p.Lb, CAUSAL, qfirst, p.ring_rank);
  SegTileFilter filt;   // with segment ids: pass over query tiles sharing no id with the keys
  auto next_tile = [&]() -> bool {
    while (walk.next<BQ>()) {
      if constexpr (!HAS_SEG) return true;
      static_assert(!HAS_SEG || BQ == 64, "the segment filter works in 64-query tiles");
      // local rows of the current rank: the id of row q sits at position pos_base + q
      const int skip = filt.skip(ids + walk.pos_base, walk.row0, walk.rend, gseg_lo, gseg_hi, lane);
      if (skip == 0) return true;
      walk.row0 += (skip - 1) * BQ;   // next() adds the last BQ
    }
    return false;
  };
  int tr0[NS], tre[NS], tpb[NS];
  bool tok[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    tok[i] = next_tile();
    tr0[i] = walk.row0;
    tre[i] = walk.rend;
    tpb[i] = walk.pos_base;
  }
#pragma unroll
  for (int i = 0; i < NS - 1; ++i)
    if (tok[i]) {
      load_small(tr0[i], tre[i], tpb[i]);
      issue_qg(tr0[i], tre[i], i);
      store_small(i);
    }
  RA_WAIT_VMCNT(0);
  __syncthreads();

  // 32-bit copies for the per-tile tests (positions are below 2^30, checked on the host): the
  // first query able to see the wave's first and last key, and each lane's key
  const int wkey = static_cast<int>(wkey0);
  const bool wk_ok = wk0 < p.Lb;
  int wq_first = wkey, wq_last = wkey + KW - 1;
  int kfq[NKB];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) kfq[kb] = wkey + kb * 32 + l32;
  if constexpr (CBLK) {
    wq_first = causal_first_query(wkey, coff, p.causal);
    wq_last = causal_first_query(wkey + KW - 1, coff, p.causal);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) kfq[kb] = causal_first_query(wkey + kb * 32 + l32, coff, p.causal);
  }
  int slot = 0;
  while (tok[0]) {
    const int row0 = tr0[0], rend = tre[0], pbase = tpb[0];
    const int ahead = slot + NS - 1 >= NS ? slot - 1 : slot + NS - 1;   // (slot + NS - 1) % NS
    const bool issue = tok[NS - 1];
    if (issue) {
      load_small(tr0[NS - 1], tre[NS - 1], tpb[NS - 1]);   // before the copies: its wait spares them
      issue_qg(tr0[NS - 1], tre[NS - 1], ahead);
    }
    const int buf = slot;
    const __bf16* Qt = sQ[buf];
    const __bf16* Gt = sG[buf];
    const int qpos0 = row0 + pbase;                      // global position of the tile's row 0
    const int nq = (rend - row0) < BQ ? (rend - row0) : BQ;
    bool wave_active = wk_ok && !(CAUSAL && qpos0 + nq - 1 < (CBLK ? wq_first : wkey));
    bool seg_mask = HAS_SEG;   // some pair of the tile may lie in different segments
    if constexpr (HAS_SEG) {
      const int tlo = __builtin_amdgcn_readfirstlane(sTileSeg[buf][0]);
      const int thi = __builtin_amdgcn_readfirstlane(sTileSeg[buf][1]);
      wave_active = wave_active && tlo <= kseg_hi && thi >= kseg_lo;
      seg_mask = !(tlo == thi && kseg_lo == kseg_hi && tlo == kseg_lo);
    }
    if (wave_active) {
      // rows past the rank's end carry -inf in sL, so their P is 0 and only the causal and
      // segment masks need the selects
      const bool need_mask = seg_mask || (CAUSAL && (CBLK ? wq_last : wkey + KW - 1) > qpos0);
      int krel[NKB];   // first query row (of the tile) that sees the lane's key, clamped to [0, BQ]
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const int rel = (CBLK ? kfq[kb] : wkey + kb * 32 + l32) - qpos0;
        krel[kb] = rel < 0 ? 0 : (rel > BQ ? BQ : rel);
      }
#pragma unroll
      for (int qb = 0; qb < BQ / 32; ++qb) {
        // the 16 query rows this lane holds: qr(v) = qb*32 + 8*(v/4) + 4*hh + v%4;
        // -lse * log2e and -Delta of each start the accumulators
        float nl[16], dl[16];
        int qs[16];
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int base = qb * 32 + 8 * g4 + 4 * hh;
          const f32x4 x = *reinterpret_cast<const f32x4*>(&sL[buf][base]);
          const f32x4 y = *reinterpret_cast<const f32x4*>(&sDl[buf][base]);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            nl[4 * g4 + i] = x[i];
            dl[4 * g4 + i] = y[i];
          }
          if (HAS_SEG && need_mask) {
            const int4 z = *reinterpret_cast<const int4*>(&sSg[buf][base]);
            qs[4 * g4 + 0] = z.x;
            qs[4 * g4 + 1] = z.y;
            qs[4 * g4 + 2] = z.z;
            qs[4 * g4 + 3] = z.w;
          }
        }
        f32x16 S[NKB], G[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            S[kb][v] = HAS_BIAS ? nl[v] + kbias[kb] : nl[v];
            G[kb][v] = dl[v];
          }
        // raised wave priority while the score products issue (as in dQ)
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const bf16x8 aq = lds_read_swz<D>(Qt, qb * 32 + l32, 2 * kk + hh);
          const bf16x8 ag = lds_read_swz<D>(Gt, qb * 32 + l32, 2 * kk + hh);
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) {
            S[kb] = mfma32(aq, Kf[kb][kk], S[kb]);
            G[kb] = mfma32(ag, Vf[kb][kk], G[kb]);
          }
        }
        __builtin_amdgcn_s_setprio(0);
        // masked scores become -inf (then P = 0) in a pass of their own, so that tiles
        // without masks run the loop below with no selects
        if (need_mask) {
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) {
            // query rows are qr0(v) + 4 * hh with qr0 a constant of v: compare against the shifted
            // first row, so the row numbers never occupy registers
            const int krel4 = krel[kb] - 4 * hh;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              bool vis = true;
              if constexpr (CAUSAL) vis = krel4 <= qb * 32 + 8 * (v >> 2) + (v & 3);
              if constexpr (HAS_SEG) vis = vis && ksg[kb] == qs[v];
              S[kb][v] = vis ? S[kb][v] : -INFINITY;
            }
          }
        }
        bf16x8 Pb[NKB][2], Sb[NKB][2];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            float pe[8], de[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const int v = 8 * st + i;
              const float pr = __builtin_amdgcn_exp2f(S[kb][v]);
              pe[i] = pr;
              de[i] = pr * G[kb][v];
            }
            Pb[kb][st] = pack_bf16x8(pe);
            Sb[kb][st] = pack_bf16x8(de);
            if constexpr (KEYSUM) dsum[kb] += ((de[0] + de[1]) + (de[2] + de[3])) + ((de[4] + de[5]) + (de[6] + de[7]));
          }
        // dV^T += dO^T . P ;  dK^T += Q^T . dS
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const bf16x8 ag = lds_read_a_transposed_swz<D>(Gt, qb * 32, st, db * 32, lane);
            const bf16x8 aq = lds_read_a_transposed_swz<D>(Qt, qb * 32, st, db * 32, lane);
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
              dV[db][kb] = mfma32(ag, Pb[kb][st], dV[db][kb]);
              dK[db][kb] = mfma32(aq, Sb[kb][st], dK[db][kb]);
            }
          }
      }
    }

    // the next tile's copies must have landed; this iteration's may stay in flight
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
    slot = slot + 1 == NS ? 0 : slot + 1;
#pragma unroll
    for (int i = 0; i + 1 < NS; ++i) {
      tok[i] = tok[i + 1];
      tr0[i] = tr0[i + 1];
      tre[i] = tre[i + 1];
      tpb[i] = tpb[i + 1];
    }
    tok[NS - 1] = next_tile();
    tr0[NS - 1] = walk.row0;
    tre[NS - 1] = walk.rend;
    tpb[NS - 1] = walk.pos_base;
  }

  // per-key sums of dS (lanes l and l + 32 hold the same key for different queries): written, or in a
  // ring step added to the sums the block carries
  if constexpr (KEYSUM) {
    if (p.dbias_keys) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const float t = pair_sum(dsum[kb]);
        const int64_t krow = wk0 + kb * 32 + l32;
        if (hh == 0 && krow < p.Lb) {
          float* dst = p.dbias_keys + (static_cast<int64_t>(b) * p.H + h) * p.Lk + static_cast<int64_t>(j) * p.Lb + krow;
          *dst = (STEP && !p.init_dkv) ? *dst + t : t;
        }
      }
    }
  }
  // dK^T / dV^T accumulators: lane holds d = db*32 + 8*(v/4) + 4*hh + v%4 of key column l32
  if constexpr (STEP) {
    // unscaled float32 sums back to caller memory
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const int64_t krow = wk0 + kb * 32 + l32;
      if (krow >= p.Lb) continue;
      const int64_t off = row_offset(b, krow, h, p.Lk, p.H, D);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
          f32x4 x, y;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            x[i] = dK[db][kb][4 * v4 + i];
            y[i] = dV[db][kb][4 * v4 + i];
          }
          *reinterpret_cast<f32x4*>(p.dk_acc + off + db * 32 + 8 * v4 + 4 * hh) = x;
          *reinterpret_cast<f32x4*>(p.dv_acc + off + db * 32 + 8 * v4 + 4 * hh) = y;
        }
    }
    return;
  }
  __bf16* __restrict__ dkp = static_cast<__bf16*>(p.dk);
  __bf16* __restrict__ dvp = static_cast<__bf16*>(p.dv);
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    const int64_t krow = wk0 + kb * 32 + l32;
    if (krow >= p.Lb) continue;
    const int64_t off = row_offset(b, static_cast<int64_t>(j) * p.Lb + krow, h, p.Lk, p.H, D);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        bf16x4 k4, v4v;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          k4[i] = (__bf16)(dK[db][kb][4 * v4 + i] * p.scale);
          v4v[i] = (__bf16)(dV[db][kb][4 * v4 + i]);
        }
        *reinterpret_cast<bf16x4*>(dkp + off + db * 32 + 8 * v4 + 4 * hh) = k4;
        *reinterpret_cast<bf16x4*>(dvp + off + db * 32 + 8 * v4 + 4 * hh) = v4v;
      }
  }
}

// ================================================================== launcher
template <int D, int NKB, bool STEP>
hipError_t dkdv_d(const Params& p, hipStream_t st) {
  constexpr int OCC = D == 64 ? 2 : 1;
  constexpr int BKW = kWaves * 32 * NKB;
  const int64_t grid = static_cast<int64_t>(p.n_ring) * ((p.Lb + BKW - 1) / BKW) * p.B * p.H;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
#define RA_L(C, B, S) \
  hipLaunchKernelGGL((dkdv_mfma_kernel<D, NKB, C, B, S, OCC, STEP>), dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, st, p)
  RA_SELECT_FLAGS(RA_L);
#undef RA_L
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_dkdv_mfma(const Params& p, hipStream_t st) {
  if (p.D == 64) return dkdv_d<64, 1, false>(p, st);
  if (p.D == 128) return dkdv_d<128, 1, false>(p, st);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_dkdv_step_mfma(const Params& p, hipStream_t st) {
  if (p.D == 64) return dkdv_d<64, 1, true>(p, st);
  if (p.D == 128) return dkdv_d<128, 1, true>(p, st);
  return hipErrorInvalidValue;
}

}  // namespace ra
