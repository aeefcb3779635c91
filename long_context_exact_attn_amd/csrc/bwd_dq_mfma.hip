// Backward blockwise ring attention, dQ kernel: bfloat16 in / float32 accumulate, MFMA on gfx950.
//
// The probabilities are recomputed from the saved logsumexp, P = exp(s - lse),
// so no score matrix is ever stored (the recompute policy of the pages'
// blockwise_kwargs).  Two kernels, each owning the rows it writes, so the
// result is deterministic and needs no atomics: this file's and the one in
// bwd_dkdv_mfma.hip (dK, dV).  The two kernels live in separate files so that neither's code
// shape can change how the compiler allocates the other's registers.
//
// dQ kernel -- the forward's tiling: one workgroup owns a query tile (Q, dO,
//   lse, Delta in VGPRs) and K/V tiles stream through LDS in ring order:
//     S^T = K . Q^T,  dP^T = V . dO^T,  dS^T = P^T (dP^T - Delta),  dQ^T += K^T . dS^T
//   with P = exp2(S * scale * log2e + bias - lse * log2e): Q held pre-multiplied by scale * log2e
//   (rounded to bfloat16), accumulators started at bias - lse * log2e and -Delta, so that the matrix
//   unit delivers the exponent and dP - Delta directly.
#include <type_traits>

#include "mfma_util.cuh"


namespace ra {
namespace {

// ================================================================== dQ (query tiles stationary)
constexpr int kBkDq = 64;   // keys per K/V tile

// STEP: one backward ring step (ra_blockwise_attn_bwd_step): the keys held are one block at
// global positions kv_pos0 + j, and dQ is summed into float32 caller memory (unscaled).
// CM: causal mode, 0 none, 1 token level, 2 causal blocks of p.causal > 1 tokens.
template <int D, int NQB, int CM, bool HAS_BIAS, bool HAS_SEG, int OCC, bool STEP>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(OCC, OCC))) void dq_mfma_kernel(Params p) {
  constexpr bool CAUSAL = CM != 0;
  constexpr bool CBLK = CM == 2;
  constexpr int BK = kBkDq;
  constexpr int QW = 32 * NQB;         // queries per wave
  constexpr int BQ = kWaves * QW;      // queries per workgroup
  constexpr int KK = D / 16;
  constexpr int DB = D / 32;
#ifndef RA_DQ_NS
#define RA_DQ_NS 2
#endif
  // LDS stages of the K/V ring (three measured 0.5% slower once the walk was unrolled and the copies took
  // the uniform-base form; before that they had gained 4.5%)
  constexpr int NS = D == 64 ? RA_DQ_NS : 2;
  constexpr int TILE = BK * D;         // unpadded, swizzled
  constexpr int NSEG = TILE * 2 / 1024 / kWaves;   // 1 KiB direct-copy segments per wave per tile
  static_assert(NSEG * 1024 * kWaves == TILE * 2, "tile must split into 1 KiB segments");

  __shared__ __attribute__((aligned(16))) __bf16 sK[NS][TILE];
  __shared__ __attribute__((aligned(16))) __bf16 sV[NS][TILE];
  __shared__ float sBias[NS][BK];
  __shared__ __attribute__((aligned(16))) int sSeg[NS][BK];
  __shared__ int sSegRange[NS][2];   // smallest and largest segment id among the tile's keys
  __shared__ int sWaveSeg[kWaves][2];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  // tile order (grid = B * H * n_qt): the heaviest query tiles of a head first; one (batch, head) per
  // XCD at a time for one rank's queries (or one ring step), whose tiles carry similar work, pairs
  // fastest for the whole ring, where a causal mask makes the work fall from tile to tile (measured
  // both ways on each kind of launch)
  const int64_t n_qt_blk = (p.Lb + BQ - 1) / BQ;
  const int64_t n_qt = (p.ring_rank < 0 ? p.n_ring : 1) * n_qt_blk;
  const HeadTile ht = head_tile(blockIdx.x, p.B * p.H, n_qt, p.ring_rank >= 0);
  const int hb = ht.hb;
  const int64_t t = n_qt - 1 - ht.t;
  const int b = hb / p.H, h = hb % p.H;
  const int r_local = static_cast<int>(t / n_qt_blk);
  const int64_t qa = (t % n_qt_blk) * BQ;
  const int r = p.ring_rank < 0 ? r_local : p.ring_rank;
  const int64_t qrow_base = static_cast<int64_t>(r_local) * p.Lb;
  // position of the tile's row 0 relative to key 0 of the keys held
  const int64_t pos0 = (STEP ? p.q_pos0 - p.kv_pos0 : static_cast<int64_t>(r) * p.Lb) + qa;
  const int64_t nrows = (p.Lb - qa) < BQ ? (p.Lb - qa) : BQ;

  const __bf16* __restrict__ qp = static_cast<const __bf16*>(p.q);
  const __bf16* __restrict__ kp = static_cast<const __bf16*>(p.k);
  const __bf16* __restrict__ vp = static_cast<const __bf16*>(p.v);
  const __bf16* __restrict__ gp = static_cast<const __bf16*>(p.dout);
  // segment ids on positions relative to the keys held (kv_pos0 = 0 outside a ring step)
  const int* __restrict__ ids = HAS_SEG ? p.seg + static_cast<int64_t>(b) * p.seg_len + p.kv_pos0 : nullptr;

  const int64_t wrow0 = qa + wave * QW;
  const int64_t wpos0 = pos0 + wave * QW;
  const int64_t wvalid = p.Lb - wrow0;
  bf16x8 Qf[NQB][KK], Gf[NQB][KK];
  float lse2[NQB], dlt[NQB];
  int qseg[NQB];
#pragma unroll
  for (int nb = 0; nb < NQB; ++nb) {
    const int64_t row = wrow0 + nb * 32 + l32;
    const bool ok = row < p.Lb;
    const int64_t off = row_offset(b, qrow_base + (ok ? row : 0), h, p.Lq, p.H, D);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const bf16x8 x = *reinterpret_cast<const bf16x8*>(qp + off + 16 * kk + 8 * hh);
      const bf16x8 y = *reinterpret_cast<const bf16x8*>(gp + off + 16 * kk + 8 * hh);
      Qf[nb][kk] = ok ? scale_bf16x8(x, p.scale * kLog2e) : bf16x8{};
      Gf[nb][kk] = ok ? y : bf16x8{};
    }
    const int64_t li = (static_cast<int64_t>(b) * p.H + h) * p.Lq + qrow_base + (ok ? row : 0);
    const float L = p.lse[li];
    // rows that do not exist or see no key get P = 0 everywhere (exp2(-inf))
    lse2[nb] = (ok && L != -INFINITY) ? L * kLog2e : INFINITY;
    dlt[nb] = ok ? p.delta[li] : 0.f;
    qseg[nb] = (HAS_SEG && ok) ? ids[wpos0 + nb * 32 + l32] : 0;
  }
  // the wave's and the workgroup's range of query segment ids: K/V tiles with no key id in the
  // workgroup's range are passed over, and a wave skips the products of a tile with none in its own
  int gseg_lo = 0, gseg_hi = 0, qseg_lo = 0, qseg_hi = 0;
  if constexpr (HAS_SEG) {
    int lo = INT32_MAX, hi = INT32_MIN;
#pragma unroll
    for (int nb = 0; nb < NQB; ++nb)
      if (wrow0 + nb * 32 + l32 < p.Lb) {
        lo = min(lo, qseg[nb]);
        hi = max(hi, qseg[nb]);
      }
    qseg_lo = __builtin_amdgcn_readfirstlane(wave_min_i32(lo));
    qseg_hi = __builtin_amdgcn_readfirstlane(wave_max_i32(hi));
    wg_id_range(qseg_lo, qseg_hi, sWaveSeg, wave, lane, gseg_lo, gseg_hi);
  }

  // starting values of the score and dP accumulators: -lse * log2e and -Delta of the lane's query
  // (with a bias the score start is formed per tile, bias - lse * log2e)
  f32x16 s_init[NQB], g_init[NQB];
#pragma unroll
  for (int nb = 0; nb < NQB; ++nb)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      s_init[nb][v] = -lse2[nb];
      g_init[nb][v] = -dlt[nb];
    }
  f32x16 dQ[DB][NQB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int nb = 0; nb < NQB; ++nb) dQ[db][nb] = f32x16{};
  if constexpr (STEP) {
    if (!p.init_dq) {
      // the sums of earlier ring steps: lane holds d = db*32 + 8*(v/4) + 4*hh + v%4 of its query
#pragma unroll
      for (int nb = 0; nb < NQB; ++nb) {
        const int64_t row = wrow0 + nb * 32 + l32;
        if (row >= p.Lb) continue;
        const float* src = p.dq_acc + row_offset(b, row, h, p.Lq, p.H, D);
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int v4 = 0; v4 < 4; ++v4) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(src + db * 32 + 8 * v4 + 4 * hh);
#pragma unroll
            for (int i = 0; i < 4; ++i) dQ[db][nb][4 * v4 + i] = x[i];
          }
      }
    }
  }

  // K/V tiles: direct global -> LDS copies into a ring of NS stages, as in the forward
  const int64_t kv_bh = (static_cast<int64_t>(b) * p.Lk * p.H + h) * D;
  const int64_t kstride = static_cast<int64_t>(p.H) * D;
  // (64-bit addresses per copy: the uniform-base form of the forward and dK/dV measured 2% slower here)
  int grow_[NSEG], goff[NSEG], goff0[NSEG];
#pragma unroll
  for (int jj = 0; jj < NSEG; ++jj) {
    const int byte = (wave * NSEG + jj) * 1024 + lane * 16;
    const int row = byte / (2 * D);
    const int chunk = ((byte % (2 * D)) >> 4) ^ swz_key<D>(row);
    grow_[jj] = row;
    goff[jj] = row * static_cast<int>(kstride) + chunk * 8;   // < 64 * H * D, checked on the host
    goff0[jj] = chunk * 8;
  }
  // (raw values are kept until the store, so that the wait for these loads lands there)
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
      if constexpr (HAS_SEG) sreg = ids[key];
    }
  };
  auto store_small = [&](int slot) {
    if (tid < BK) {
      if constexpr (HAS_BIAS) sBias[slot][tid] = kok ? breg * kLog2e : 0.f;
      if constexpr (HAS_SEG) {
        const int sid = kok ? sreg : 0;
        sSeg[slot][tid] = sid;
        const int lo = wave_min_i32(kok ? sid : INT32_MAX);   // BK = 64: one wave holds the tile
        const int hi = wave_max_i32(kok ? sid : INT32_MIN);
        if (tid == 0) {
          sSegRange[slot][0] = lo;
          sSegRange[slot][1] = hi;
        }
      }
    }
  };
  // head_dim 64 without bias or segment ids: copies from the tile's wave-uniform base plus each lane's fixed
  // offset, full tiles in a branch of their own (no per-chunk selects); measured, as for the forward
  constexpr bool kUniformCopies = D == 64 && !HAS_BIAS && !HAS_SEG;
  auto issue_kv = [&](int key0, int kend, int slot) {
    const __bf16* kb = kp + kv_bh + static_cast<int64_t>(key0) * kstride;
    const __bf16* vb = vp + kv_bh + static_cast<int64_t>(key0) * kstride;
    if constexpr (kUniformCopies) {
      if (key0 + BK <= kend) {
#pragma unroll
        for (int jj = 0; jj < NSEG; ++jj) {
          const unsigned off = 2u * static_cast<unsigned>(goff[jj]);
          dma16_sb(kb, off, &sK[slot][(wave * NSEG + jj) * 512]);
          dma16_sb(vb, off, &sV[slot][(wave * NSEG + jj) * 512]);
        }
      } else {
        const int nvalid = kend - key0;
#pragma unroll
        for (int jj = 0; jj < NSEG; ++jj) {
          const unsigned off = 2u * static_cast<unsigned>(grow_[jj] < nvalid ? goff[jj] : goff0[jj]);
          dma16_sb(kb, off, &sK[slot][(wave * NSEG + jj) * 512]);
          dma16_sb(vb, off, &sV[slot][(wave * NSEG + jj) * 512]);
        }
      }
    } else {
      const bool full = key0 + BK <= kend;
      const int nvalid = kend - key0;
#pragma unroll
      for (int jj = 0; jj < NSEG; ++jj) {
        const int off = (full || grow_[jj] < nvalid) ? goff[jj] : goff0[jj];
        dma16(kb + off, &sK[slot][(wave * NSEG + jj) * 512]);
        dma16(vb + off, &sV[slot][(wave * NSEG + jj) * 512]);
      }
    }
  };

  // causal limits: relative positions have their origin at global position kv_pos0 (0 outside a
  // ring step); the walk stops after the last key the workgroup's last query can see
  const int coff = static_cast<int>(p.kv_pos0);
  RingWalk walk;
  walk.begin(p.n_ring, r, p.Lb, CAUSAL,
             CBLK && nrows > 0 ? causal_last_key(static_cast<int>(pos0 + nrows - 1), coff, p.causal) : pos0 + nrows - 1);
  SegTileFilter filt;   // with segment ids: pass over tiles sharing no id with the queries
  auto next_tile = [&]() -> bool {
    while (walk.next<BK>()) {
      if constexpr (!HAS_SEG) return true;
      static_assert(BK == 64, "the segment filter works in 64-key tiles");
      const int skip = filt.skip(ids, walk.key0, walk.kend, gseg_lo, gseg_hi, lane);
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
#pragma unroll
  for (int i = 0; i < NS - 1; ++i)
    if (tok[i]) {
      load_small(tk0[i], tke[i]);
      issue_kv(tk0[i], tke[i], i);
      store_small(i);
    }
  RA_WAIT_VMCNT(0);
  __syncthreads();

  // 32-bit copies of the wave's first query position and last existing row (token positions
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
  // one step of the walk; for head_dim 64 without bias or segment ids it is unrolled over the ring
  // stages, so each stage's LDS addresses are compile-time offsets
  constexpr bool kUnrollWalk = D == 64 && !HAS_BIAS && !HAS_SEG;
  auto step = [&](auto slot_c) {
    const int slot = slot_c;   // a compile-time constant when the walk is unrolled
    const int key0 = tk0[0], kend = tke[0];
    const int ahead = slot + NS - 1 >= NS ? slot - 1 : slot + NS - 1;   // (slot + NS - 1) % NS
    const bool issue = tok[NS - 1];
    if (issue) {
      load_small(tk0[NS - 1], tke[NS - 1]);
      issue_kv(tk0[NS - 1], tke[NS - 1], ahead);
    }
    const int buf = slot;

    const __bf16* Kt = sK[buf];
    const __bf16* Vt = sV[buf];
    bool wave_active = wlast >= 0 && !(CAUSAL && key0 > (CBLK ? wlim_last : wpos + wlast));
    bool seg_mask = HAS_SEG;   // some pair of the tile may lie in different segments
    if constexpr (HAS_SEG) {
      const int klo = __builtin_amdgcn_readfirstlane(sSegRange[buf][0]);
      const int khi = __builtin_amdgcn_readfirstlane(sSegRange[buf][1]);
      wave_active = wave_active && klo <= qseg_hi && khi >= qseg_lo;
      seg_mask = !(klo == khi && qseg_lo == qseg_hi && klo == qseg_lo);
    }
    if (wave_active) {
      f32x16 S[2][NQB], G[2][NQB];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < NQB; ++nb) {
          if constexpr (HAS_BIAS) {
#pragma unroll
            for (int v = 0; v < 16; ++v)
              S[mb][nb][v] = sBias[buf][mb * 32 + 8 * (v >> 2) + 4 * hh + (v & 3)] + s_init[nb][v];
          } else {
            S[mb][nb] = s_init[nb];
          }
          G[mb][nb] = g_init[nb];
        }
      // a raised wave priority while the score products issue keeps the matrix unit fed
      // while the other wave on the SIMD does its exponentials (measured: ~2% on dQ)
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const bf16x8 ak = lds_read_swz<D>(Kt, mb * 32 + l32, 2 * kk + hh);
          const bf16x8 av = lds_read_swz<D>(Vt, mb * 32 + l32, 2 * kk + hh);
#pragma unroll
          for (int nb = 0; nb < NQB; ++nb) {
            S[mb][nb] = mfma32(ak, Qf[nb][kk], S[mb][nb]);
            G[mb][nb] = mfma32(av, Gf[nb][kk], G[mb][nb]);
          }
        }
      }
      __builtin_amdgcn_s_setprio(0);

      const bool need_mask = seg_mask || (key0 + BK > kend) || (CAUSAL && key0 + BK - 1 > (CBLK ? wlim_first : wpos));
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
      bf16x8 dS[NQB][2][2];
#pragma unroll
      for (int nb = 0; nb < NQB; ++nb) {
        // key kr of the tile is visible to this lane's query iff kr <= klim and (segments) ids match
        int klim = BK - 1;
        if (need_mask) {
          klim = (kend - key0 < BK ? kend - key0 : BK) - 1;
          if constexpr (CAUSAL) {
            // the query's last visible key, relative to key 0
            const int rel = CBLK ? qlim[nb] - key0 : wpos - key0 + nb * 32 + l32;
            klim = rel < klim ? (rel < -1 ? -1 : rel) : klim;
          }
        }
        // masked scores become -inf (then P = 0) in a pass of their own, so that tiles
        // without masks run the loop below with no selects
        if (need_mask) {
          // key rows are kr0(v) + 4 * hh with kr0 a constant of v: compare against the shifted limit
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
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            float e[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const int v = 8 * st + i;
              e[i] = __builtin_amdgcn_exp2f(S[mb][nb][v]) * G[mb][nb][v];
            }
            dS[nb][mb][st] = pack_bf16x8(e);
          }
      }

      // dQ^T += K^T . dS^T
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const bf16x8 a = lds_read_a_transposed_swz<D>(Kt, mb * 32, st, db * 32, lane);
#pragma unroll
            for (int nb = 0; nb < NQB; ++nb) dQ[db][nb] = mfma32(a, dS[nb][mb][st], dQ[db][nb]);
          }
    }

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
    // unscaled float32 sums back to caller memory
#pragma unroll
    for (int nb = 0; nb < NQB; ++nb) {
      const int64_t row = wrow0 + nb * 32 + l32;
      if (row >= p.Lb) continue;
      float* dst = p.dq_acc + row_offset(b, row, h, p.Lq, p.H, D);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
          f32x4 x;
#pragma unroll
          for (int i = 0; i < 4; ++i) x[i] = dQ[db][nb][4 * v4 + i];
          *reinterpret_cast<f32x4*>(dst + db * 32 + 8 * v4 + 4 * hh) = x;
        }
    }
    return;
  }
  __bf16* __restrict__ dqp = static_cast<__bf16*>(p.dq);
#pragma unroll
  for (int nb = 0; nb < NQB; ++nb) {
    const int64_t row = wrow0 + nb * 32 + l32;
    if (row >= p.Lb) continue;
    __bf16* dst = dqp + row_offset(b, qrow_base + row, h, p.Lq, p.H, D);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        bf16x4 o4;
#pragma unroll
        for (int i = 0; i < 4; ++i) o4[i] = (__bf16)(dQ[db][nb][4 * v4 + i] * p.scale);
        *reinterpret_cast<bf16x4*>(dst + db * 32 + 8 * v4 + 4 * hh) = o4;
      }
  }
}

// ================================================================== launcher
// head_dim 64 fits two waves per SIMD without spilling; head_dim 128 keeps one
template <int D, int NQB, bool STEP>
hipError_t dq_d(const Params& p, hipStream_t st) {
  constexpr int OCC = D == 64 ? 2 : 1;
  constexpr int BQ = kWaves * 32 * NQB;
  const int64_t grid = (p.ring_rank < 0 ? p.n_ring : 1) * ((p.Lb + BQ - 1) / BQ) * p.B * p.H;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
#define RA_L(C, B, S) \
  hipLaunchKernelGGL((dq_mfma_kernel<D, NQB, C, B, S, OCC, STEP>), dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, st, p)
  RA_SELECT_FLAGS(RA_L);
#undef RA_L
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_dq_mfma(const Params& p, hipStream_t st) {
  if (p.D == 64) return dq_d<64, 1, false>(p, st);
  if (p.D == 128) return dq_d<128, 1, false>(p, st);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_dq_step_mfma(const Params& p, hipStream_t st) {
  if (p.D == 64) return dq_d<64, 1, true>(p, st);
  if (p.D == 128) return dq_d<128, 1, true>(p, st);
  return hipErrorInvalidValue;
}

}  // namespace ra
