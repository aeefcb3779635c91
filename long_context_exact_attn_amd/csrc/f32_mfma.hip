// Float32 attention on the matrix unit: forward, dK/dV and dQ kernels for float32 tensors, with
// float32 products throughout (v_mfma_f32_16x16x4_f32, float32 operands and accumulation) and no
// bfloat16 rounding anywhere.  They compute what the bfloat16 kernels compute -- exact softmax
// attention of a query block against the K/V blocks of a ring, merged with an online softmax
// ("手把手拆解RingAttention", section 1) -- and follow the same ring walks.
//
// Tiling.  A workgroup holds 16 stationary rows (queries in the forward and dQ, keys in dK/dV) in
// all four of its waves; the waves take the tiles of the walk (16 rows of the other side) in turn
// and the workgroup adds their partial results in a fixed order at the end, so results are
// deterministic.  One 16x16 score tile is D/4 matrix products; the probability tile then feeds the
// second product straight from the accumulator:
//  * v_mfma_f32_16x16x4_f32 operands: lane l holds A[l & 15][l >> 4] and B[l >> 4][l & 15]; the
//    result C[4 (l >> 4) + v][l & 15] sits in element v of lane l.
//  * Score products contract over the head dimension.  Both operands are read as rows: lane l reads
//    its row l & 15 in 16-byte pieces at d = 16 c + 4 (l >> 4), and product 4 c + e uses element e.
//    The same permutation of d on both sides leaves the dot product unchanged.
//  * The second product contracts over the tile's 16 rows of the other side, four per product:
//    lane group g = l >> 4 supplies row 4 g + v in product v, which is exactly the score element v
//    the lane already holds.
#include "ra_common.cuh"

namespace ra {
namespace {

constexpr int kRows = 16;     // stationary rows per workgroup, and rows per tile of the walk
constexpr int kWaves = 4;     // waves per workgroup
constexpr int kThreads = 64 * kWaves;

__device__ __forceinline__ f32x4 mma(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// the lane's 16-byte pieces of one row (d = 16 c + 4 g .. + 3), zero when the row does not exist
template <int D>
__device__ __forceinline__ void load_frag(f32x4 (&x)[D / 16], const float* row, bool ok, int g) {
#pragma unroll
  for (int c = 0; c < D / 16; ++c)
    x[c] = ok ? *reinterpret_cast<const f32x4*>(row + 16 * c + 4 * g) : f32x4{0.f, 0.f, 0.f, 0.f};
}

// sum over the four lane groups (lanes l, l ^ 16, l ^ 32, l ^ 48)
__device__ __forceinline__ float group_sum(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}
__device__ __forceinline__ float group_max(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}

// Stationary query tile: 16 queries of one (batch, head); the heaviest causal tiles start first.
struct QueryTile {
  int b, h, nrows;
  int64_t qrow;     // local row of query 0 in q / out / lse
  int pos0;         // global position of query 0
  int rank;         // ring rank of the queries
  __device__ QueryTile(const Params& p) {
    const int HB = p.B * p.H;
    const int64_t n_qt_blk = (p.Lb + kRows - 1) / kRows;
    const int64_t n_qt = (p.ring_rank < 0 ? p.n_ring : 1) * n_qt_blk;
    const int64_t wg = blockIdx.x;
    const int hb = static_cast<int>(wg % HB);
    const int64_t t = n_qt - 1 - wg / HB;
    b = hb / p.H;
    h = hb % p.H;
    const int r_local = static_cast<int>(t / n_qt_blk);
    const int64_t qa = (t % n_qt_blk) * kRows;
    rank = p.ring_rank < 0 ? r_local : p.ring_rank;
    qrow = static_cast<int64_t>(r_local) * p.Lb + qa;
    pos0 = static_cast<int>(static_cast<int64_t>(rank) * p.Lb + qa);
    nrows = static_cast<int>((p.Lb - qa) < kRows ? (p.Lb - qa) : kRows);
  }
};

// ------------------------------------------------------------------ forward
// S^T = K Q^T (lane l: query l & 15, keys 4 g + v), online softmax per wave, O^T += V^T P^T; the
// four waves' (m, l, O) are merged at the end by the online-softmax identity.
template <int D, bool CAUSAL, bool HAS_BIAS, bool HAS_SEG>
__global__ __launch_bounds__(kThreads) void fwd_f32_kernel(Params p) {
  constexpr int NC = D / 16;
  __shared__ float sO[kWaves][kRows][D];
  __shared__ float sM[kWaves][kRows];
  __shared__ float sL[kWaves][kRows];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, col = lane & 15;
  const QueryTile t(p);
  const float* qp = static_cast<const float*>(p.q);
  const float* kp = static_cast<const float*>(p.k);
  const float* vp = static_cast<const float*>(p.v);
  const bool qok = col < t.nrows;
  const int qpos = t.pos0 + col;
  f32x4 qf[NC];
  load_frag<D>(qf, qp + row_offset(t.b, t.qrow + (qok ? col : 0), t.h, p.Lq, p.H, D), qok, g);
  const int qseg = (HAS_SEG && qok) ? p.seg[static_cast<int64_t>(t.b) * p.Lk + qpos] : 0;
  const int qlim = CAUSAL ? causal_last_key(qpos, 0, p.causal) : 0;   // last visible key
  const float c = p.scale * kLog2e;
  const float* brow = HAS_BIAS ? p.bias + static_cast<int64_t>(t.h) * p.bias_len : nullptr;
  const int32_t* srow = HAS_SEG ? p.seg + static_cast<int64_t>(t.b) * p.Lk : nullptr;

  f32x4 o[NC];
#pragma unroll
  for (int dt = 0; dt < NC; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, lpart = 0.f;   // lpart: this lane's share (keys 4 g + v) of the row sum

  RingWalk walk;
  const int plast = t.pos0 + t.nrows - 1;
  walk.begin(p.n_ring, t.rank, p.Lb, CAUSAL, CAUSAL ? causal_last_key(plast, 0, p.causal) : plast);
  for (int n = 0; walk.next<kRows>(); ++n) {
    if ((n & (kWaves - 1)) != wave) continue;
    const int key0 = walk.key0, kend = walk.kend;
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    {
      const int key = key0 + col;
      f32x4 kf[NC];
      load_frag<D>(kf, kp + row_offset(t.b, key < kend ? key : key0, t.h, p.Lk, p.H, D), key < kend, g);
#pragma unroll
      for (int cc = 0; cc < NC; ++cc)
#pragma unroll
        for (int e = 0; e < 4; ++e) s = mma(kf[cc][e], qf[cc][e], s);
    }
    float x[4];
    float tmax = -INFINITY;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int key = key0 + 4 * g + v;
      bool vis = qok && key < kend;
      if (CAUSAL) vis = vis && key <= qlim;
      if (HAS_SEG) vis = vis && srow[key < kend ? key : key0] == qseg;
      float y = s[v] * c;
      if (HAS_BIAS) y += brow[(key < kend ? key : key0) % p.bias_len] * kLog2e;
      x[v] = vis ? y : -INFINITY;
      tmax = fmaxf(tmax, x[v]);
    }
    const float mnew = fmaxf(m, group_max(tmax));
    const float alpha = mnew == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m - mnew);
    const float msub = mnew == -INFINITY ? 0.f : mnew;
    m = mnew;
    lpart *= alpha;
#pragma unroll
    for (int dt = 0; dt < NC; ++dt) o[dt] *= alpha;
    float pr[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      pr[v] = __builtin_amdgcn_exp2f(x[v] - msub);
      lpart += pr[v];
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int key = key0 + 4 * g + v;
      const float* vrow = vp + row_offset(t.b, key < kend ? key : key0, t.h, p.Lk, p.H, D);
#pragma unroll
      for (int dt = 0; dt < NC; ++dt) o[dt] = mma(key < kend ? vrow[16 * dt + col] : 0.f, pr[v], o[dt]);
    }
  }

  // merge the four waves: weights exp2(m_w - M) against the largest maximum M
  const float l = group_sum(lpart);
#pragma unroll
  for (int dt = 0; dt < NC; ++dt)
#pragma unroll
    for (int v = 0; v < 4; ++v) sO[wave][col][16 * dt + 4 * g + v] = o[dt][v];
  if (g == 0) {
    sM[wave][col] = m;
    sL[wave][col] = l;
  }
  __syncthreads();
  const int q = threadIdx.x >> 4, dl = threadIdx.x & 15;   // 16 threads per query
  if (q >= t.nrows) return;
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sM[w][q]);
  float wt[kWaves], L = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    wt[w] = sM[w][q] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sM[w][q] - M);
    L += wt[w] * sL[w][q];
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  float* op = static_cast<float*>(p.out) + row_offset(t.b, t.qrow + q, t.h, p.Lq, p.H, D);
  for (int d = dl; d < D; d += 16) {
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) acc += wt[w] * sO[w][q][d];
    op[d] = acc * inv;
  }
  if (dl == 0)
    p.lse[(static_cast<int64_t>(t.b) * p.H + t.h) * p.Lq + t.qrow + q] =
        L > 0.f ? (M + __builtin_amdgcn_logf(L)) * kLn2 : -INFINITY;
}

// ------------------------------------------------------------------ backward dK/dV
// 16 keys held; S = Q K^T and dP = dO V^T (lane l: key l & 15, queries 4 g + v), then
// dV^T += dO^T P and dK^T += Q^T dS.  With a bias, per-key sums of dS feed the bias gradient.
template <int D, bool CAUSAL, bool HAS_BIAS, bool HAS_SEG>
__global__ __launch_bounds__(kThreads) void dkdv_f32_kernel(Params p) {
  constexpr int NC = D / 16;
  __shared__ float sR[kWaves][kRows][D];
  __shared__ float sB[kWaves][kRows];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, col = lane & 15;
  const int HB = p.B * p.H;
  const int64_t n_kt_blk = (p.Lb + kRows - 1) / kRows;
  const int64_t wg = blockIdx.x;
  const int hb = static_cast<int>(wg % HB);
  const int64_t kt = wg / HB;
  const int b = hb / p.H, h = hb % p.H;
  const int j = static_cast<int>(kt / n_kt_blk);
  const int64_t ka = (kt % n_kt_blk) * kRows;
  const int kfirst = static_cast<int>(static_cast<int64_t>(j) * p.Lb + ka);
  const int nkeys = static_cast<int>((p.Lb - ka) < kRows ? (p.Lb - ka) : kRows);
  const bool kok = col < nkeys;
  const int key = kfirst + col;
  const float* qp = static_cast<const float*>(p.q);
  const float* kp = static_cast<const float*>(p.k);
  const float* vp = static_cast<const float*>(p.v);
  const float* gp = static_cast<const float*>(p.dout);

  f32x4 kf[NC], vf[NC];
  const int64_t koff = row_offset(b, kok ? key : kfirst, h, p.Lk, p.H, D);
  load_frag<D>(kf, kp + koff, kok, g);
  load_frag<D>(vf, vp + koff, kok, g);
  const int32_t* srow = HAS_SEG ? p.seg + static_cast<int64_t>(b) * p.Lk : nullptr;
  const int kseg = (HAS_SEG && kok) ? srow[key] : 0;
  const float bias_l2 = (HAS_BIAS && kok) ? p.bias[static_cast<int64_t>(h) * p.bias_len + key % p.bias_len] * kLog2e : 0.f;
  const int kfq = CAUSAL ? causal_first_query(key, 0, p.causal) : 0;   // first query able to see the key
  const float c = p.scale * kLog2e;
  const float* lrow = p.lse + (static_cast<int64_t>(b) * p.H + h) * p.Lq;
  const float* drow = p.delta + (static_cast<int64_t>(b) * p.H + h) * p.Lq;

  f32x4 dk[NC], dv[NC];
#pragma unroll
  for (int dt = 0; dt < NC; ++dt) dk[dt] = dv[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float dsum = 0.f;

  QueryWalk walk;
  walk.begin(p.n_ring, j, p.Lb, CAUSAL, CAUSAL ? causal_first_query(kfirst, 0, p.causal) : kfirst, p.ring_rank);
  for (int n = 0; walk.next<kRows>(); ++n) {
    if ((n & (kWaves - 1)) != wave) continue;
    const int row0 = walk.row0, rend = walk.rend, pbase = walk.pos_base;
    f32x4 s = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
    {
      const int row = row0 + col;
      const int64_t off = row_offset(b, row < rend ? row : row0, h, p.Lq, p.H, D);
      f32x4 qf[NC], gf[NC];
      load_frag<D>(qf, qp + off, row < rend, g);
      load_frag<D>(gf, gp + off, row < rend, g);
#pragma unroll
      for (int cc = 0; cc < NC; ++cc)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s = mma(qf[cc][e], kf[cc][e], s);
          dp = mma(gf[cc][e], vf[cc][e], dp);
        }
    }
    float pr[4], ds[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = row0 + 4 * g + v;
      const bool rok = row < rend;
      const int rr = rok ? row : row0;
      const int qpos = rr + pbase;
      bool vis = rok && kok;
      if (CAUSAL) vis = vis && qpos >= kfq;
      if (HAS_SEG) vis = vis && srow[qpos] == kseg;
      const float y = s[v] * c + bias_l2 - lrow[rr] * kLog2e;
      pr[v] = vis ? __builtin_amdgcn_exp2f(y) : 0.f;
      ds[v] = pr[v] * (dp[v] - drow[rr]);
      if (HAS_BIAS) dsum += ds[v];
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = row0 + 4 * g + v;
      const bool rok = row < rend;
      const int64_t off = row_offset(b, rok ? row : row0, h, p.Lq, p.H, D);
#pragma unroll
      for (int dt = 0; dt < NC; ++dt) {
        dv[dt] = mma(rok ? gp[off + 16 * dt + col] : 0.f, pr[v], dv[dt]);
        dk[dt] = mma(rok ? qp[off + 16 * dt + col] : 0.f, ds[v], dk[dt]);
      }
    }
  }

  // the four waves' sums, in a fixed order: dK first, then dV through the same LDS
  if (HAS_BIAS) dsum = group_sum(dsum);
  const int kq = threadIdx.x >> 4, dl = threadIdx.x & 15;   // 16 threads per key
  const int64_t out_off = row_offset(b, kfirst + kq, h, p.Lk, p.H, D);
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    if (pass) __syncthreads();
#pragma unroll
    for (int dt = 0; dt < NC; ++dt)
#pragma unroll
      for (int v = 0; v < 4; ++v) sR[wave][col][16 * dt + 4 * g + v] = pass ? dv[dt][v] : dk[dt][v];
    if (HAS_BIAS && pass == 0 && g == 0) sB[wave][col] = dsum;
    __syncthreads();
    if (kq < nkeys) {
      float* dst = static_cast<float*>(pass ? p.dv : p.dk) + out_off;
      const float f = pass ? 1.f : p.scale;
      for (int d = dl; d < D; d += 16) {
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) acc += sR[w][kq][d];
        dst[d] = acc * f;
      }
      if (HAS_BIAS && pass == 0 && dl == 0 && p.dbias_keys) {
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) acc += sB[w][kq];
        p.dbias_keys[(static_cast<int64_t>(b) * p.H + h) * p.Lk + kfirst + kq] = acc;
      }
    }
  }
}

// ------------------------------------------------------------------ backward dQ
// 16 queries held; S^T = K Q^T and dP^T = V dO^T (lane l: query l & 15, keys 4 g + v), then
// dQ^T += K^T dS^T.
template <int D, bool CAUSAL, bool HAS_BIAS, bool HAS_SEG>
__global__ __launch_bounds__(kThreads) void dq_f32_kernel(Params p) {
  constexpr int NC = D / 16;
  __shared__ float sR[kWaves][kRows][D];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, col = lane & 15;
  const QueryTile t(p);
  const float* qp = static_cast<const float*>(p.q);
  const float* kp = static_cast<const float*>(p.k);
  const float* vp = static_cast<const float*>(p.v);
  const float* gp = static_cast<const float*>(p.dout);
  const bool qok = col < t.nrows;
  const int qpos = t.pos0 + col;
  f32x4 qf[NC], gf[NC];
  const int64_t qoff = row_offset(t.b, t.qrow + (qok ? col : 0), t.h, p.Lq, p.H, D);
  load_frag<D>(qf, qp + qoff, qok, g);
  load_frag<D>(gf, gp + qoff, qok, g);
  const int64_t li = (static_cast<int64_t>(t.b) * p.H + t.h) * p.Lq + t.qrow + (qok ? col : 0);
  const float lse_l2 = p.lse[li] * kLog2e;
  const float delta = p.delta[li];
  const int32_t* srow = HAS_SEG ? p.seg + static_cast<int64_t>(t.b) * p.Lk : nullptr;
  const int qseg = (HAS_SEG && qok) ? srow[qpos] : 0;
  const int qlim = CAUSAL ? causal_last_key(qpos, 0, p.causal) : 0;
  const float c = p.scale * kLog2e;
  const float* brow = HAS_BIAS ? p.bias + static_cast<int64_t>(t.h) * p.bias_len : nullptr;

  f32x4 dq[NC];
#pragma unroll
  for (int dt = 0; dt < NC; ++dt) dq[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  RingWalk walk;
  const int plast = t.pos0 + t.nrows - 1;
  walk.begin(p.n_ring, t.rank, p.Lb, CAUSAL, CAUSAL ? causal_last_key(plast, 0, p.causal) : plast);
  for (int n = 0; walk.next<kRows>(); ++n) {
    if ((n & (kWaves - 1)) != wave) continue;
    const int key0 = walk.key0, kend = walk.kend;
    f32x4 s = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
    {
      const int key = key0 + col;
      const int64_t off = row_offset(t.b, key < kend ? key : key0, t.h, p.Lk, p.H, D);
      f32x4 kf[NC], vf[NC];
      load_frag<D>(kf, kp + off, key < kend, g);
      load_frag<D>(vf, vp + off, key < kend, g);
#pragma unroll
      for (int cc = 0; cc < NC; ++cc)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s = mma(kf[cc][e], qf[cc][e], s);
          dp = mma(vf[cc][e], gf[cc][e], dp);
        }
    }
    float ds[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int key = key0 + 4 * g + v;
      const int kk = key < kend ? key : key0;
      bool vis = qok && key < kend;
      if (CAUSAL) vis = vis && key <= qlim;
      if (HAS_SEG) vis = vis && srow[kk] == qseg;
      float y = s[v] * c;
      if (HAS_BIAS) y += brow[kk % p.bias_len] * kLog2e;
      const float pr = vis ? __builtin_amdgcn_exp2f(y - lse_l2) : 0.f;
      ds[v] = pr * (dp[v] - delta);
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int key = key0 + 4 * g + v;
      const float* krow = kp + row_offset(t.b, key < kend ? key : key0, t.h, p.Lk, p.H, D);
#pragma unroll
      for (int dt = 0; dt < NC; ++dt) dq[dt] = mma(key < kend ? krow[16 * dt + col] : 0.f, ds[v], dq[dt]);
    }
  }

#pragma unroll
  for (int dt = 0; dt < NC; ++dt)
#pragma unroll
    for (int v = 0; v < 4; ++v) sR[wave][col][16 * dt + 4 * g + v] = dq[dt][v];
  __syncthreads();
  const int q = threadIdx.x >> 4, dl = threadIdx.x & 15;
  if (q >= t.nrows) return;
  float* dst = static_cast<float*>(p.dq) + row_offset(t.b, t.qrow + q, t.h, p.Lq, p.H, D);
  for (int d = dl; d < D; d += 16) {
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) acc += sR[w][q][d];
    dst[d] = acc * p.scale;
  }
}

// ------------------------------------------------------------------ launchers
#define RA_F32_FLAGS(CALL)                                                         \
  do {                                                                             \
    const bool c_ = p.causal != 0, b_ = p.bias != nullptr, s_ = p.seg != nullptr;  \
    if (c_) {                                                                      \
      if (b_) { if (s_) CALL(true, true, true); else CALL(true, true, false); }    \
      else { if (s_) CALL(true, false, true); else CALL(true, false, false); }     \
    } else {                                                                       \
      if (b_) { if (s_) CALL(false, true, true); else CALL(false, true, false); }  \
      else { if (s_) CALL(false, false, true); else CALL(false, false, false); }   \
    }                                                                              \
  } while (0)

int64_t query_tiles(const Params& p) {
  return (p.ring_rank < 0 ? p.n_ring : 1) * ((p.Lb + kRows - 1) / kRows) * p.B * p.H;
}

template <int D>
hipError_t fwd_d(const Params& p, hipStream_t st) {
  const int64_t grid = query_tiles(p);
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
#define RA_L(C, B, S) hipLaunchKernelGGL((fwd_f32_kernel<D, C, B, S>), dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, st, p)
  RA_F32_FLAGS(RA_L);
#undef RA_L
  return hipGetLastError();
}
template <int D>
hipError_t dkdv_d(const Params& p, hipStream_t st) {
  const int64_t grid = static_cast<int64_t>(p.n_ring) * ((p.Lb + kRows - 1) / kRows) * p.B * p.H;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
#define RA_L(C, B, S) hipLaunchKernelGGL((dkdv_f32_kernel<D, C, B, S>), dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, st, p)
  RA_F32_FLAGS(RA_L);
#undef RA_L
  return hipGetLastError();
}
template <int D>
hipError_t dq_d(const Params& p, hipStream_t st) {
  const int64_t grid = query_tiles(p);
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
#define RA_L(C, B, S) hipLaunchKernelGGL((dq_f32_kernel<D, C, B, S>), dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, st, p)
  RA_F32_FLAGS(RA_L);
#undef RA_L
  return hipGetLastError();
}
#undef RA_F32_FLAGS

}  // namespace

hipError_t launch_fwd_f32(const Params& p, hipStream_t st) {
  if (p.D == 64) return fwd_d<64>(p, st);
  if (p.D == 128) return fwd_d<128>(p, st);
  return hipErrorInvalidValue;
}
hipError_t launch_bwd_dkdv_f32(const Params& p, hipStream_t st) {
  if (p.D == 64) return dkdv_d<64>(p, st);
  if (p.D == 128) return dkdv_d<128>(p, st);
  return hipErrorInvalidValue;
}
hipError_t launch_bwd_dq_f32(const Params& p, hipStream_t st) {
  if (p.D == 64) return dq_d<64>(p, st);
  if (p.D == 128) return dq_d<128>(p, st);
  return hipErrorInvalidValue;
}

}  // namespace ra
