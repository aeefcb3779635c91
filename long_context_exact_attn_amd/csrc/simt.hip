// Scalar (one lane per query or per key) kernels of libra_attn:
//  * the float32 forward -- the exact-arithmetic path: float32 products and
//    float32 probabilities, no bfloat16 rounding anywhere;
//  * the backward preprocess Delta = rowsum(dO * O) for both dtypes;
//  * float32 backward dK/dV and dQ kernels.
// They follow the same ring walks as the MFMA kernels.
#include "ra_common.cuh"

namespace ra {
namespace {

constexpr int kLanes = 64;   // one wavefront per workgroup
constexpr int BKS = 16;      // keys per LDS tile (forward / dQ)
constexpr int BQS = 16;      // queries per LDS tile (dK/dV)

template <typename T>
__device__ __forceinline__ void load_row(float* dst, const T* src, int D) {
  for (int d = 0; d < D; ++d) dst[d] = to_f32(src[d]);
}

// ------------------------------------------------------------------ forward (float32)
template <int D, bool CAUSAL, bool HAS_BIAS, bool HAS_SEG>
__global__ __launch_bounds__(kLanes) void fwd_simt_kernel(Params p) {
  __shared__ float sK[BKS][D];
  __shared__ float sV[BKS][D];
  __shared__ float sB[BKS];
  __shared__ int sS[BKS];
  const int tid = threadIdx.x;
  const int HB = p.B * p.H;
  const int64_t n_qt_blk = (p.Lb + kLanes - 1) / kLanes;
  const int64_t n_qt = (p.ring_rank < 0 ? p.n_ring : 1) * n_qt_blk;
  const int64_t wg = blockIdx.x;
  const int hb = static_cast<int>(wg % HB);
  const int64_t t = n_qt - 1 - wg / HB;
  const int b = hb / p.H, h = hb % p.H;
  const int r_local = static_cast<int>(t / n_qt_blk);
  const int64_t qa = (t % n_qt_blk) * kLanes;
  const int r = p.ring_rank < 0 ? r_local : p.ring_rank;
  const int64_t qrow_base = static_cast<int64_t>(r_local) * p.Lb;
  const int64_t pos0 = static_cast<int64_t>(r) * p.Lb + qa;
  const int64_t nrows = (p.Lb - qa) < kLanes ? (p.Lb - qa) : kLanes;
  const bool valid = tid < nrows;
  const int64_t qpos = pos0 + tid;
  const float* qp = static_cast<const float*>(p.q);
  const float* kp = static_cast<const float*>(p.k);
  const float* vp = static_cast<const float*>(p.v);

  float qr[D], o[D];
  const int64_t qoff = row_offset(b, qrow_base + (valid ? qa + tid : 0), h, p.Lq, p.H, D);
  for (int d = 0; d < D; ++d) { qr[d] = valid ? qp[qoff + d] : 0.f; o[d] = 0.f; }
  const int qseg = (HAS_SEG && valid) ? p.seg[static_cast<int64_t>(b) * p.Lk + qpos] : 0;
  const float c = p.scale * kLog2e;
  float m = -INFINITY, l = 0.f;

  RingWalk walk;
  walk.begin(p.n_ring, r, p.Lb, CAUSAL,
             CAUSAL && nrows > 0 ? causal_last_key(static_cast<int>(pos0 + nrows - 1), 0, p.causal) : pos0 + nrows - 1);
  const int64_t qlim = CAUSAL ? causal_last_key(static_cast<int>(qpos), 0, p.causal) : qpos;   // last visible key
  while (nrows > 0 && walk.next<BKS>()) {
    const int64_t key0 = walk.key0, kend = walk.kend;
    __syncthreads();
    for (int e = tid; e < BKS * D; e += kLanes) {
      const int j = e / D, d = e % D;
      const int64_t key = key0 + j;
      const bool ok = key < kend;
      const int64_t off = row_offset(b, ok ? key : 0, h, p.Lk, p.H, D) + d;
      sK[j][d] = ok ? kp[off] : 0.f;
      sV[j][d] = ok ? vp[off] : 0.f;
    }
    if (tid < BKS) {
      const int64_t key = key0 + tid;
      if (HAS_BIAS) sB[tid] = key < kend ? p.bias[h * p.bias_len + key % p.bias_len] * kLog2e : 0.f;
      if (HAS_SEG) sS[tid] = key < kend ? p.seg[static_cast<int64_t>(b) * p.Lk + key] : 0;
    }
    __syncthreads();
    if (!valid) continue;
    float s[BKS];
    float mx = -INFINITY;
    for (int j = 0; j < BKS; ++j) {
      const int64_t key = key0 + j;
      bool vis = key < kend;
      if (CAUSAL) vis = vis && key <= qlim;
      if (HAS_SEG) vis = vis && sS[j] == qseg;
      float acc = 0.f;
      for (int d = 0; d < D; ++d) acc = __builtin_fmaf(qr[d], sK[j][d], acc);
      float x = acc * c;
      if (HAS_BIAS) x += sB[j];
      s[j] = vis ? x : -INFINITY;
      mx = fmaxf(mx, s[j]);
    }
    const float mnew = fmaxf(m, mx);
    const float alpha = mnew == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m - mnew);
    const float msub = mnew == -INFINITY ? 0.f : mnew;
    l *= alpha;
    for (int d = 0; d < D; ++d) o[d] *= alpha;
    for (int j = 0; j < BKS; ++j) {
      const float pj = __builtin_amdgcn_exp2f(s[j] - msub);
      l += pj;
      for (int d = 0; d < D; ++d) o[d] = __builtin_fmaf(pj, sV[j][d], o[d]);
    }
    m = mnew;
  }
  if (!valid) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  float* op = static_cast<float*>(p.out) + qoff;
  for (int d = 0; d < D; ++d) op[d] = o[d] * inv;
  p.lse[(static_cast<int64_t>(b) * p.H + h) * p.Lq + qrow_base + qa + tid] =
      l > 0.f ? (m + __builtin_amdgcn_logf(l)) * kLn2 : -INFINITY;
}

// ------------------------------------------------------------------ backward preprocess
// delta[b, h, i] = sum_d dout[b, i, h, d] * out[b, i, h, d]; one lane per row.
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(Params p) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;   // (b, i, h) in memory order
  const int64_t rows = static_cast<int64_t>(p.B) * p.Lq * p.H;
  if (idx >= rows) return;
  const int h = static_cast<int>(idx % p.H);
  const int64_t i = (idx / p.H) % p.Lq;
  const int b = static_cast<int>(idx / (static_cast<int64_t>(p.H) * p.Lq));
  const T* o = static_cast<const T*>(p.out) + idx * D;
  const T* g = static_cast<const T*>(p.dout) + idx * D;
  float acc = 0.f;
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int d = 0; d < D; d += 8) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(o + d);
      const bf16x8 c = *reinterpret_cast<const bf16x8*>(g + d);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)a[e], (float)c[e], acc);
    }
  } else {
#pragma unroll
    for (int d = 0; d < D; d += 4) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(o + d);
      const f32x4 c = *reinterpret_cast<const f32x4*>(g + d);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = __builtin_fmaf(a[e], c[e], acc);
    }
  }
  p.delta_out[(static_cast<int64_t>(b) * p.H + h) * p.Lq + i] = acc;
}

// ------------------------------------------------------------------ ring-step finalize and merge
// One lane per (b, i, h) row.  finalize: out = O / l, lse = (m + log2 l) ln 2 from the running state
// of ra_blockwise_attn_fwd_step (m in log2 units).  merge: the attention over the union of two
// disjoint key sets from the attention over each,
//   lse = log(exp(lse_a) + exp(lse_b)),  out = exp(lse_a - lse) out_a + exp(lse_b - lse) out_b.
template <typename T, int D>
__global__ __launch_bounds__(256) void finalize_kernel(Params p) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;   // (b, i, h) in memory order
  const int64_t rows = static_cast<int64_t>(p.B) * p.Lq * p.H;
  if (idx >= rows) return;
  const int h = static_cast<int>(idx % p.H);
  const int64_t i = (idx / p.H) % p.Lq;
  const int b = static_cast<int>(idx / (static_cast<int64_t>(p.H) * p.Lq));
  const int64_t si = (static_cast<int64_t>(b) * p.H + h) * p.Lq + i;
  const float l = p.l_state[si];
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const float* o = p.o_state + idx * D;
  T* dst = static_cast<T*>(p.out) + idx * D;
#pragma unroll
  for (int d = 0; d < D; d += 4) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(o + d);
#pragma unroll
    for (int e = 0; e < 4; ++e) dst[d + e] = from_f32<T>(x[e] * inv);
  }
  p.lse[si] = l > 0.f ? (p.m_state[si] + __builtin_amdgcn_logf(l)) * kLn2 : -INFINITY;
}

template <typename T, int D>
__global__ __launch_bounds__(256) void merge_kernel(Params p, const T* out_b, const float* lse_b) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t rows = static_cast<int64_t>(p.B) * p.Lq * p.H;
  if (idx >= rows) return;
  const int h = static_cast<int>(idx % p.H);
  const int64_t i = (idx / p.H) % p.Lq;
  const int b = static_cast<int>(idx / (static_cast<int64_t>(p.H) * p.Lq));
  const int64_t si = (static_cast<int64_t>(b) * p.H + h) * p.Lq + i;
  const float la = p.lse[si], lb = lse_b[si];     // p.lse / p.out: the first pair, also the result
  const float mx = fmaxf(la, lb);
  float wa = 0.f, wb = 0.f, lse = -INFINITY;
  if (mx != -INFINITY) {
    wa = __builtin_amdgcn_exp2f((la - mx) * kLog2e);
    wb = __builtin_amdgcn_exp2f((lb - mx) * kLog2e);
    const float sum = wa + wb;
    lse = mx + __builtin_amdgcn_logf(sum) * kLn2;
    wa /= sum;
    wb /= sum;
  }
  T* oa = static_cast<T*>(p.out) + idx * D;
  const T* ob = out_b + idx * D;
  for (int d = 0; d < D; ++d) oa[d] = from_f32<T>(wa * to_f32(oa[d]) + wb * to_f32(ob[d]));
  p.lse[si] = lse;
}

// ------------------------------------------------------------------ backward dK/dV (one lane per key)
template <typename T, int D, bool CAUSAL, bool HAS_BIAS, bool HAS_SEG>
__global__ __launch_bounds__(kLanes) void dkdv_simt_kernel(Params p) {
  __shared__ float sQ[BQS][D];
  __shared__ float sG[BQS][D];
  __shared__ float sL[BQS];
  __shared__ float sD[BQS];
  __shared__ int sS[BQS];
  __shared__ int64_t sP[BQS];
  const int tid = threadIdx.x;
  const int HB = p.B * p.H;
  const int64_t n_kt_blk = (p.Lb + kLanes - 1) / kLanes;
  const int64_t wg = blockIdx.x;
  const int hb = static_cast<int>(wg % HB);
  const int64_t kt = wg / HB;
  const int b = hb / p.H, h = hb % p.H;
  const int j = static_cast<int>(kt / n_kt_blk);
  const int64_t ka = (kt % n_kt_blk) * kLanes;
  const int64_t kfirst = static_cast<int64_t>(j) * p.Lb + ka;
  const bool valid = ka + tid < p.Lb;
  const int64_t key = kfirst + tid;
  const T* qp = static_cast<const T*>(p.q);
  const T* kp = static_cast<const T*>(p.k);
  const T* vp = static_cast<const T*>(p.v);
  const T* gp = static_cast<const T*>(p.dout);

  float kr[D], vr[D], dk[D], dv[D];
  const int64_t koff = row_offset(b, valid ? key : 0, h, p.Lk, p.H, D);
  for (int d = 0; d < D; ++d) {
    kr[d] = valid ? to_f32(kp[koff + d]) : 0.f;
    vr[d] = valid ? to_f32(vp[koff + d]) : 0.f;
    dk[d] = 0.f;
    dv[d] = 0.f;
  }
  const int kseg = (HAS_SEG && valid) ? p.seg[static_cast<int64_t>(b) * p.Lk + key] : 0;
  const float bias_l2 = (HAS_BIAS && valid) ? p.bias[h * p.bias_len + key % p.bias_len] * kLog2e : 0.f;
  const float c = p.scale * kLog2e;
  float dsum = 0.f;   // with a bias: sum_i dS_ij of this key, from which the bias gradient is formed

  QueryWalk walk;
  // the first query able to see this thread's key, and the first able to see the tile's first key
  const int64_t kfq = CAUSAL ? causal_first_query(static_cast<int>(key), 0, p.causal) : key;
  walk.begin(p.n_ring, j, p.Lb, CAUSAL, CAUSAL ? causal_first_query(static_cast<int>(kfirst), 0, p.causal) : kfirst,
             p.ring_rank);
  while (walk.next<BQS>()) {
    const int64_t row0 = walk.row0, rend = walk.rend, pbase = walk.pos_base;
    __syncthreads();
    for (int e = tid; e < BQS * D; e += kLanes) {
      const int i = e / D, d = e % D;
      const int64_t row = row0 + i;
      const bool ok = row < rend;
      const int64_t off = row_offset(b, ok ? row : 0, h, p.Lq, p.H, D) + d;
      sQ[i][d] = ok ? to_f32(qp[off]) : 0.f;
      sG[i][d] = ok ? to_f32(gp[off]) : 0.f;
    }
    if (tid < BQS) {
      const int64_t row = row0 + tid;
      const bool ok = row < rend;
      const int64_t li = (static_cast<int64_t>(b) * p.H + h) * p.Lq + (ok ? row : 0);
      sL[tid] = ok ? p.lse[li] * kLog2e : INFINITY;
      sD[tid] = ok ? p.delta[li] : 0.f;
      sP[tid] = ok ? row + pbase : -1;
      if (HAS_SEG) sS[tid] = ok ? p.seg[static_cast<int64_t>(b) * p.Lk + row + pbase] : 0;
    }
    __syncthreads();
    if (!valid) continue;
    for (int i = 0; i < BQS; ++i) {
      const int64_t qpos = sP[i];
      bool vis = qpos >= 0;
      if (CAUSAL) vis = vis && qpos >= kfq;
      if (HAS_SEG) vis = vis && sS[i] == kseg;
      if (!vis) continue;
      float s = 0.f, dp = 0.f;
      for (int d = 0; d < D; ++d) {
        s = __builtin_fmaf(sQ[i][d], kr[d], s);
        dp = __builtin_fmaf(sG[i][d], vr[d], dp);
      }
      const float pr = __builtin_amdgcn_exp2f(s * c + bias_l2 - sL[i]);
      const float ds0 = pr * (dp - sD[i]);
      if (HAS_BIAS) dsum += ds0;
      const float ds = ds0 * p.scale;
      for (int d = 0; d < D; ++d) {
        dv[d] = __builtin_fmaf(pr, sG[i][d], dv[d]);
        dk[d] = __builtin_fmaf(ds, sQ[i][d], dk[d]);
      }
    }
  }
  if (!valid) return;
  if (HAS_BIAS && p.dbias_keys) p.dbias_keys[(static_cast<int64_t>(b) * p.H + h) * p.Lk + key] = dsum;
  T* dkp = static_cast<T*>(p.dk) + koff;
  T* dvp = static_cast<T*>(p.dv) + koff;
  for (int d = 0; d < D; ++d) {
    dkp[d] = from_f32<T>(dk[d]);
    dvp[d] = from_f32<T>(dv[d]);
  }
}

// ------------------------------------------------------------------ backward dQ (one lane per query)
template <typename T, int D, bool CAUSAL, bool HAS_BIAS, bool HAS_SEG>
__global__ __launch_bounds__(kLanes) void dq_simt_kernel(Params p) {
  __shared__ float sK[BKS][D];
  __shared__ float sV[BKS][D];
  __shared__ float sB[BKS];
  __shared__ int sS[BKS];
  const int tid = threadIdx.x;
  const int HB = p.B * p.H;
  const int64_t n_qt_blk = (p.Lb + kLanes - 1) / kLanes;
  const int64_t n_qt = (p.ring_rank < 0 ? p.n_ring : 1) * n_qt_blk;
  const int64_t wg = blockIdx.x;
  const int hb = static_cast<int>(wg % HB);
  const int64_t t = n_qt - 1 - wg / HB;
  const int b = hb / p.H, h = hb % p.H;
  const int r_local = static_cast<int>(t / n_qt_blk);
  const int64_t qa = (t % n_qt_blk) * kLanes;
  const int r = p.ring_rank < 0 ? r_local : p.ring_rank;
  const int64_t qrow_base = static_cast<int64_t>(r_local) * p.Lb;
  const int64_t pos0 = static_cast<int64_t>(r) * p.Lb + qa;
  const int64_t nrows = (p.Lb - qa) < kLanes ? (p.Lb - qa) : kLanes;
  const bool valid = tid < nrows;
  const int64_t qpos = pos0 + tid;
  const T* qp = static_cast<const T*>(p.q);
  const T* kp = static_cast<const T*>(p.k);
  const T* vp = static_cast<const T*>(p.v);
  const T* gp = static_cast<const T*>(p.dout);

  float qr[D], g[D], dq[D];
  const int64_t qoff = row_offset(b, qrow_base + (valid ? qa + tid : 0), h, p.Lq, p.H, D);
  for (int d = 0; d < D; ++d) {
    qr[d] = valid ? to_f32(qp[qoff + d]) : 0.f;
    g[d] = valid ? to_f32(gp[qoff + d]) : 0.f;
    dq[d] = 0.f;
  }
  const int64_t li = (static_cast<int64_t>(b) * p.H + h) * p.Lq + qrow_base + (valid ? qa + tid : 0);
  const float lse_l2 = p.lse[li] * kLog2e;
  const float delta = p.delta[li];
  const int qseg = (HAS_SEG && valid) ? p.seg[static_cast<int64_t>(b) * p.Lk + qpos] : 0;
  const float c = p.scale * kLog2e;

  RingWalk walk;
  walk.begin(p.n_ring, r, p.Lb, CAUSAL,
             CAUSAL && nrows > 0 ? causal_last_key(static_cast<int>(pos0 + nrows - 1), 0, p.causal) : pos0 + nrows - 1);
  const int64_t qlim = CAUSAL ? causal_last_key(static_cast<int>(qpos), 0, p.causal) : qpos;   // last visible key
  while (nrows > 0 && walk.next<BKS>()) {
    const int64_t key0 = walk.key0, kend = walk.kend;
    __syncthreads();
    for (int e = tid; e < BKS * D; e += kLanes) {
      const int j = e / D, d = e % D;
      const int64_t key = key0 + j;
      const bool ok = key < kend;
      const int64_t off = row_offset(b, ok ? key : 0, h, p.Lk, p.H, D) + d;
      sK[j][d] = ok ? to_f32(kp[off]) : 0.f;
      sV[j][d] = ok ? to_f32(vp[off]) : 0.f;
    }
    if (tid < BKS) {
      const int64_t key = key0 + tid;
      if (HAS_BIAS) sB[tid] = key < kend ? p.bias[h * p.bias_len + key % p.bias_len] * kLog2e : 0.f;
      if (HAS_SEG) sS[tid] = key < kend ? p.seg[static_cast<int64_t>(b) * p.Lk + key] : 0;
    }
    __syncthreads();
    if (!valid) continue;
    for (int j = 0; j < BKS; ++j) {
      const int64_t key = key0 + j;
      bool vis = key < kend;
      if (CAUSAL) vis = vis && key <= qlim;
      if (HAS_SEG) vis = vis && sS[j] == qseg;
      if (!vis) continue;
      float s = 0.f, dp = 0.f;
      for (int d = 0; d < D; ++d) {
        s = __builtin_fmaf(qr[d], sK[j][d], s);
        dp = __builtin_fmaf(g[d], sV[j][d], dp);
      }
      float x = s * c;
      if (HAS_BIAS) x += sB[j];
      const float pr = __builtin_amdgcn_exp2f(x - lse_l2);
      const float ds = pr * (dp - delta) * p.scale;
      for (int d = 0; d < D; ++d) dq[d] = __builtin_fmaf(ds, sK[j][d], dq[d]);
    }
  }
  if (!valid) return;
  T* dqp = static_cast<T*>(p.dq) + qoff;
  for (int d = 0; d < D; ++d) dqp[d] = from_f32<T>(dq[d]);
}

// ------------------------------------------------------------------ launchers
int64_t q_tiles(const Params& p, int bq) { return (p.ring_rank < 0 ? p.n_ring : 1) * ((p.Lb + bq - 1) / bq); }

#define RA_SELECT_FLAGS(CALL)                                                      \
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

template <int D>
hipError_t fwd_simt_d(const Params& p, hipStream_t st) {
  const int64_t grid = q_tiles(p, kLanes) * p.B * p.H;
  if (grid == 0) return hipSuccess;
#define RA_L(C, B, S) hipLaunchKernelGGL((fwd_simt_kernel<D, C, B, S>), dim3(grid), dim3(kLanes), 0, st, p)
  RA_SELECT_FLAGS(RA_L);
#undef RA_L
  return hipGetLastError();
}

template <typename T, int D>
hipError_t dkdv_simt_d(const Params& p, hipStream_t st) {
  const int64_t grid = static_cast<int64_t>(p.n_ring) * ((p.Lb + kLanes - 1) / kLanes) * p.B * p.H;
  if (grid == 0) return hipSuccess;
#define RA_L(C, B, S) hipLaunchKernelGGL((dkdv_simt_kernel<T, D, C, B, S>), dim3(grid), dim3(kLanes), 0, st, p)
  RA_SELECT_FLAGS(RA_L);
#undef RA_L
  return hipGetLastError();
}

template <typename T, int D>
hipError_t dq_simt_d(const Params& p, hipStream_t st) {
  const int64_t grid = q_tiles(p, kLanes) * p.B * p.H;
  if (grid == 0) return hipSuccess;
#define RA_L(C, B, S) hipLaunchKernelGGL((dq_simt_kernel<T, D, C, B, S>), dim3(grid), dim3(kLanes), 0, st, p)
  RA_SELECT_FLAGS(RA_L);
#undef RA_L
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_simt(const Params& p, hipStream_t st) {
  if (p.D == 64) return fwd_simt_d<64>(p, st);
  if (p.D == 128) return fwd_simt_d<128>(p, st);
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_bwd_preprocess_t(const Params& p, hipStream_t st) {
  const int64_t rows = static_cast<int64_t>(p.B) * p.Lq * p.H;
  if (rows == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((rows + 255) / 256));
  if (p.D == 64) hipLaunchKernelGGL((bwd_pre_kernel<T, 64>), grid, dim3(256), 0, st, p);
  else if (p.D == 128) hipLaunchKernelGGL((bwd_pre_kernel<T, 128>), grid, dim3(256), 0, st, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}


template <typename T>
hipError_t launch_bwd_dkdv_simt_t(const Params& p, hipStream_t st) {
  if (p.D == 64) return dkdv_simt_d<T, 64>(p, st);
  if (p.D == 128) return dkdv_simt_d<T, 128>(p, st);
  return hipErrorInvalidValue;
}
template <typename T>
hipError_t launch_bwd_dq_simt_t(const Params& p, hipStream_t st) {
  if (p.D == 64) return dq_simt_d<T, 64>(p, st);
  if (p.D == 128) return dq_simt_d<T, 128>(p, st);
  return hipErrorInvalidValue;
}
template <typename T>
hipError_t launch_finalize_t(const Params& p, hipStream_t st) {
  const int64_t rows = static_cast<int64_t>(p.B) * p.Lq * p.H;
  if (rows == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((rows + 255) / 256));
  if (p.D == 64) hipLaunchKernelGGL((finalize_kernel<T, 64>), grid, dim3(256), 0, st, p);
  else if (p.D == 128) hipLaunchKernelGGL((finalize_kernel<T, 128>), grid, dim3(256), 0, st, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}
template <typename T>
hipError_t launch_merge_t(const Params& p, const void* out_b, const float* lse_b, hipStream_t st) {
  const int64_t rows = static_cast<int64_t>(p.B) * p.Lq * p.H;
  if (rows == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((rows + 255) / 256));
  const T* ob = static_cast<const T*>(out_b);
  if (p.D == 64) hipLaunchKernelGGL((merge_kernel<T, 64>), grid, dim3(256), 0, st, p, ob, lse_b);
  else if (p.D == 128) hipLaunchKernelGGL((merge_kernel<T, 128>), grid, dim3(256), 0, st, p, ob, lse_b);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}
// factor * acc converted to the output type, four elements per lane (the row length is a
// multiple of 4, so the element count is too)
template <typename T>
__global__ __launch_bounds__(256) void grad_finalize_kernel(const float* __restrict__ acc, float factor,
                                                            T* __restrict__ out, int64_t n4) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n4) return;
  const f32x4 x = reinterpret_cast<const f32x4*>(acc)[i];
#pragma unroll
  for (int e = 0; e < 4; ++e) out[4 * i + e] = from_f32<T>(x[e] * factor);
}

hipError_t launch_grad_finalize(const float* acc, float factor, void* out, int64_t elems, bool bf16, hipStream_t st) {
  const int64_t n4 = elems / 4;
  if (n4 == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((n4 + 255) / 256));
  if (bf16) hipLaunchKernelGGL(grad_finalize_kernel<__bf16>, grid, dim3(256), 0, st, acc, factor, static_cast<__bf16*>(out), n4);
  else hipLaunchKernelGGL(grad_finalize_kernel<float>, grid, dim3(256), 0, st, acc, factor, static_cast<float*>(out), n4);
  return hipGetLastError();
}

// dbias[h, t] = sum over batch rows b and keys j = t, t + bias_len, ... of key_sums[b, h, j]; one
// lane per (h, t), summing in a fixed order (deterministic)
__global__ __launch_bounds__(256) void bias_grad_kernel(const float* __restrict__ key_sums, float* __restrict__ dbias,
                                                        int B, int H, int64_t Lk, int64_t nb) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<int64_t>(H) * nb) return;
  const int h = static_cast<int>(i / nb);
  const int64_t t = i % nb;
  float acc = 0.f;
  for (int b = 0; b < B; ++b) {
    const float* row = key_sums + (static_cast<int64_t>(b) * H + h) * Lk;
    for (int64_t j = t; j < Lk; j += nb) acc += row[j];
  }
  dbias[i] = acc;
}

// One K/V block's share of dbias: the block's keys sit at global positions kv_pos0 + j, so key j feeds
// bias entry t = (kv_pos0 + j) mod bias_len; one lane per (h, t), a fixed summation order.  accumulate:
// add to dbias (the blocks of a ring, one call each), else overwrite it.
__global__ __launch_bounds__(256) void bias_grad_block_kernel(const float* __restrict__ key_sums,
                                                              float* __restrict__ dbias, int B, int H, int64_t Lb,
                                                              int64_t kv_pos0, int64_t nb, int accumulate) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<int64_t>(H) * nb) return;
  const int h = static_cast<int>(i / nb);
  const int64_t t = i % nb;
  const int64_t j0 = ((t - kv_pos0 % nb) % nb + nb) % nb;   // first j of the block with (kv_pos0 + j) % nb == t
  float acc = 0.f;
  for (int b = 0; b < B; ++b) {
    const float* row = key_sums + (static_cast<int64_t>(b) * H + h) * Lb;
    for (int64_t j = j0; j < Lb; j += nb) acc += row[j];
  }
  dbias[i] = accumulate ? dbias[i] + acc : acc;
}

hipError_t launch_bias_grad_block(const float* key_sums, float* dbias, int B, int H, int64_t Lb, int64_t kv_pos0,
                                  int64_t bias_len, int accumulate, hipStream_t st) {
  const int64_t n = static_cast<int64_t>(H) * bias_len;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(bias_grad_block_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st, key_sums,
                     dbias, B, H, Lb, kv_pos0, bias_len, accumulate);
  return hipGetLastError();
}

hipError_t launch_bias_grad(const float* key_sums, float* dbias, int B, int H, int64_t Lk, int64_t bias_len,
                            hipStream_t st) {
  const int64_t n = static_cast<int64_t>(H) * bias_len;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(bias_grad_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st, key_sums, dbias,
                     B, H, Lk, bias_len);
  return hipGetLastError();
}

hipError_t launch_fwd_finalize(const Params& p, hipStream_t st) {
  return p.bf16 ? launch_finalize_t<__bf16>(p, st) : launch_finalize_t<float>(p, st);
}
hipError_t launch_merge(const Params& p, const void* out_b, const float* lse_b, hipStream_t st) {
  return p.bf16 ? launch_merge_t<__bf16>(p, out_b, lse_b, st) : launch_merge_t<float>(p, out_b, lse_b, st);
}

hipError_t launch_bwd_preprocess(const Params& p, hipStream_t st) {
  return p.bf16 ? launch_bwd_preprocess_t<__bf16>(p, st) : launch_bwd_preprocess_t<float>(p, st);
}
hipError_t launch_bwd_dkdv_simt(const Params& p, hipStream_t st) {
  return p.bf16 ? launch_bwd_dkdv_simt_t<__bf16>(p, st) : launch_bwd_dkdv_simt_t<float>(p, st);
}
hipError_t launch_bwd_dq_simt(const Params& p, hipStream_t st) {
  return p.bf16 ? launch_bwd_dq_simt_t<__bf16>(p, st) : launch_bwd_dq_simt_t<float>(p, st);
}

}  // namespace ra
