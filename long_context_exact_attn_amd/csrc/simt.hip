// One-lane-per-row kernels of libra_attn, for both dtypes: the backward preprocess
// Delta = rowsum(dO * O), the ring-step finalize and merge, the float32-to-output conversion of
// gradient sums, the fixed-order reductions that form the bias gradient from per-key sums, and a
// zero fill (a kernel, not a memset, so that a caller may capture the call in a HIP graph).
#include "ra_common.cuh"

namespace ra {
namespace {

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

}  // namespace

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

// p[0 .. n) = 0 (grid-stride)
__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ p, int64_t n) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0.f;
}

hipError_t launch_bias_grad_block(const float* key_sums, float* dbias, int B, int H, int64_t Lb, int64_t kv_pos0,
                                  int64_t bias_len, int accumulate, hipStream_t st) {
  const int64_t n = static_cast<int64_t>(H) * bias_len;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(bias_grad_block_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st, key_sums,
                     dbias, B, H, Lb, kv_pos0, bias_len, accumulate);
  return hipGetLastError();
}

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(static_cast<unsigned>(blocks < 65536 ? blocks : 65536)), dim3(256), 0, st,
                     p, n);
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
}  // namespace ra
