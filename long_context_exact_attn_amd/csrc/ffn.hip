// Blockwise feed-forward (SwiGLU), bfloat16 in / float32 accumulate.
//
// The feed-forward is applied chunk by chunk over the tokens ("RingAttention核心功能全解析",
// 快速上手, blockwise_feedforward), so the [tokens, d_ff] intermediate exists for one chunk at a
// time.  The three products per chunk are plain GEMMs and run on rocBLAS (bf16 inputs, float32
// accumulation); the SwiGLU gate and its derivative are hand-written elementwise kernels between
// them.  Matrices are row-major; a row-major [r, c] matrix is handed to the column-major GEMM as
// its [c, r] transpose, so y = x W^T for a row-major weight W [out, in] becomes the column-major
// product Y^T = W_cm^T X^T with W_cm = W^T.
#include <rocblas/rocblas.h>

#include <mutex>

#include "ra_common.cuh"

namespace ra {
namespace {

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float sigmoid(float a) { return 1.f / (1.f + __expf(-a)); }

// The gate and up projections of a chunk come out of one GEMM against the stacked weight
// [W1; W3]: column j of gu (column-major [2 d_ff, chunk]) holds g = W1 x_j in rows [0, d_ff) and
// u = W3 x_j in rows [d_ff, 2 d_ff).  Four elements of a column per lane (d_ff % 4 == 0).

// h[:, j] = silu(g) * u
__global__ __launch_bounds__(256) void swiglu_fwd_kernel(const __bf16* __restrict__ gu, __bf16* __restrict__ h, int f,
                                                         int64_t n4) {
  const int64_t i4 = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i4 >= n4) return;
  const int64_t e = 4 * i4, j = e / f, r = e % f;
  const bf16x4 a = *reinterpret_cast<const bf16x4*>(gu + j * 2 * f + r);
  const bf16x4 b = *reinterpret_cast<const bf16x4*>(gu + j * 2 * f + f + r);
  bf16x4 o;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float g = (float)a[k];
    o[k] = (__bf16)(g * sigmoid(g) * (float)b[k]);
  }
  *reinterpret_cast<bf16x4*>(h + e) = o;
}

// dg = dh * u * silu'(g), du = dh * silu(g), with silu'(g) = s (1 + g (1 - s)), s = sigmoid(g);
// written in the stacked layout of gu, so that one GEMM against [W1; W3] gives dx
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const __bf16* __restrict__ dh, const __bf16* __restrict__ gu,
                                                         __bf16* __restrict__ dgdu, int f, int64_t n4) {
  const int64_t i4 = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i4 >= n4) return;
  const int64_t e = 4 * i4, j = e / f, r = e % f;
  const bf16x4 d = *reinterpret_cast<const bf16x4*>(dh + e);
  const bf16x4 a = *reinterpret_cast<const bf16x4*>(gu + j * 2 * f + r);
  const bf16x4 b = *reinterpret_cast<const bf16x4*>(gu + j * 2 * f + f + r);
  bf16x4 og, ou;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float g = (float)a[k], u = (float)b[k], dd = (float)d[k];
    const float s = sigmoid(g);
    og[k] = (__bf16)(dd * u * s * (1.f + g * (1.f - s)));
    ou[k] = (__bf16)(dd * g * s);
  }
  *reinterpret_cast<bf16x4*>(dgdu + j * 2 * f + r) = og;
  *reinterpret_cast<bf16x4*>(dgdu + j * 2 * f + f + r) = ou;
}

// One rocBLAS handle per device, created on first use and kept for the process.
std::mutex g_blas_mutex;
rocblas_handle g_blas[64] = {};

hipError_t blas_handle(rocblas_handle* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  if (!g_blas[dev] && rocblas_create_handle(&g_blas[dev]) != rocblas_status_success) return hipErrorNotInitialized;
  *out = g_blas[dev];
  return hipSuccess;
}

// column-major C[m, n] = alpha op(A) op(B) + beta C, bf16 A and B, float32 accumulation
hipError_t gemm(rocblas_handle hd, bool ta, bool tb, int64_t m, int64_t n, int64_t k, const void* A, int64_t lda,
                const void* B, int64_t ldb, float beta, void* C, bool c_bf16, int64_t ldc) {
  const float alpha = 1.f;
  const rocblas_datatype ct = c_bf16 ? rocblas_datatype_bf16_r : rocblas_datatype_f32_r;
  const rocblas_status s = rocblas_gemm_ex(
      hd, ta ? rocblas_operation_transpose : rocblas_operation_none, tb ? rocblas_operation_transpose : rocblas_operation_none,
      static_cast<rocblas_int>(m), static_cast<rocblas_int>(n), static_cast<rocblas_int>(k), &alpha, A,
      rocblas_datatype_bf16_r, static_cast<rocblas_int>(lda), B, rocblas_datatype_bf16_r, static_cast<rocblas_int>(ldb),
      &beta, C, ct, static_cast<rocblas_int>(ldc), C, ct, static_cast<rocblas_int>(ldc), rocblas_datatype_f32_r,
      rocblas_gemm_algo_standard, 0, 0);
  return s == rocblas_status_success ? hipSuccess : hipErrorLaunchFailure;
}

#define RA_HIP(x)                         \
  do {                                    \
    const hipError_t e_ = (x);            \
    if (e_ != hipSuccess) return e_;      \
  } while (0)

dim3 grid4(int64_t n4) { return dim3(static_cast<unsigned>((n4 + 255) / 256)); }

}  // namespace

FfnWorkspace ffn_workspace(int64_t tokens, int d_model, int d_ff, int64_t chunk, bool backward) {
  auto up = [](size_t b) { return (b + 255) / 256 * 256; };
  const int64_t c = tokens < chunk ? tokens : chunk;
  const size_t f = static_cast<size_t>(d_ff), d = static_cast<size_t>(d_model);
  FfnWorkspace w{};
  size_t off = 0;
  w.w13 = off; off += up(2 * f * d * 2);       // [W1; W3], bf16
  w.gu = off; off += up(2 * f * c * 2);        // gate and up projections of a chunk, bf16
  w.h = off; off += up(f * c * 2);             // silu(g) * u, bf16
  if (backward) {
    w.dh = off; off += up(f * c * 2);          // W2^T dout, bf16
    w.dgdu = off; off += up(2 * f * c * 2);    // gradients of g and u, stacked like gu, bf16
    w.dw13 = off; off += up(2 * f * d * 4);    // [dW1; dW3] sums, float32
  }
  w.bytes = off;
  return w;
}

namespace {
// [W1; W3] stacked (row-major [2 d_ff, d_model]) in the workspace
hipError_t stack_weights(const __bf16* w1, const __bf16* w3, __bf16* w13, int d, int f, hipStream_t st) {
  const size_t bytes = static_cast<size_t>(f) * d * sizeof(__bf16);
  RA_HIP(hipMemcpyAsync(w13, w1, bytes, hipMemcpyDeviceToDevice, st));
  return hipMemcpyAsync(w13 + static_cast<size_t>(f) * d, w3, bytes, hipMemcpyDeviceToDevice, st);
}
}  // namespace

hipError_t ffn_forward(const __bf16* x, const __bf16* w1, const __bf16* w3, const __bf16* w2, __bf16* out,
                       int64_t tokens, int d, int f, int64_t chunk, char* ws, hipStream_t st) {
  std::lock_guard<std::mutex> lock(g_blas_mutex);
  rocblas_handle hd;
  RA_HIP(blas_handle(&hd));
  if (rocblas_set_stream(hd, st) != rocblas_status_success) return hipErrorInvalidValue;
  const FfnWorkspace w = ffn_workspace(tokens, d, f, chunk, false);
  __bf16* w13 = reinterpret_cast<__bf16*>(ws + w.w13);
  __bf16* gu = reinterpret_cast<__bf16*>(ws + w.gu);
  __bf16* h = reinterpret_cast<__bf16*>(ws + w.h);
  RA_HIP(stack_weights(w1, w3, w13, d, f, st));
  for (int64_t t0 = 0; t0 < tokens; t0 += chunk) {
    const int64_t c = tokens - t0 < chunk ? tokens - t0 : chunk;
    const __bf16* xc = x + t0 * d;
    RA_HIP(gemm(hd, true, false, 2 * f, c, d, w13, d, xc, d, 0.f, gu, true, 2 * f));   // [g; u]^T = [W1; W3] x^T
    const int64_t n4 = static_cast<int64_t>(f) * c / 4;
    hipLaunchKernelGGL(swiglu_fwd_kernel, grid4(n4), dim3(256), 0, st, gu, h, f, n4);
    RA_HIP(hipGetLastError());
    RA_HIP(gemm(hd, true, false, d, c, f, w2, f, h, f, 0.f, out + t0 * d, true, d));   // y^T = W2 h^T
  }
  return hipSuccess;
}

hipError_t ffn_backward(const __bf16* x, const __bf16* w1, const __bf16* w3, const __bf16* w2, const __bf16* dout,
                        __bf16* dx, float* dw1, float* dw3, float* dw2, int64_t tokens, int d, int f, int64_t chunk,
                        char* ws, hipStream_t st) {
  std::lock_guard<std::mutex> lock(g_blas_mutex);
  if (tokens == 0) {
    // no token contributes: the weight gradients are zero
    RA_HIP(hipMemsetAsync(dw1, 0, sizeof(float) * f * d, st));
    RA_HIP(hipMemsetAsync(dw3, 0, sizeof(float) * f * d, st));
    RA_HIP(hipMemsetAsync(dw2, 0, sizeof(float) * d * f, st));
    return hipSuccess;
  }
  rocblas_handle hd;
  RA_HIP(blas_handle(&hd));
  if (rocblas_set_stream(hd, st) != rocblas_status_success) return hipErrorInvalidValue;
  const FfnWorkspace w = ffn_workspace(tokens, d, f, chunk, true);
  __bf16* w13 = reinterpret_cast<__bf16*>(ws + w.w13);
  __bf16* gu = reinterpret_cast<__bf16*>(ws + w.gu);
  __bf16* h = reinterpret_cast<__bf16*>(ws + w.h);
  __bf16* dh = reinterpret_cast<__bf16*>(ws + w.dh);
  __bf16* dgdu = reinterpret_cast<__bf16*>(ws + w.dgdu);
  float* dw13 = reinterpret_cast<float*>(ws + w.dw13);
  RA_HIP(stack_weights(w1, w3, w13, d, f, st));
  for (int64_t t0 = 0; t0 < tokens; t0 += chunk) {
    const int64_t c = tokens - t0 < chunk ? tokens - t0 : chunk;
    const float acc = t0 == 0 ? 0.f : 1.f;   // weight gradients: the first chunk overwrites
    const __bf16* xc = x + t0 * d;
    const __bf16* dc = dout + t0 * d;
    const int64_t n4 = static_cast<int64_t>(f) * c / 4;
    // recompute the chunk's intermediate
    RA_HIP(gemm(hd, true, false, 2 * f, c, d, w13, d, xc, d, 0.f, gu, true, 2 * f));
    hipLaunchKernelGGL(swiglu_fwd_kernel, grid4(n4), dim3(256), 0, st, gu, h, f, n4);
    RA_HIP(hipGetLastError());
    RA_HIP(gemm(hd, false, false, f, c, d, w2, f, dc, d, 0.f, dh, true, f));               // dh^T = W2^T dout^T
    hipLaunchKernelGGL(swiglu_bwd_kernel, grid4(n4), dim3(256), 0, st, dh, gu, dgdu, f, n4);
    RA_HIP(hipGetLastError());
    RA_HIP(gemm(hd, false, false, d, c, 2 * f, w13, d, dgdu, 2 * f, 0.f, dx + t0 * d, true, d));   // dx^T
    RA_HIP(gemm(hd, false, true, d, 2 * f, c, xc, d, dgdu, 2 * f, acc, dw13, false, d));   // [dW1; dW3]^T += x^T [dg du]
    RA_HIP(gemm(hd, false, true, f, d, c, h, f, dc, d, acc, dw2, false, f));               // dW2^T += h^T dout
  }
  const size_t bytes = sizeof(float) * f * d;
  RA_HIP(hipMemcpyAsync(dw1, dw13, bytes, hipMemcpyDeviceToDevice, st));
  return hipMemcpyAsync(dw3, dw13 + static_cast<size_t>(f) * d, bytes, hipMemcpyDeviceToDevice, st);
}

}  // namespace ra
