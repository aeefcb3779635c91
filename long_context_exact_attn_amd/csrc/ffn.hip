// Blockwise feed-forward (SwiGLU), bfloat16 in / float32 accumulate, on this library's own MFMA
// GEMM (gemm.cuh).
//
// The feed-forward is applied chunk by chunk over the tokens ("RingAttention核心功能全解析",
// 快速上手, blockwise_feedforward), so the [tokens, d_ff] intermediate exists for one chunk at a
// time.  Matrices are row-major: x, out, dout, dx [tokens, d]; W1, W3 [f, d]; W2 [d, f].
//
// Forward, per chunk:
//   h = silu(x W1^T) * (x W3^T)   one GEMM against W1 and W3 together: each workgroup's B tile
//                                 holds 64 rows of W1 and the same 64 rows of W3, so a lane owns g
//                                 and u of the same (token, j) and the gate runs in the epilogue
//   out = h W2^T
// Backward, per chunk (the intermediate is recomputed):
//   dh = dout W2                  stored, bfloat16
//   [g u] = x [W1; W3]^T          epilogue: dg = dh u silu'(g), du = dh silu(g), h = silu(g) u
//   dx = [dg du] [W1; W3]
//   [dW1; dW3] (+)= [dg du]^T x,  dW2 (+)= dout^T h     float32, split over K (tokens) into partial
//                                 sums that a small kernel adds in a fixed order (deterministic)
#include "gemm.cuh"

namespace ra {
namespace {

using gemm::Operand;

constexpr int64_t kNone = INT64_MAX;

__device__ __forceinline__ float sigmoidf_(float a) {
  return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-a * kLog2e));
}

// B rows of the gate GEMM: tile rows 32 b + r (b = 0..7) hold W1 (b even) or W3 (b odd) row
// j = n0 / 2 + 32 (b / 2) + r, as rows j and f + j of the virtual stacked [W1; W3]
struct GateRows {
  int64_t f;
  __device__ int64_t operator()(int64_t n0, int r) const {
    const int b = r >> 5;
    const int64_t j = n0 / 2 + 32 * (b >> 1) + (r & 31);
    if (j >= f) return 2 * f;   // past the last row: the zero chunk
    return (b & 1) ? f + j : j;
  }
};

struct StoreBf16 {
  __bf16* C;
  int64_t ldc;
  __device__ void operator()(const f32x16 (&acc)[4][2], int64_t mb0, int64_t nb0, int, int l32, int hh, int64_t M,
                             int64_t N) const {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int64_t m = mb0 + 32 * a + l32;
      if (m >= M) continue;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int64_t n = nb0 + 32 * b + 8 * g + 4 * hh;   // N is a multiple of 8: n < N covers n + 3
          if (n >= N) continue;
          bf16x4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = (__bf16)acc[a][b][4 * g + e];
          *reinterpret_cast<bf16x4*>(C + m * ldc + n) = o;
        }
    }
  }
};

// h = silu(g) u into H [M, f]: block b = 0 of the wave holds g, b = 1 holds u, of hidden units
// j = nb0 / 2 + 8 g + 4 hh + e
struct GateFwd {
  __bf16* H;
  int64_t f;
  __device__ void operator()(const f32x16 (&acc)[4][2], int64_t mb0, int64_t nb0, int, int l32, int hh, int64_t M,
                             int64_t) const {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int64_t m = mb0 + 32 * a + l32;
      if (m >= M) continue;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t j = nb0 / 2 + 8 * g + 4 * hh;   // f is a multiple of 8: j < f covers j + 3
        if (j >= f) continue;
        bf16x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float gv = acc[a][0][4 * g + e], uv = acc[a][1][4 * g + e];
          o[e] = (__bf16)(gv * sigmoidf_(gv) * uv);
        }
        *reinterpret_cast<bf16x4*>(H + m * f + j) = o;
      }
    }
  }
};

// The backward's gate product [g u] = x [W1; W3]^T with the gate's derivative in its epilogue:
// with dh = dout W2 already in DH [M, f] and s = sigmoid(g),
//   dg = dh u s (1 + g (1 - s)),  du = dh g s   into DGDU [M, 2 f] (g's columns, then u's)
//   h = g s u                                   into H [M, f]
// so g and u never leave the registers.  Four hidden units per access.
//
// The wave's results for one row m and four hidden units j .. j + 3 from its g and u accumulators
__device__ __forceinline__ void gate_bwd_units(__bf16* __restrict__ DGDU, __bf16* __restrict__ H, const f32x16 (&acc)[2],
                                               int g, bf16x4 dh, int64_t m, int64_t j, int64_t f) {
  bf16x4 dg, du, h;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float gv = acc[0][4 * g + e], uv = acc[1][4 * g + e], sv = sigmoidf_(gv), d = (float)dh[e];
    dg[e] = (__bf16)(d * uv * sv * (1.f + gv * (1.f - sv)));
    du[e] = (__bf16)(d * gv * sv);
    h[e] = (__bf16)(gv * sv * uv);
  }
  *reinterpret_cast<bf16x4*>(DGDU + m * 2 * f + j) = dg;
  *reinterpret_cast<bf16x4*>(DGDU + m * 2 * f + f + j) = du;
  *reinterpret_cast<bf16x4*>(H + m * f + j) = h;
}

struct GateBwd {
  const __bf16* DH;
  __bf16* DGDU;
  __bf16* H;
  int64_t f;
  __device__ void operator()(const f32x16 (&acc)[4][2], int64_t mb0, int64_t nb0, int, int l32, int hh, int64_t M,
                             int64_t) const {
    const int64_t j0 = nb0 / 2 + 4 * hh;   // the lane's first hidden unit; it owns j0 + 8 g + 0..3
    if (mb0 + 128 <= M && nb0 / 2 + 32 <= f) {
      // the wave's 128 rows and 32 hidden units are all inside: every dh load is issued before the first
      // store, with no branch in between.  (Stores count in the same counter as loads; with a branch
      // around each load, the wait for a row's dh also waited for every store issued before it.)
      bf16x4 dh[4][4];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          dh[a][g] = *reinterpret_cast<const bf16x4*>(DH + (mb0 + 32 * a + l32) * f + j0 + 8 * g);
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int g = 0; g < 4; ++g) gate_bwd_units(DGDU, H, acc[a], g, dh[a][g], mb0 + 32 * a + l32, j0 + 8 * g, f);
      return;
    }
    // a ragged tile: rows past M and hidden units past f are left out, one row at a time
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int64_t m = mb0 + 32 * a + l32;
      if (m >= M) continue;
      bf16x4 dh[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t j = j0 + 8 * g;
        dh[g] = j < f ? *reinterpret_cast<const bf16x4*>(DH + m * f + j) : bf16x4{};
      }
#pragma unroll
      for (int g = 0; g < 4; ++g)
        if (j0 + 8 * g < f) gate_bwd_units(DGDU, H, acc[a], g, dh[g], m, j0 + 8 * g, f);
    }
  }
};

// float32 result rows [0, rsplit) into out1 and the rest into out2 (row length ldo): written
// (splits == 1) or as split `split`'s partial sum into part [splits][M][N]; four columns per store
struct F32Out {
  float* out1;
  float* out2;
  int64_t rsplit, ldo;
  float* part;
  int splits;
  int accumulate;
  __device__ void operator()(const f32x16 (&acc)[4][2], int64_t mb0, int64_t nb0, int split, int l32, int hh,
                             int64_t M, int64_t N) const {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int64_t m = mb0 + 32 * a + l32;
      if (m >= M) continue;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int64_t n = nb0 + 32 * b + 8 * g + 4 * hh;   // N is a multiple of 8
          if (n >= N) continue;
          f32x4 x;
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = acc[a][b][4 * g + e];
          if (splits > 1) {
            *reinterpret_cast<f32x4*>(part + (static_cast<int64_t>(split) * M + m) * N + n) = x;
          } else {
            float* o = m < rsplit ? out1 + m * ldo + n : out2 + (m - rsplit) * ldo + n;
            if (accumulate) x += *reinterpret_cast<const f32x4*>(o);
            *reinterpret_cast<f32x4*>(o) = x;
          }
        }
    }
  }
};

// out (+)= sum over s = 0 .. splits - 1 of part[s] (in that order), rows split over out1 / out2; four
// consecutive columns per thread (N is a multiple of 8 and every pointer 16-byte aligned)
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part, float* out1, float* out2,
                                                            int64_t rsplit, int64_t ldo, int64_t M, int64_t N,
                                                            int splits, int accumulate) {
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) * 4;
  if (i >= M * N) return;
  const int64_t m = i / N, n = i % N;
  float* o = m < rsplit ? out1 + m * ldo + n : out2 + (m - rsplit) * ldo + n;
  f32x4 s = accumulate ? *reinterpret_cast<const f32x4*>(o) : f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < splits; ++k) s += *reinterpret_cast<const f32x4*>(part + static_cast<int64_t>(k) * M * N + i);
  *reinterpret_cast<f32x4*>(o) = s;
}

#define RA_HIP(x)                         \
  do {                                    \
    const hipError_t e_ = (x);            \
    if (e_ != hipSuccess) return e_;      \
  } while (0)

int cdiv(int64_t a, int64_t b) { return static_cast<int>((a + b - 1) / b); }

// C [M, N] of A [M, K] and B [K, N] on tiles_n column tiles (the gate GEMM's tiles hold 128 columns
// of h); the B tile at column n0 lies inside B when n0 + BN <= N
template <bool AK, bool BK_, typename Map, typename Epi>
hipError_t run(const Operand& A, const Operand& B, int64_t M, int64_t N, int64_t K, int tiles_n, int splits, Map map,
               Epi epi, hipStream_t st) {
  const int tiles_m = cdiv(M, gemm::BM);
  const int64_t kps = (cdiv(K, splits * gemm::BK)) * static_cast<int64_t>(gemm::BK);
  const int64_t grid = static_cast<int64_t>(tiles_m) * tiles_n * splits;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((gemm::gemm_kernel<AK, BK_, Map, Epi>), dim3(static_cast<unsigned>(grid)), dim3(gemm::kThreadsG),
                     0, st, A, B, M, N, K, tiles_m, tiles_n, splits, kps, N, map, epi);
  return hipGetLastError();
}

constexpr int kMaxSplits = 4;   // the partial sums' extra traffic grows with the splits
constexpr int kSlots = 256;   // workgroups resident at once: one 128 KiB-LDS workgroup per CU

// K splits for the weight-gradient products: enough workgroups to fill the chip in whole rounds,
// each split at least 512 deep
int pick_splits(int64_t tiles, int64_t K) {
  int best = 1;
  double best_eff = 0.0;
  for (int s = 1; s <= kMaxSplits; ++s) {
    if (s > 1 && K / s < 512) break;
    const int64_t wg = tiles * s;
    const int64_t rounds = (wg + kSlots - 1) / kSlots;
    const double eff = static_cast<double>(wg) / static_cast<double>(rounds * kSlots);
    if (eff > best_eff + 1e-9) {
      best_eff = eff;
      best = s;
    }
  }
  return best;
}

Operand op(const __bf16* base, int64_t ld, int64_t rows, int64_t kdim, const __bf16* base2 = nullptr,
           int64_t split = kNone) {
  Operand o;
  o.base = base;
  o.base2 = base2 ? base2 : base;
  o.ld = ld;
  o.split = split;
  o.rows = rows;
  o.kdim = kdim;
  return o;
}

// the float32 weight-gradient product C [M, N] (+)= A B over the chunk's tokens, split over K
template <typename Map>
hipError_t weight_grad(const Operand& A, const Operand& B, int64_t M, int64_t N, int64_t K, float* out1, float* out2,
                       int64_t rsplit, int accumulate, float* part, int splits, Map map, hipStream_t st) {
  const int tiles_n = cdiv(N, gemm::BN);
  F32Out epi{out1, out2, rsplit, N, part, splits, accumulate};
  RA_HIP((run<false, false>(A, B, M, N, K, tiles_n, splits, map, epi, st)));
  if (splits > 1) {
    const int64_t n4 = M * N / 4;   // N is a multiple of 8
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3(static_cast<unsigned>((n4 + 255) / 256)), dim3(256), 0, st, part,
                       out1, out2, rsplit, N, M, N, splits, accumulate);
    RA_HIP(hipGetLastError());
  }
  return hipSuccess;
}

}  // namespace

FfnWorkspace ffn_workspace(int64_t tokens, int d_model, int d_ff, int64_t chunk, bool backward) {
  auto up = [](size_t b) { return (b + 255) / 256 * 256; };
  const int64_t c = tokens < chunk ? tokens : chunk;
  const size_t f = static_cast<size_t>(d_ff), d = static_cast<size_t>(d_model);
  FfnWorkspace w{};
  size_t off = 0;
  w.h = off; off += up(f * c * 2);             // silu(g) * u of a chunk, bf16
  if (backward) {
    w.gu = off; off += up(f * c * 2);          // dh = dout W2 of a chunk, bf16
    w.dgdu = off; off += up(2 * f * c * 2);    // gradients of g and u, stacked like gu, bf16
    // partial sums of the split weight-gradient products
    const int s13 = pick_splits(static_cast<int64_t>(cdiv(2 * f, gemm::BM)) * cdiv(d, gemm::BN), c);
    const int s2 = pick_splits(static_cast<int64_t>(cdiv(d, gemm::BM)) * cdiv(f, gemm::BN), c);
    const size_t p13 = s13 > 1 ? static_cast<size_t>(s13) * 2 * f * d : 0, p2 = s2 > 1 ? static_cast<size_t>(s2) * d * f : 0;
    w.dw13 = off; off += up((p13 > p2 ? p13 : p2) * 4);
  }
  w.bytes = off;
  return w;
}

hipError_t ffn_forward(const __bf16* x, const __bf16* w1, const __bf16* w3, const __bf16* w2, __bf16* out,
                       int64_t tokens, int d, int f, int64_t chunk, char* ws, hipStream_t st) {
  const FfnWorkspace w = ffn_workspace(tokens, d, f, chunk, false);
  __bf16* h = reinterpret_cast<__bf16*>(ws + w.h);
  for (int64_t t0 = 0; t0 < tokens; t0 += chunk) {
    const int64_t c = tokens - t0 < chunk ? tokens - t0 : chunk;
    const __bf16* xc = x + t0 * d;
    // h = silu(x W1^T) * (x W3^T): B rows are those of the virtual [W1; W3] (split at f)
    RA_HIP((run<true, true>(op(xc, d, c, d), op(w1, d, 2 * int64_t(f), d, w3, f), c, 2 * int64_t(f), d,
                            cdiv(f, gemm::BN / 2), 1, GateRows{f}, GateFwd{h, f}, st)));
    // out = h W2^T
    RA_HIP((run<true, true>(op(h, f, c, f), op(w2, f, d, f), c, d, f, cdiv(d, gemm::BN), 1, gemm::LinearRows{},
                            StoreBf16{out + t0 * d, d}, st)));
  }
  return hipSuccess;
}

hipError_t ffn_backward(const __bf16* x, const __bf16* w1, const __bf16* w3, const __bf16* w2, const __bf16* dout,
                        __bf16* dx, float* dw1, float* dw3, float* dw2, int64_t tokens, int d, int f, int64_t chunk,
                        char* ws, hipStream_t st) {
  if (tokens == 0) {
    // no token contributes: the weight gradients are zero
    RA_HIP(launch_fill_zero(dw1, static_cast<int64_t>(f) * d, st));
    RA_HIP(launch_fill_zero(dw3, static_cast<int64_t>(f) * d, st));
    RA_HIP(launch_fill_zero(dw2, static_cast<int64_t>(d) * f, st));
    return hipSuccess;
  }
  const FfnWorkspace w = ffn_workspace(tokens, d, f, chunk, true);
  __bf16* h = reinterpret_cast<__bf16*>(ws + w.h);
  __bf16* dhb = reinterpret_cast<__bf16*>(ws + w.gu);
  __bf16* dgdu = reinterpret_cast<__bf16*>(ws + w.dgdu);
  float* part = reinterpret_cast<float*>(ws + w.dw13);
  const int64_t F = f, F2 = 2 * int64_t(f), Dm = d;
  for (int64_t t0 = 0; t0 < tokens; t0 += chunk) {
    const int64_t c = tokens - t0 < chunk ? tokens - t0 : chunk;
    const int acc = t0 == 0 ? 0 : 1;   // weight gradients: the first chunk writes, later ones add
    const __bf16* xc = x + t0 * d;
    const __bf16* dc = dout + t0 * d;
    // dh = dout W2 (W2 is [d, f] = [K, N])
    RA_HIP((run<true, false>(op(dc, Dm, c, Dm), op(w2, F, F, Dm), c, F, Dm, cdiv(F, gemm::BN), 1, gemm::LinearRows{},
                             StoreBf16{dhb, F}, st)));
    // [g u] = x [W1; W3]^T, with the gate's derivative and h in the epilogue
    RA_HIP((run<true, true>(op(xc, Dm, c, Dm), op(w1, Dm, F2, Dm, w3, F), c, F2, Dm, cdiv(F, gemm::BN / 2), 1,
                            GateRows{F}, GateBwd{dhb, dgdu, h, F}, st)));
    // dx = [dg du] [W1; W3] ([W1; W3] is [2 f, d] = [K, N], split at K = f)
    RA_HIP((run<true, false>(op(dgdu, F2, c, F2), op(w1, Dm, Dm, F2, w3, F), c, Dm, F2, cdiv(Dm, gemm::BN), 1,
                             gemm::LinearRows{}, StoreBf16{dx + t0 * d, Dm}, st)));
    // [dW1; dW3] (+)= [dg du]^T x: A = [dg du] stored [c, 2 f] = [K, M]; B = x [c, d] = [K, N]
    const int s13 = pick_splits(static_cast<int64_t>(cdiv(F2, gemm::BM)) * cdiv(Dm, gemm::BN), c);
    RA_HIP(weight_grad(op(dgdu, F2, F2, c), op(xc, Dm, Dm, c), F2, Dm, c, dw1, dw3, F, acc, part, s13,
                       gemm::LinearRows{}, st));
    // dW2 (+)= dout^T h: A = dout stored [c, d] = [K, M]; B = h [c, f] = [K, N]
    const int s2 = pick_splits(static_cast<int64_t>(cdiv(Dm, gemm::BM)) * cdiv(F, gemm::BN), c);
    RA_HIP(weight_grad(op(dc, Dm, Dm, c), op(h, F, F, c), Dm, F, c, dw2, dw2, Dm, acc, part, s2, gemm::LinearRows{},
                       st));
  }
  return hipSuccess;
}

}  // namespace ra
