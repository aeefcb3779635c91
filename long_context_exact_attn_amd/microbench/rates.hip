// Issue-rate microbenchmarks for gfx950, used to set the ceilings the attention kernels are
// measured against: sustained v_mfma_f32_32x32x16_bf16 throughput, cycles per wave64
// instruction of v_exp_f32, v_fma_f32, v_dot2_f32_bf16 and v_max, and whether exponentials
// issued between matrix products of one wave overlap them, and LDS read bandwidth.  Every thread writes one float
// of `out` (sized for the largest grid); nothing else is read or written.
#include <hip/hip_runtime.h>
#include <cstdio>
#include <cstdlib>
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
constexpr int N = 4096;

__global__ __launch_bounds__(256) void k_mfma(float* out, float seed) {
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) { a[i] = (__bf16)(seed * i); b[i] = (__bf16)(seed + i); }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < N; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0; for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}
template <int OP>
__global__ __launch_bounds__(256) void k_valu(float* out, float seed) {
  float x[8];
  _Float16 xh[8];
  for (int i = 0; i < 8; ++i) {
    x[i] = seed * (threadIdx.x + i);
    xh[i] = (_Float16)x[i];
  }
  bf16x2 one = {(__bf16)1.f, (__bf16)1.f};
  for (int it = 0; it < N; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (OP == 0) x[i] = __builtin_amdgcn_exp2f(-x[i]);
      if (OP == 4) xh[i] = __builtin_elementwise_exp2(-xh[i]);
      if (OP == 1) x[i] = __builtin_fmaf(x[i], 0.999f, 0.001f);
      if (OP == 2) { bf16x2 p = {(__bf16)seed, (__bf16)(seed * 2)}; x[i] = __builtin_amdgcn_fdot2_f32_bf16(p, one, x[i], false); }
      if (OP == 3) x[i] = fmaxf(fmaxf(x[i], seed), x[(i + 1) & 7]);
    }
  }
  float s = 0; for (int i = 0; i < 8; ++i) s += x[i] + (float)xh[i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}
// one wave mixes MFMA chains with exp chains: do the pipes overlap?
template <int NEXP>
__global__ __launch_bounds__(256) void k_mix(float* out, float seed) {
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) { a[i] = (__bf16)(seed * i); b[i] = (__bf16)(seed + i); }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  float x[8];
  for (int i = 0; i < 8; ++i) x[i] = seed * (threadIdx.x + i);
  for (int it = 0; it < N; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < NEXP / 4; ++i) x[i & 7] = __builtin_amdgcn_exp2f(-x[i & 7]);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < NEXP / 4; ++i) x[(i + 2) & 7] = __builtin_amdgcn_exp2f(-x[(i + 2) & 7]);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < NEXP / 4; ++i) x[(i + 4) & 7] = __builtin_amdgcn_exp2f(-x[(i + 4) & 7]);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < NEXP / 4; ++i) x[(i + 6) & 7] = __builtin_amdgcn_exp2f(-x[(i + 6) & 7]);
  }
  float s = 0; for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  for (int i = 0; i < 8; ++i) s += x[i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// wave-specialised: in a 512-thread workgroup (two waves per SIMD) waves 0-3 run only matrix
// products and waves 4-7 only VALU work (OP 0: v_exp_f32, 1: v_fma_f32; 8 independent chains);
// timing each part alone and both together shows whether the SIMD overlaps them across waves.
template <int OP>
__global__ __launch_bounds__(512) void k_split(float* out, float seed, int n_mfma, int n_valu) {
  const int w = threadIdx.x >> 6;
  float s = 0;
  if (w < 4) {
    bf16x8 a, b;
    for (int i = 0; i < 8; ++i) { a[i] = (__bf16)(seed * i); b[i] = (__bf16)(seed + i); }
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < n_mfma; ++it) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    }
    for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  } else {
    float x[8];
    for (int i = 0; i < 8; ++i) x[i] = seed * (threadIdx.x + i);
    for (int it = 0; it < n_valu; ++it) {
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = OP == 0 ? __builtin_amdgcn_exp2f(-x[i]) : __builtin_fmaf(x[i], 0.999f, 0.001f);
    }
    for (int i = 0; i < 8; ++i) s += x[i];
  }
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// LDS read bandwidth with the attention kernels' operand patterns on a 64-column bf16 tile
// whose 16-byte chunks are XOR-swizzled by row: MODE 0 reads 16 bytes per lane (row l % 32,
// chunk 2 u + l / 32), MODE 1 the two 8-byte transposing reads of one transposed operand,
// MODE 2 a broadcast 16-byte read in which each half of the wave reads one address (the
// per-row statistics of a 32-row block, four rows per read).  The per-lane byte offsets are
// formed once; each read takes its offset through an empty asm statement, so that the compiler
// can neither hoist the loads out of the loop nor add address arithmetic to it.  Each wave
// reads its own 64-row region of a 32 KiB buffer; the loaded words are folded with xor.
typedef short i16x4 __attribute__((ext_vector_type(4)));
template <int MODE>
__global__ __launch_bounds__(256) void k_lds(float* out, int n) {
  __shared__ __attribute__((aligned(16))) __bf16 buf[16384];
  for (int i = threadIdx.x; i < 16384; i += 256) buf[i] = (__bf16)(float)(i & 255);
  __syncthreads();
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, l32 = lane & 31, hh = lane >> 5;
  const int region = w * 4096;   // element offset of the wave's 64 x 64 region (< 16384)
  int off[4], off2[4];           // byte offsets, per u
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    if (MODE == 0) {
      const int row = l32, chunk = (2 * u + hh) & 7;
      off[u] = 2 * (region + row * 64 + ((chunk ^ (row & 7)) << 3));
      off2[u] = 0;
    } else if (MODE == 2) {
      off[u] = 2 * region + 4 * (8 * u + 4 * hh);
      off2[u] = 0;
    } else {
      const int g = lane >> 4, gi = lane & 15;
      const int row = (u & 1) * 16 + 4 * hh + (gi >> 2);
      const int col = (u >> 1) * 32 + 16 * (g & 1) + 4 * (gi & 3);
      off[u] = 2 * (region + row * 64 + (((col >> 3) ^ (row & 7)) << 3) + (col & 7));
      off2[u] = 2 * (region + (row + 8) * 64 + (((col >> 3) ^ ((row + 8) & 7)) << 3) + (col & 7));
    }
  }
  const char* base = reinterpret_cast<const char*>(buf);
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  unsigned acc = 0;
  for (int it = 0; it < n; ++it) {
    int o[4] = {off[0], off[1], off[2], off[3]};
    int o2[4] = {off2[0], off2[1], off2[2], off2[3]};
    // one statement for all of the iteration's offsets: its four (eight) reads issue back to back
    asm volatile("" : "+v"(o[0]), "+v"(o[1]), "+v"(o[2]), "+v"(o[3]), "+v"(o2[0]), "+v"(o2[1]), "+v"(o2[2]),
                 "+v"(o2[3]));
    if (MODE != 1) {
      uint4 x[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) x[u] = *reinterpret_cast<const uint4*>(base + o[u]);
#pragma unroll
      for (int u = 0; u < 4; ++u) acc ^= x[u].x ^ x[u].y ^ x[u].z ^ x[u].w;
    } else {
      i16x4 lo[4], hi[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        lo[u] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + o[u]));
        hi[u] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + o2[u]));
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        acc ^= (unsigned)(unsigned short)lo[u][0] ^ ((unsigned)(unsigned short)lo[u][1] << 16) ^
               (unsigned)(unsigned short)lo[u][2] ^ ((unsigned)(unsigned short)lo[u][3] << 16) ^
               (unsigned)(unsigned short)hi[u][0] ^ ((unsigned)(unsigned short)hi[u][1] << 16) ^
               (unsigned)(unsigned short)hi[u][2] ^ ((unsigned)(unsigned short)hi[u][3] << 16);
    }
  }
  out[blockIdx.x * blockDim.x + threadIdx.x] = (float)acc;
}

// Phase alternation of the attention kernels: each wave runs a matrix phase (32 MFMAs: four
// accumulators, eight dependent products each) and then a vector phase that depends on it (64
// exponentials, 64 adds and bf16 packs, whose output is the next matrix phase's operand).  Two
// waves per SIMD.  MODE 0: one 8-wave workgroup per CU, free-running; MODE 1: a barrier after every
// phase, waves 0-3 and 4-7 in the same phase; MODE 2: the same barriers with waves 4-7 one phase
// behind (ping-pong); MODE 3: two 4-wave workgroups per CU, free-running; MODE 4: MODE 3 with one
// barrier per iteration in each workgroup (as the attention loops have per tile); MODE 5: MODE 4
// with the matrix phase's A operands read from LDS (seven 16-byte reads per iteration, each feeding
// four products, as the forward's K fragments do); MODE 6: MODE 5 plus direct global -> LDS copies
// of 16 KiB per workgroup and iteration (a K and a V tile of 64 x 64 bf16), issued at the start of
// the iteration and waited for before its barrier, as the forward's loop does.  The source is a
// 64 MiB buffer; workgroup w reads tile (131 w + it) mod 4096 of it.
template <int MODE>
__global__ __launch_bounds__(512) void k_phase(float* out, float seed, int n, const __bf16* src) {
  __shared__ __attribute__((aligned(16))) __bf16 sbuf[8192];
  __shared__ __attribute__((aligned(16))) __bf16 sdst[8192];   // MODE 6: the copies' destination
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (MODE >= 5) {
    for (int i = threadIdx.x; i < 8192; i += blockDim.x) sbuf[i] = (__bf16)(float)(i & 7);
    __syncthreads();
  }
  const int uwave = __builtin_amdgcn_readfirstlane(wave);
  auto copies = [&](int it) {
    // four 1 KiB copies per wave (4 waves x 4 KiB = 16 KiB); byte offset < 4096 * 16 KiB = 64 MiB
    const int64_t tile = (static_cast<int64_t>(blockIdx.x) * 131 + it) % 4096;
    const char* g = reinterpret_cast<const char*>(src) + tile * 16384 + uwave * 4096 + lane * 16;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const unsigned d = static_cast<unsigned>(
          reinterpret_cast<size_t>((__attribute__((address_space(3))) void*)(sdst + uwave * 2048 + k * 512)));
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                   : : "s"(d), "v"(g + k * 1024) : "memory", "m0");
    }
  };
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) { a[i] = (__bf16)(seed * i); b[i] = (__bf16)(seed + i); }
  f32x16 acc[4];
  for (int j = 0; j < 4; ++j) acc[j] = f32x16{};
  float lsum = 0.f;
  // MODE 5: per-lane byte offsets of eight 16-byte reads (row lane % 32, a swizzled chunk), inside
  // the wave's own 4 KiB region of sbuf (waves 0-3)
  int off[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int row = lane & 31, chunk = (2 * (k & 3) + (lane >> 5)) ^ (row & 7);
    off[k] = 2 * ((wave & 3) * 2048 + row * 64 + chunk * 8);
  }
  const char* sb = reinterpret_cast<const char*>(sbuf);
  auto mma_phase = [&]() {
    if constexpr (MODE >= 5) {
      int o[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) o[k] = off[k];
      asm volatile("" : "+v"(o[0]), "+v"(o[1]), "+v"(o[2]), "+v"(o[3]), "+v"(o[4]), "+v"(o[5]), "+v"(o[6]), "+v"(o[7]));
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        // step 0 takes the previous vector phase's output, the others an LDS fragment
        const bf16x8 aa = kk == 0 ? a : *reinterpret_cast<const bf16x8*>(sb + o[kk]);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aa, b, acc[j], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
    }
  };
  auto vec_phase = [&]() {
    float part = 0.f;
    bf16x8 na;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; v += 2) {
        const float e0 = __builtin_amdgcn_exp2f(acc[j][v] * -1e-6f);
        const float e1 = __builtin_amdgcn_exp2f(acc[j][v + 1] * -1e-6f);
        part += e0 + e1;
        const bf16x2 pr = __builtin_convertvector((f32x2){e0, e1}, bf16x2);
        na[(v >> 1) & 7] = pr[0];   // the last packs of the phase feed the next matrix phase
      }
    lsum += part;
    a = na;
  };
  if (MODE == 2 && wave >= 4) {
    vec_phase();
    __syncthreads();
  }
  for (int it = 0; it < n; ++it) {
    if (MODE == 6) copies(it);
    mma_phase();
    if (MODE == 1 || MODE == 2) __syncthreads();
    vec_phase();
    if (MODE == 6) __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));   // vmcnt(0)
    if (MODE != 0 && MODE != 3) __syncthreads();
  }
  if (MODE == 2 && wave < 4) __syncthreads();
  float s2 = lsum;
  for (int j = 0; j < 4; ++j) for (int v = 0; v < 16; ++v) s2 += acc[j][v];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s2;
}

// Accumulating into a float32 array with hardware atomics: each workgroup adds 32 KiB tiles (128 rows
// of 64 floats, the partial dQ a 128-key workgroup would add for one query tile) into a 32 MiB array.
// MODE 0: workgroup w adds tile (37 w + it) mod T (spread); MODE 1: tile it mod T (every workgroup on
// the same tile at once); MODE 2: plain stores, spread.
template <int MODE>
__global__ __launch_bounds__(256) void k_atomic(float* dst, int T, int iters) {
  for (int it = 0; it < iters; ++it) {
    const int t = MODE == 1 ? (it % T) : ((static_cast<int>(blockIdx.x) * 37 + it) % T);
    float* base = dst + static_cast<size_t>(t) * 8192;   // t < T: inside the T * 8192 floats
#pragma unroll 4
    for (int i = threadIdx.x; i < 8192; i += 256) {
      if (MODE == 2) base[i] = 1.0f;
      else unsafeAtomicAdd(base + i, 1.0f);
    }
  }
}

#define CHECK(x)                                                                  \
  do {                                                                            \
    hipError_t e_ = (x);                                                          \
    if (e_ != hipSuccess) {                                                       \
      fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));              \
      exit(1);                                                                    \
    }                                                                             \
  } while (0)

template <typename F>
float timeit(F f) {
  hipEvent_t a, b;
  CHECK(hipEventCreate(&a));
  CHECK(hipEventCreate(&b));
  f();
  CHECK(hipDeviceSynchronize());
  CHECK(hipEventRecord(a));
  f();
  CHECK(hipEventRecord(b));
  CHECK(hipEventSynchronize(b));
  float ms;
  CHECK(hipEventElapsedTime(&ms, a, b));
  return ms;
}

int main() {
  hipDeviceProp_t pr;
  CHECK(hipGetDeviceProperties(&pr, 0));
  printf("device %s CUs %d clock %d kHz\n", pr.gcnArchName, pr.multiProcessorCount, pr.clockRate);
  const int cus = pr.multiProcessorCount;
  float* out; const int maxwg = cus * 8;
  CHECK(hipMalloc(&out, sizeof(float) * maxwg * 256));
  for (int wpc : {1, 2, 4, 8}) {   // workgroups (4 waves each) per CU
    const int g = cus * wpc;
    float ms = timeit([&] { hipLaunchKernelGGL(k_mfma, dim3(g), dim3(256), 0, 0, out, 1.0f); });
    double fl = double(g) * 4 * N * 4 * 32768.0;
    printf("mfma32x32x16 wg/CU=%d: %.3f ms %.1f TFLOP/s  cycles/mfma/SIMD(at 2.4GHz)=%.2f\n", wpc, ms, fl / ms / 1e9,
           ms * 1e-3 * 2.4e9 / (double(wpc) * N * 4));
  }
  const char* names[] = {"v_exp_f32", "v_fma_f32", "v_dot2_f32_bf16", "v_max(2)", "v_exp_f16"};
  for (int op = 0; op < 5; ++op)
    for (int wpc : {1, 2, 4}) {
      const int g = cus * wpc;
      float ms = timeit([&] {
        if (op == 0) hipLaunchKernelGGL(k_valu<0>, dim3(g), dim3(256), 0, 0, out, 0.5f);
        if (op == 1) hipLaunchKernelGGL(k_valu<1>, dim3(g), dim3(256), 0, 0, out, 0.5f);
        if (op == 2) hipLaunchKernelGGL(k_valu<2>, dim3(g), dim3(256), 0, 0, out, 0.5f);
        if (op == 3) hipLaunchKernelGGL(k_valu<3>, dim3(g), dim3(256), 0, 0, out, 0.5f);
        if (op == 4) hipLaunchKernelGGL(k_valu<4>, dim3(g), dim3(256), 0, 0, out, 0.5f);
      });
      double ops = double(g) * 4 * N * 8;   // wave-instructions
      printf("%s wg/CU=%d: %.3f ms  cycles per wave-instr per SIMD (2.4GHz) = %.2f\n", names[op], wpc, ms,
             ms * 1e-3 * 2.4e9 * cus * 4 / ops);
    }
  for (int wpc : {1, 2}) {
    const int g = cus * wpc;
    float m0 = timeit([&] { hipLaunchKernelGGL(k_mix<0>, dim3(g), dim3(256), 0, 0, out, 0.5f); });
    float m16 = timeit([&] { hipLaunchKernelGGL(k_mix<16>, dim3(g), dim3(256), 0, 0, out, 0.5f); });
    float m32 = timeit([&] { hipLaunchKernelGGL(k_mix<32>, dim3(g), dim3(256), 0, 0, out, 0.5f); });
    float m64 = timeit([&] { hipLaunchKernelGGL(k_mix<64>, dim3(g), dim3(256), 0, 0, out, 0.5f); });
    printf("mix wg/CU=%d (4 mfma + E exp per iter): E=0 %.3f ms, E=16 %.3f, E=32 %.3f, E=64 %.3f\n", wpc, m0, m16, m32, m64);
  }
  for (int op = 0; op < 2; ++op) {
    const int g = cus;   // one 8-wave workgroup per CU
    auto run = [&](int nm, int nv) {
      return timeit([&] {
        if (op == 0) hipLaunchKernelGGL(k_split<0>, dim3(g), dim3(512), 0, 0, out, 0.5f, nm, nv);
        else hipLaunchKernelGGL(k_split<1>, dim3(g), dim3(512), 0, 0, out, 0.5f, nm, nv);
      });
    };
    for (int nv : {N, 2 * N}) {
      const float tm = run(N, 0), tv = run(0, nv), tb = run(N, nv);
      printf("split %s: mfma wave %d x 4 MFMA %.3f ms; valu wave %d x 8 %s %.3f ms; both %.3f ms (sum %.3f, max %.3f)\n",
             op == 0 ? "exp" : "fma", N, tm, nv, op == 0 ? "exp" : "fma", tv, tb, tm + tv, tm > tv ? tm : tv);
    }
  }
  const char* lds_names[] = {"ds_read_b128", "2x ds_read_b64_tr_b16", "ds_read_b128 broadcast (2 addresses)"};
  for (int mode = 0; mode < 3; ++mode)
    for (int wpc : {1, 2, 4}) {   // 4, 8 or 16 waves per CU (32 KiB of LDS per workgroup)
      const int g = cus * wpc;
      const int n = 4096;
      float ms = timeit([&] {
        if (mode == 0) hipLaunchKernelGGL(k_lds<0>, dim3(g), dim3(256), 0, 0, out, n);
        else if (mode == 1) hipLaunchKernelGGL(k_lds<1>, dim3(g), dim3(256), 0, 0, out, n);
        else hipLaunchKernelGGL(k_lds<2>, dim3(g), dim3(256), 0, 0, out, n);
      });
      const double bytes = double(g) * 4 * n * 4 * 1024;   // every operand read moves 1 KiB per wave
      printf("lds %s wg/CU=%d: %.3f ms, %.1f bytes/clk/CU at 2.4 GHz\n", lds_names[mode], wpc, ms,
             bytes / (ms * 1e-3 * 2.4e9) / cus);
    }
  {
    const int g = cus, n = 512;   // one 8-wave workgroup per CU
    const char* phase_names[] = {"8-wave workgroup, free-running", "8-wave workgroup, barriers, in phase",
                                 "8-wave workgroup, barriers, ping-pong", "two 4-wave workgroups, free-running",
                                 "two 4-wave workgroups, a barrier per iteration",
                                 "two 4-wave workgroups, a barrier per iteration, A operands from LDS",
                                 "the same plus 16 KiB of direct global -> LDS copies per iteration"};
    __bf16* src;
    CHECK(hipMalloc(&src, size_t(64) << 20));
    CHECK(hipMemset(src, 0, size_t(64) << 20));
    for (int mode = 0; mode < 7; ++mode) {
      const int threads = mode >= 3 ? 256 : 512, wgs = mode >= 3 ? 2 * g : g;
      const float t = timeit([&] {
        if (mode == 0) hipLaunchKernelGGL(k_phase<0>, dim3(wgs), dim3(threads), 0, 0, out, 0.5f, n, src);
        else if (mode == 1) hipLaunchKernelGGL(k_phase<1>, dim3(wgs), dim3(threads), 0, 0, out, 0.5f, n, src);
        else if (mode == 2) hipLaunchKernelGGL(k_phase<2>, dim3(wgs), dim3(threads), 0, 0, out, 0.5f, n, src);
        else if (mode == 3) hipLaunchKernelGGL(k_phase<3>, dim3(wgs), dim3(threads), 0, 0, out, 0.5f, n, src);
        else if (mode == 4) hipLaunchKernelGGL(k_phase<4>, dim3(wgs), dim3(threads), 0, 0, out, 0.5f, n, src);
        else if (mode == 5) hipLaunchKernelGGL(k_phase<5>, dim3(wgs), dim3(threads), 0, 0, out, 0.5f, n, src);
        else hipLaunchKernelGGL(k_phase<6>, dim3(wgs), dim3(threads), 0, 0, out, 0.5f, n, src);
      });
      // MFMA work: 8 waves x n x 32 products per CU
      const double fl = double(g) * 8 * n * 32 * 32768.0;
      printf("phases %s: %.3f ms, %.1f TFLOP/s\n", phase_names[mode], t, fl / (t * 1e-3) / 1e12);
    }
    CHECK(hipFree(src));
  }
  {
    const int T = 1024, iters = 64, wgs = 2048;
    float* acc;
    CHECK(hipMalloc(&acc, size_t(T) * 8192 * 4));
    CHECK(hipMemset(acc, 0, size_t(T) * 8192 * 4));
    const char* atomic_names[] = {"fp32 atomic add, spread tiles", "fp32 atomic add, one tile at a time",
                                  "plain stores, spread tiles"};
    for (int mode = 0; mode < 3; ++mode) {
      const float t = timeit([&] {
        if (mode == 0) hipLaunchKernelGGL(k_atomic<0>, dim3(wgs), dim3(256), 0, 0, acc, T, iters);
        else if (mode == 1) hipLaunchKernelGGL(k_atomic<1>, dim3(wgs), dim3(256), 0, 0, acc, T, iters);
        else hipLaunchKernelGGL(k_atomic<2>, dim3(wgs), dim3(256), 0, 0, acc, T, iters);
      });
      printf("accumulate %s: %.3f ms, %.2f TB/s of float32 added\n", atomic_names[mode], t,
             double(wgs) * iters * 32768.0 / (t * 1e-3) / 1e12);
    }
    CHECK(hipFree(acc));
  }
  CHECK(hipFree(out));
  return 0;
}
