// Internal definitions shared by the kernels and the C-ABI layer of libra_attn.
//
// Ring schedule (the one fact every kernel shares): the query block of ring
// rank r meets K/V block (r - s) mod n at ring step s, because each device
// keeps its queries while key/value blocks move one device round the ring per
// step ("手把手拆解RingAttention", section 1; section 2 for the exchange).
// Under a causal mask K/V blocks past the query block are invisible and are
// skipped without being read; inside the diagonal block only keys up to the
// tile's last query are visited.  In the backward pass a K/V block meets
// the query blocks in the opposite direction: ranks j, j+1, ... (mod n).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ra {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

// Everything a kernel needs; filled by the C-ABI layer after validation.
struct Params {
  const void* q;
  const void* k;
  const void* v;
  const float* bias;        // [H, bias_len] or null
  const int32_t* seg;       // [B, Lk] or null
  void* out;                // [B, Lq, H, D]
  float* lse;               // [B, H, Lq]
  const void* dout;         // [B, Lq, H, D]
  const float* delta;       // [B, H, Lq]
  float* delta_out;         // preprocess output
  void* dq;
  void* dk;
  void* dv;
  int64_t Lq, Lk, Lb, bias_len;
  int32_t B, H, D, n_ring, ring_rank;
  int32_t causal;           // causal block size (1: token-level causal), 0: no causal mask
  int32_t bf16;             // 1: bfloat16 tensors, 0: float32
  float scale;              // resolved (> 0)
  // one ring step (ra_blockwise_attn_fwd_step): the keys held are global positions
  // kv_pos0 + j, the queries q_pos0 + i; segment ids are [B, seg_len] on global positions
  int64_t q_pos0, kv_pos0, seg_len;
  float* o_state;           // [B, Lq, H, D] unnormalised accumulator
  float* m_state;           // [B, H, Lq] reference maximum, log2 units
  float* l_state;           // [B, H, Lq] sum of exponentials against m_state
  int32_t step_init;        // 1: start from an empty state (the incoming one is not read)
  // one backward ring step (ra_blockwise_attn_bwd_step): unscaled float32 gradient sums in
  // caller memory, dQ for the queries held, dK / dV for the K/V block held
  float* dq_acc;            // [B, Lq, H, D]
  float* dk_acc;            // [B, Lk, H, D]
  float* dv_acc;            // [B, Lk, H, D]
  int32_t init_dq, init_dkv;   // 1: the sums start at zero (the incoming ones are not read)
  // bias gradient: per-key sums of dS over the queries, [B, H, Lk] (ra_blockwise_attn_bwd_dbias), or the
  // sums one K/V block carries round a ring, [B, H, block length] (ra_blockwise_attn_bwd_step)
  float* dbias_keys;
};

// ---------------------------------------------------------------- element access
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }

__device__ __forceinline__ int64_t row_offset(int b, int64_t row, int h, int64_t L, int H, int D) {
  return ((static_cast<int64_t>(b) * L + row) * H + h) * static_cast<int64_t>(D);
}

// ---------------------------------------------------------------- causal block size
// With causal block size c (c = 1: token-level causal attention), positions fall into blocks
// of c tokens and a key is visible to a query when the key's block does not come after the
// query's.  Positions here are relative to an origin at global position off >= 0 (so that
// rel + off >= 0 is the global position).
// The last key position a query at rel can see: the end of its block.
__device__ __forceinline__ int causal_last_key(int rel, int off, int c) {
  if (c == 1) return rel;
  const int g = rel + off;
  return (g / c + 1) * c - 1 - off;
}
// The first query position that can see a key at rel: the start of the key's block.
__device__ __forceinline__ int causal_first_query(int rel, int off, int c) {
  if (c == 1) return rel;
  const int g = rel + off;
  return (g / c) * c - off;
}

// ---------------------------------------------------------------- workgroup order
// The (batch, head) pair hb and the tile t of workgroup `id`, for HB pairs of n_t tiles each (the grid
// is HB * n_t; tile 0 of a pair is its first to run).  The dispatcher hands consecutive workgroup ids to
// the 8 XCDs in turn (XCD id % 8), and each XCD has an L2 of its own.
// - by_pair (only when HB is a multiple of 8): XCD x takes the pairs x, x + 8, x + 16, ... one after
//   the other, all tiles of a pair before the next.  The workgroups an XCD holds at once then belong to
//   one pair and stream the same K/V (or Q and dO) through its L2, and every XCD still gets pairs of
//   every batch row.
// - otherwise pairs vary fastest, so an XCD holds tiles of HB / 8 pairs at once.
// (32-bit arithmetic: the host keeps every grid below 2^31 workgroups.)
struct HeadTile {
  int hb;
  int64_t t;
};
__device__ __forceinline__ HeadTile head_tile(unsigned id, int HB, int64_t n_t, bool by_pair) {
  const unsigned nt = static_cast<unsigned>(n_t), hbs = static_cast<unsigned>(HB);
  if (by_pair && (hbs & 7u) == 0) {
    const unsigned i = id >> 3;
    return {static_cast<int>((id & 7u) + 8u * (i / nt)), static_cast<int64_t>(i % nt)};
  }
  return {static_cast<int>(id % hbs), static_cast<int64_t>(id / hbs)};
}

// ---------------------------------------------------------------- forward-direction ring walk
// Walks the K/V tiles one query tile must visit, in ring order, tile size BK.
// Start with begin(); each next() moves to the following tile and returns
// false when the walk is over.  key0 is the tile's first global key; kend is
// the end of its K/V block (keys at or past kend are padding of a ragged
// tile and must be treated as invisible).
struct RingWalk {
  // key positions fit in 32 bits (the host rejects kv_len >= 2^30), so the walk's compares
  // stay on the scalar unit
  int n, r, s;
  bool causal;
  int Lb, plast;  // plast: last global query position of the tile
  int key0, kend, kstop;
  __device__ void begin(int n_, int r_, int64_t Lb_, bool causal_, int64_t plast_) {
    n = n_; r = r_; Lb = static_cast<int>(Lb_); causal = causal_; plast = static_cast<int>(plast_);
    s = -1; key0 = 0; kend = 0; kstop = 0;
  }
  template <int BK>
  __device__ bool next() {
    key0 += BK;
    while (key0 >= kstop) {
      ++s;
      if (s >= n) return false;
      int j = r - s;
      if (j < 0) j += n;
      if (causal && j > r) continue;   // a block from the future: fully masked, skipped
      key0 = j * Lb;
      kend = key0 + Lb;
      kstop = (causal && j == r) ? (plast + 1 < kend ? plast + 1 : kend) : kend;
    }
    return true;
  }
};

// ---------------------------------------------------------------- backward-direction ring walk
// Walks the query tiles one K/V tile must meet: the K/V block j visits ranks
// j, j+1, ... (mod n).  With ring_rank >= 0 only that rank's queries exist.
// Under a causal mask ranks before j are skipped and, in rank j itself, query
// tiles that end before the K/V tile's first key are skipped.
struct QueryWalk {
  // 32-bit rows and positions (below 2^30, checked on the host): the compares stay scalar
  int n, j, s, rank_only;
  bool causal;
  int Lb, kfirst;   // kfirst: first global key of the K/V tile
  int row0, rend, rstop;   // local query rows [row0, row0+BQ) of q; rend: end of the rank's rows
  int pos_base;            // global position of local row 0 of the current rank
  int cur_rank;
  bool step;               // one ring step: one query block, positions relative to the keys held
  int step_off;            // ... its row 0's position relative to key 0 of the block held
  __device__ void begin(int n_, int j_, int64_t Lb_, bool causal_, int64_t kfirst_, int rank_only_) {
    n = n_; j = j_; Lb = static_cast<int>(Lb_); causal = causal_; kfirst = static_cast<int>(kfirst_);
    rank_only = rank_only_;
    s = -1; row0 = 0; rend = 0; rstop = 0; pos_base = 0; cur_rank = 0;
    step = false; step_off = 0;
  }
  // one ring step: rows [0, Lq) of the query block, at positions off + row relative to the keys
  __device__ void begin_step(int64_t Lq_, bool causal_, int64_t kfirst_, int64_t off) {
    begin(1, 0, Lq_, causal_, kfirst_, 0);
    step = true;
    step_off = static_cast<int>(off);
  }
  template <int BQ>
  __device__ bool next() {
    row0 += BQ;
    while (row0 >= rstop) {
      ++s;
      if (s >= n) return false;
      int r = j + s;
      if (r >= n) r -= n;
      if (rank_only >= 0 && r != rank_only) continue;
      if (!step && causal && r < j) continue;   // queries before the block see none of it
      cur_rank = r;
      const int local0 = rank_only >= 0 ? 0 : r * Lb;   // first local row of rank r
      pos_base = step ? step_off : r * Lb - local0;     // global pos = local row + pos_base
      rend = local0 + Lb;
      row0 = local0;
      if (causal && (step || r == j)) {
        // skip whole query tiles that end before kfirst: first row with pos >= kfirst
        const int first_row = kfirst - pos_base;
        if (first_row > row0) row0 += ((first_row - row0) / BQ) * BQ;
      }
      rstop = rend;
    }
    return true;
  }
};

// ---------------------------------------------------------------- launchers (validated Params only)
hipError_t launch_fwd_mfma(const Params& p, hipStream_t st);
hipError_t launch_fwd_step_mfma(const Params& p, hipStream_t st);
hipError_t launch_fwd_finalize(const Params& p, hipStream_t st);
hipError_t launch_merge(const Params& p, const void* out_b, const float* lse_b, hipStream_t st);
hipError_t launch_fwd_f32(const Params& p, hipStream_t st);
hipError_t launch_bwd_preprocess(const Params& p, hipStream_t st);
hipError_t launch_bwd_dkdv_f32(const Params& p, hipStream_t st);
hipError_t launch_bwd_dq_f32(const Params& p, hipStream_t st);
hipError_t launch_bwd_dkdv_mfma(const Params& p, hipStream_t st);
hipError_t launch_bwd_dq_mfma(const Params& p, hipStream_t st);
hipError_t launch_bwd_dkdv_step_mfma(const Params& p, hipStream_t st);
hipError_t launch_bwd_dq_step_mfma(const Params& p, hipStream_t st);
hipError_t launch_grad_finalize(const float* acc, float factor, void* out, int64_t elems, bool bf16, hipStream_t st);
// blockwise feed-forward (ffn.hip): workspace regions (byte offsets) for one chunk of tokens
struct FfnWorkspace {
  size_t w13, gu, h, dh, dgdu, dw13, bytes;
};
FfnWorkspace ffn_workspace(int64_t tokens, int d_model, int d_ff, int64_t chunk, bool backward);
hipError_t ffn_forward(const __bf16* x, const __bf16* w1, const __bf16* w3, const __bf16* w2, __bf16* out,
                       int64_t tokens, int d, int f, int64_t chunk, char* ws, hipStream_t st);
hipError_t ffn_backward(const __bf16* x, const __bf16* w1, const __bf16* w3, const __bf16* w2, const __bf16* dout,
                        __bf16* dx, float* dw1, float* dw3, float* dw2, int64_t tokens, int d, int f, int64_t chunk,
                        char* ws, hipStream_t st);
hipError_t launch_bias_grad(const float* key_sums, float* dbias, int B, int H, int64_t Lk, int64_t bias_len,
                            hipStream_t st);
hipError_t launch_bias_grad_block(const float* key_sums, float* dbias, int B, int H, int64_t Lb, int64_t kv_pos0,
                                  int64_t bias_len, int accumulate, hipStream_t st);
// p[0 .. n) = 0 with a kernel (no memset node when the caller captures a graph)
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t st);

}  // namespace ra
