/*
 * ra_attn.h -- C ABI of the blockwise exact ring-attention library (libra_attn.so).
 *
 * What is computed.  Exact softmax attention, organised as ring attention:
 * each device keeps its block of queries while key/value blocks travel
 * round a ring of n devices, so that every query block meets every K/V
 * block and the whole attention map is formed ("手把手拆解RingAttention",
 * section 1 and its comparison table; section 2 for the neighbour
 * exchange).  On one GPU the ring is a loop: the query block of ring rank r
 * takes K/V block (r - s) mod n at step s.  The call mirrors the
 * ringattention(xq, xk, xv, attention_bias, segment_ids, blockwise_kwargs)
 * interface of "RingAttention核心功能全解析" (section "快速上手"), whose
 * blockwise_kwargs carry query_chunk_size, key_chunk_size and
 * causal_block_size=1 (section "分块注意力计算").
 *
 * For query i with global position p_i and key j of the same batch row and
 * head:
 *   visible(i,j) = (!causal || j / c <= p_i / c) && (segment_ids == NULL || seg[j] == seg[p_i])
 * with c = causal (the causal block size; integer division).
 *   s_ij   = scale * <q_i, k_j> + (bias ? bias[h, j mod bias_len] : 0)
 *   lse_i  = log sum_{visible j} exp(s_ij)            (natural log; -inf if none)
 *   out_i  = sum_{visible j} exp(s_ij - lse_i) v_j    (0 if none)
 * and the backward, given dout, recomputes P from lse (the recompute policy
 * "nothing_saveable" of the same section):
 *   Delta_i = <dout_i, out_i>,  dS_ij = P_ij (<dout_i, v_j> - Delta_i)
 *   dq_i = scale sum_j dS_ij k_j,  dk_j = scale sum_i dS_ij q_i,  dv_j = sum_i P_ij dout_i
 *
 * Conventions shared by every entry point.
 *  - Layout.  q, out, dout, dq: [B, Lq, H, D]; k, v, dk, dv: [B, Lk, H, D];
 *    all row-major and contiguous (the [batch, sequence, heads, head_dim]
 *    sharding layout of the wmrh.cn page, section "计算与通信重叠").
 *    lse and delta: float32 [B, H, Lq].  bias: float32 [H, bias_len].
 *    segment_ids: int32 [B, Lk], indexed by global key position.
 *  - Pointers are DEVICE pointers, 16-byte aligned; the library keeps none
 *    after it returns and the caller keeps them alive until the stream has
 *    passed the work.  stream is a hipStream_t (NULL = the null stream).
 *  - Ring.  n_ring >= 1 blocks of Lb = Lk / n_ring tokens (Lk must be a
 *    multiple of n_ring: the ring must close).  ring_rank = -1: q holds all
 *    n_ring blocks (Lq == Lk) and query block r follows its own ring order;
 *    ring_rank = r in [0, n_ring): q is block r only (Lq == Lb) and
 *    p_i = r*Lb + i.  In that mode dk/dv are the contributions of rank r's
 *    queries to every K/V block (zero where none is visible).
 *  - Chunks.  q_chunk and k_chunk are query_chunk_size / key_chunk_size:
 *    each must be >= 1 and divide Lb.  The kernels' own tiles nest inside
 *    any such chunking and masked keys contribute exact zeros, so results do
 *    not depend on the chunk sizes at all.
 *  - causal is 0 (no mask) or the causal block size c in [1, 2^30): the
 *    page's causal_block_size, where 1 turns on (token-level) causal
 *    attention.  For c > 1 the reading taken is block-granular causality:
 *    positions fall into consecutive blocks of c tokens and a key is visible
 *    when its block does not come after the query's (j / c <= p_i / c, on
 *    global positions).  c must divide the ring block length Lb.  Fully
 *    masked K/V blocks and tiles are skipped.
 *  - dtype: RA_BF16 (inputs/outputs bfloat16, float32 accumulation, P
 *    rounded to bfloat16 before the P.V product) or RA_F32 (float32
 *    throughout).  head_dim must be 64 or 128.
 *  - Inputs must be finite.
 *  - Errors.  All validation runs on the host before anything is enqueued;
 *    a non-zero return means nothing was launched, and ra_last_error()
 *    describes it.  RA_ERR_HIP reports a failed launch.  Faults during
 *    execution surface at the caller's next synchronisation.
 *  - Thread safety.  The attention entry points keep no state apart from the
 *    per-thread error string; concurrent calls on different streams are safe.
 *    The feed-forward entry points are stateless too.
 */
#ifndef RA_ATTN_H
#define RA_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ra_dtype { RA_F32 = 0, RA_BF16 = 1 } ra_dtype;

typedef enum ra_status {
  RA_OK = 0,
  RA_ERR_ARG = -1,          /* null pointer, bad causal block size, bad chunk, bad rank */
  RA_ERR_SHAPE = -2,        /* ring does not close, Lq inconsistent with ring_rank, negative size */
  RA_ERR_UNSUPPORTED = -3,  /* head_dim or dtype the kernels do not implement */
  RA_ERR_WORKSPACE = -4,    /* workspace missing or too small */
  RA_ERR_HIP = -5           /* the HIP runtime refused a launch */
} ra_status;

/* Problem description shared by all calls (48 bytes, no padding). */
typedef struct ra_shape {
  int32_t batch;      /* B >= 0 */
  int32_t heads;      /* H >= 0, with heads * head_dim < 2^24 */
  int32_t head_dim;   /* D: 64 or 128 */
  int32_t ring_rank;  /* -1: all blocks; r in [0, n_ring): one rank's query block */
  int64_t q_len;      /* Lq */
  int64_t kv_len;     /* Lk = n_ring * Lb */
  int64_t bias_len;   /* bias row length (>= 1 when bias != NULL); key j uses bias[h, j % bias_len] */
  float scale;        /* softmax scale; <= 0 selects 1/sqrt(head_dim) */
  int32_t dtype;      /* ra_dtype of q, k, v, out, dout, dq, dk, dv */
} ra_shape;

/*
 * Forward pass (steps of the ring for one query block, online-softmax merge).
 * In:  q [B,Lq,H,D], k, v [B,Lk,H,D] (dtype); bias [H,bias_len] float32 or NULL;
 *      segment_ids [B,Lk] int32 or NULL.
 * Out: out [B,Lq,H,D] (dtype, written in full); lse [B,H,Lq] float32 (natural log).
 * Allocates nothing.
 */
int ra_blockwise_attn_fwd(const void* q, const void* k, const void* v, const float* bias,
                          const int32_t* segment_ids, int32_t n_ring, int64_t q_chunk, int64_t k_chunk,
                          int32_t causal, void* out, float* lse, const ra_shape* shape, void* stream);

/* Bytes of device workspace ra_blockwise_attn_bwd needs for this shape on a ring of n_ring blocks:
 * Delta, float32 [B,H,Lq], rounded up to 256 (the two backward kernels each own the rows they
 * write, so no partial sums are needed and the size does not depend on n_ring).  Returns 0 for a
 * NULL shape, negative sizes or n_ring < 1. */
size_t ra_blockwise_attn_bwd_workspace_size(const ra_shape* shape, int32_t n_ring);

/*
 * The backward pass plus the gradient of the additive bias (NEXT-4 of the pages' attention_bias,
 * "RingAttention核心功能全解析", 快速上手; the pages define no gradient, the plain one is taken):
 * key j adds bias[h, j mod bias_len] to every query's score, so
 *   dbias[h, t] = sum over b, i and keys j with j mod bias_len = t of dS_ij   (float32, [H, bias_len])
 * with dS as above (no scale factor).  Arguments as ra_blockwise_attn_bwd, plus dbias (device,
 * 4-byte aligned); bias must be given (RA_BF16 or RA_F32).  The workspace must hold
 * ra_blockwise_attn_bwd_dbias_workspace_size(shape) bytes (Delta and per-key sums of dS).  The
 * sums run in a fixed order: the result is deterministic.
 */
int ra_blockwise_attn_bwd_dbias(const void* q, const void* k, const void* v, const float* bias,
                                const int32_t* segment_ids, int32_t n_ring, int64_t q_chunk, int64_t k_chunk,
                                int32_t causal, const void* out, const float* lse, const void* dout, void* dq,
                                void* dk, void* dv, float* dbias, void* workspace, size_t workspace_bytes,
                                const ra_shape* shape, void* stream);

/* Workspace bytes ra_blockwise_attn_bwd_dbias needs for this shape. */
size_t ra_blockwise_attn_bwd_dbias_workspace_size(const ra_shape* shape);

/*
 * Backward pass: recomputes P from lse and writes dq, dk, dv (dtype, same
 * layouts as q, k, v, written in full).  out and lse are the forward's
 * outputs for the same arguments.  Runs the three phases below in order on
 * `stream`; workspace (device, >= ra_blockwise_attn_bwd_workspace_size
 * bytes) holds Delta.
 */
int ra_blockwise_attn_bwd(const void* q, const void* k, const void* v, const float* bias,
                          const int32_t* segment_ids, int32_t n_ring, int64_t q_chunk, int64_t k_chunk,
                          int32_t causal, const void* out, const float* lse, const void* dout, void* dq,
                          void* dk, void* dv, void* workspace, size_t workspace_bytes, const ra_shape* shape,
                          void* stream);

/*
 * The backward pass for callers that cannot allocate (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): ra_blockwise_attn_bwd with no workspace argument.  Delta
 * goes to a 16 MiB array in the library's static device memory, one per GPU, held until the process
 * ends; the call itself allocates nothing and calls no allocating routine.  Limit: batch * heads *
 * q_len <= 4,194,304 (ra_blockwise_attn_bwd_noalloc_max_workspace() bytes of Delta), else
 * RA_ERR_WORKSPACE and nothing is launched.  Results are those of ra_blockwise_attn_bwd, bit for bit.
 * Every call on a GPU uses that GPU's one array: calls that overlap on one GPU (other streams or
 * threads) race and must be serialised by the caller.  Errors: as ra_blockwise_attn_bwd, whose
 * message ra_last_error() holds; errors of this wrapper itself (shape NULL, size over the limit,
 * no current device) are described by ra_noalloc_last_error().
 */
int ra_blockwise_attn_bwd_noalloc(const void* q, const void* k, const void* v, const float* bias,
                                  const int32_t* segment_ids, int32_t n_ring, int64_t q_chunk, int64_t k_chunk,
                                  int32_t causal, const void* out, const float* lse, const void* dout, void* dq,
                                  void* dk, void* dv, const ra_shape* shape, void* stream);

/* Bytes of the static scratch array ra_blockwise_attn_bwd_noalloc uses (its size limit). */
size_t ra_blockwise_attn_bwd_noalloc_max_workspace(void);

/* Description of the last error of ra_blockwise_attn_bwd_noalloc's own checks on this thread
 * ("" when the last call passed them). */
const char* ra_noalloc_last_error(void);

/* Backward phase 1: delta[b,h,i] = sum_d dout[b,i,h,d] * out[b,i,h,d] (float32 [B,H,Lq]). */
int ra_blockwise_attn_bwd_preprocess(const void* out, const void* dout, float* delta, const ra_shape* shape,
                                     void* stream);

/* Backward phase 2: dk, dv for every key, K/V tiles stationary, query blocks in the order the
 * K/V block meets them on the ring (its own rank first, then r+1, r+2, ...). */
int ra_blockwise_attn_bwd_dkdv(const void* q, const void* k, const void* v, const float* bias,
                               const int32_t* segment_ids, int32_t n_ring, int64_t q_chunk, int64_t k_chunk,
                               int32_t causal, const float* lse, const float* delta, const void* dout,
                               void* dk, void* dv, const ra_shape* shape, void* stream);

/* Backward phase 3: dq, query tiles stationary, K/V blocks in ring order (as the forward). */
int ra_blockwise_attn_bwd_dq(const void* q, const void* k, const void* v, const float* bias,
                             const int32_t* segment_ids, int32_t n_ring, int64_t q_chunk, int64_t k_chunk,
                             int32_t causal, const float* lse, const float* delta, const void* dout, void* dq,
                             const ra_shape* shape, void* stream);

/*
 * One ring step of the forward pass, for use inside a real ring where the K/V blocks arrive one
 * at a time ("手把手拆解RingAttention", section 2: each device works on the key/value block it
 * holds while that block moves on to the next device).  The queries q [B,Lq,H,D] sit at global
 * positions q_pos0 + i; the block k, v [B,Lk,H,D] (Lk == Lq: ring blocks are equal) holds the
 * keys at global positions kv_pos0 + j.  The call folds that block into the running state with
 * the online-softmax merge (the reading of the pages' "complete attention map", section 1):
 *   o_state [B,Lq,H,D] float32: unnormalised accumulator;
 *   m_state [B,H,Lq] float32: reference row maximum in log2 units (score * log2 e);
 *   l_state [B,H,Lq] float32: sum of exponentials against m_state.
 * init = 1 starts from the empty state (the incoming state is not read); otherwise the state
 * left by the previous step is read and updated in place.  The masks, bias and scale are those
 * of ra_blockwise_attn_fwd, on global positions: causal compares kv_pos0 + j with q_pos0 + i,
 * bias is read at key position kv_pos0 + j, and segment_ids [B, seg_len] (seg_len covering
 * both blocks' positions) are indexed by global position.  shape.ring_rank is ignored;
 * shape.q_len == shape.kv_len is the block length.  Blocks may come in any order; after the
 * last step ra_blockwise_attn_fwd_finalize gives out and lse.  RA_BF16 only.
 */
int ra_blockwise_attn_fwd_step(const void* q, const void* k, const void* v, const float* bias,
                               const int32_t* segment_ids, int64_t seg_len, int64_t q_pos0, int64_t kv_pos0,
                               int32_t causal, float* o_state, float* m_state, float* l_state, int32_t init,
                               const ra_shape* shape, void* stream);

/* out [B,Lq,H,D] (dtype) = o_state / l_state and lse [B,H,Lq] = natural log of l_state plus the
 * reference maximum: the forward's outputs from the state of the last ring step (rows that saw no
 * visible key: out 0, lse -inf).  shape gives B, H, D, Lq (= q_len) and the dtype of out. */
int ra_blockwise_attn_fwd_finalize(const float* o_state, const float* m_state, const float* l_state, void* out,
                                   float* lse, const ra_shape* shape, void* stream);

/* Merge of two partial attentions of the same queries over disjoint key sets (for instance two
 * halves of the ring computed separately): with lse = log(exp(lse_a) + exp(lse_b)),
 *   out_a <- exp(lse_a - lse) out_a + exp(lse_b - lse) out_b,   lse_a <- lse   (in place).
 * out_a, out_b [B,Lq,H,D] (dtype), lse_a, lse_b [B,H,Lq] float32; shape gives B, H, D, Lq and the
 * dtype.  This is the online-softmax merge rule applied to normalised partial results. */
int ra_attn_merge(void* out_a, float* lse_a, const void* out_b, const float* lse_b, const ra_shape* shape,
                  void* stream);

/*
 * One ring step of the backward pass (the recompute policy of "RingAttention核心功能全解析",
 * 快速上手: P is recomputed from the saved lse).  Positions, masks, bias and segment ids are as in
 * ra_blockwise_attn_fwd_step: queries q, dout [B,Lq,H,D] at q_pos0 + i, the K/V block k, v
 * [B,Lk,H,D] (Lk == Lq) at kv_pos0 + j.  lse [B,H,Lq] is the final lse of these queries (over
 * the whole ring) and delta [B,H,Lq] = rowsum(dout * out) (ra_blockwise_attn_bwd_preprocess).
 * With P = exp(scale * q k^T + bias - lse) on the visible pairs and dS = P * (dout v^T - delta),
 * the call adds, in float32 and without the scale factor of dq and dk:
 *   dq_acc [B,Lq,H,D] += dS k,   dk_acc [B,Lk,H,D] += dS^T q,   dv_acc [B,Lk,H,D] += P^T dout.
 * With a bias and dbias_acc != NULL (float32 [B,H,Lk], 4-byte aligned) the call also adds the
 * block's per-key sums of dS (no scale factor), the bias gradient's share of each key:
 *   dbias_acc[b,h,j] += sum_i dS_ij.
 * init_dq = 1 (init_dkv = 1) starts dq_acc (dk_acc, dv_acc, dbias_acc) at zero without reading it.
 * In a ring, dq_acc stays with the queries while dk_acc, dv_acc and dbias_acc travel with their K/V
 * block and return to its owner after the last step ("手把手拆解RingAttention", section 2).  The
 * two kernels run in order on the stream; RA_BF16 only.  dbias_acc without a bias: RA_ERR_ARG.
 */
int ra_blockwise_attn_bwd_step(const void* q, const void* k, const void* v, const float* bias,
                               const int32_t* segment_ids, int64_t seg_len, int64_t q_pos0, int64_t kv_pos0,
                               int32_t causal, const float* lse, const float* delta, const void* dout, float* dq_acc,
                               float* dk_acc, float* dv_acc, float* dbias_acc, int32_t init_dq, int32_t init_dkv,
                               const ra_shape* shape, void* stream);

/* A K/V block's share of the bias gradient from the per-key sums it carried round the ring
 * (dbias_acc of ra_blockwise_attn_bwd_step): its keys sit at global positions kv_pos0 + j, so
 *   dbias[h, t] (+)= sum over b and j with (kv_pos0 + j) mod bias_len = t of key_sums[b,h,j]
 * key_sums [B,H,Lk] float32 with Lk = shape.kv_len, dbias [H, bias_len] float32 (shape.bias_len >= 1);
 * accumulate = 1 adds to dbias (one call per block: the blocks' shares sum to the whole gradient; on
 * several devices the per-device results are summed), 0 overwrites it.  A fixed summation order:
 * deterministic.  Any dtype; kv_pos0 >= 0. */
int ra_blockwise_attn_bwd_dbias_reduce(const float* key_sums, int64_t kv_pos0, float* dbias, int32_t accumulate,
                                       const ra_shape* shape, void* stream);

/* Gradients from the ring-step sums: dq = scale * dq_acc [B,Lq,H,D], dk = scale * dk_acc and
 * dv = dv_acc [B,Lk,H,D], converted to shape.dtype (scale: shape.scale, or 1/sqrt(head_dim)). */
int ra_blockwise_attn_bwd_finalize(const float* dq_acc, const float* dk_acc, const float* dv_acc, void* dq, void* dk,
                                   void* dv, const ra_shape* shape, void* stream);

/*
 * Blockwise feed-forward ("RingAttention核心功能全解析", 快速上手: blockwise_feedforward is
 * exported next to ringattention; the pages give only its name).  The sharding example of the
 * same page builds its mesh from LLaMAConfig, so the feed-forward is LLaMA's SwiGLU, per token:
 *   out = W2 (silu(W1 x) * (W3 x)),   silu(a) = a / (1 + exp(-a)),
 * computed over chunks of `chunk` tokens so that the [tokens, d_ff] intermediate only ever
 * exists for one chunk (the result does not depend on the chunk).  bfloat16 tensors, float32
 * accumulation on the library's own MFMA products; the gate silu(g) * u is formed in the epilogue
 * of the product that makes g and u (in float32), and its derivative in the epilogue of the product
 * that makes dh.  The gated activation h, the backward's g and u and the gradients of the
 * intermediate are rounded to bfloat16 between the products.
 *   x, out, dout, dx: [tokens, d_model];  w1, w3: [d_ff, d_model];  w2: [d_model, d_ff]
 *   (row-major, a linear layer's [out, in]);  dw1, dw3, dw2: float32, same shapes as the weights.
 * d_model and d_ff are multiples of 8; chunk * d_ff < 2^31.  The workspace (device, 256-byte
 * aligned) holds ra_blockwise_ffn_workspace_size(...) bytes (backward = 1 for the backward).
 * The backward recomputes each chunk's intermediate, writes dx and overwrites dw1, dw3, dw2
 * with the sums over all tokens; the weight gradients' products are split over the chunk's
 * tokens into partial sums in the workspace, added in a fixed order (deterministic).
 */
size_t ra_blockwise_ffn_workspace_size(int64_t tokens, int32_t d_model, int32_t d_ff, int64_t chunk,
                                       int32_t backward);
int ra_blockwise_ffn_fwd(const void* x, const void* w1, const void* w3, const void* w2, void* out, int64_t tokens,
                         int32_t d_model, int32_t d_ff, int64_t chunk, void* workspace, size_t workspace_bytes,
                         void* stream);
int ra_blockwise_ffn_bwd(const void* x, const void* w1, const void* w3, const void* w2, const void* dout, void* dx,
                         float* dw1, float* dw3, float* dw2, int64_t tokens, int32_t d_model, int32_t d_ff,
                         int64_t chunk, void* workspace, size_t workspace_bytes, void* stream);

/* Description of the last error on the calling thread ("" after a success). */
const char* ra_last_error(void);

/* Library ABI version: 2. */
int32_t ra_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RA_ATTN_H */
