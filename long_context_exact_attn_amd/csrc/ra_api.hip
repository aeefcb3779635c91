// C ABI of libra_attn: argument validation on the host, then kernel dispatch.
// The operations are defined in include/ra_attn.h.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include <rocprofiler-sdk-roctx/roctx.h>

#include "../../include/ra_attn.h"
#include "ra_common.cuh"

namespace {

thread_local std::string g_last_error;

constexpr int64_t kMaxPos = int64_t(1) << 30;   // token positions are 32-bit in the kernels

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return RA_OK;
}

#define RA_TRY(x)              \
  do {                         \
    const int rc_ = (x);       \
    if (rc_ != RA_OK) return rc_; \
  } while (0)

// One roctx range per call of an entry point, from entry to return: it spans the validation and the
// enqueue on the host, not the kernels' run.  Under a profiler's marker trace each ring step (one
// _fwd_step or _bwd_step call) and each whole-ring call shows as one named range beside the kernels
// it launched.  Names use the scalar arguments only, which are valid before validation.
class Range {
 public:
  explicit Range(const char* fmt, ...) {
    char buf[160];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    roctxRangePushA(buf);
  }
  ~Range() { roctxRangePop(); }
  Range(const Range&) = delete;
  Range& operator=(const Range&) = delete;
};

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Checked {
  ra::Params p;
  int64_t q_elems, kv_elems, rows;   // rows = B*H*Lq
};

// dtype, head_dim and sign checks.
int check_dims(const ra_shape* s) {
  if (!s) return fail(RA_ERR_ARG, "shape is NULL");
  if (s->dtype != RA_F32 && s->dtype != RA_BF16) return fail(RA_ERR_UNSUPPORTED, "dtype %d is not RA_F32 or RA_BF16", s->dtype);
  if (s->head_dim != 64 && s->head_dim != 128)
    return fail(RA_ERR_UNSUPPORTED, "head_dim %d is not supported (64 or 128)", s->head_dim);
  if (s->batch < 0 || s->heads < 0 || s->q_len < 0 || s->kv_len < 0)
    return fail(RA_ERR_SHAPE, "negative size (batch %d, heads %d, q_len %lld, kv_len %lld)", s->batch, s->heads,
                (long long)s->q_len, (long long)s->kv_len);
  return RA_OK;
}

// Shape-level checks shared by every entry point that walks the ring.
int check_shape(const ra_shape* s, int32_t n_ring, Checked* c) {
  RA_TRY(check_dims(s));
  if (n_ring < 1) return fail(RA_ERR_ARG, "n_ring must be >= 1 (got %d)", n_ring);
  if (s->kv_len % n_ring != 0)
    return fail(RA_ERR_SHAPE, "ring does not close: kv_len %lld is not a multiple of n_ring %d", (long long)s->kv_len,
                n_ring);
  const int64_t Lb = s->kv_len / n_ring;
  if (s->ring_rank < -1 || s->ring_rank >= n_ring)
    return fail(RA_ERR_ARG, "ring_rank %d outside [-1, %d)", s->ring_rank, n_ring);
  if (s->ring_rank < 0 && s->q_len != s->kv_len)
    return fail(RA_ERR_SHAPE, "ring_rank -1 needs q_len == kv_len (got %lld and %lld)", (long long)s->q_len,
                (long long)s->kv_len);
  if (s->ring_rank >= 0 && s->q_len != Lb)
    return fail(RA_ERR_SHAPE, "ring_rank %d needs q_len == kv_len / n_ring = %lld (got %lld)", s->ring_rank,
                (long long)Lb, (long long)s->q_len);
  if (std::isnan(s->scale)) return fail(RA_ERR_ARG, "scale is NaN");
  const int64_t HB = static_cast<int64_t>(s->batch) * s->heads;
  if (HB > (int64_t(1) << 30)) return fail(RA_ERR_SHAPE, "batch*heads too large");
  // token positions are 32-bit inside the kernels
  if (s->kv_len >= kMaxPos || s->q_len >= kMaxPos)
    return fail(RA_ERR_SHAPE, "sequence lengths must be below 2^30 (q_len %lld, kv_len %lld)", (long long)s->q_len,
                (long long)s->kv_len);
  // the kernels address the rows of one tile (at most 128 rows) with 32-bit element offsets and
  // 32-bit unsigned byte offsets
  if (static_cast<int64_t>(s->heads) * s->head_dim * 128 >= (int64_t(1) << 31))
    return fail(RA_ERR_SHAPE, "heads*head_dim too large (%lld)", (long long)s->heads * s->head_dim);
  ra::Params& p = c->p;
  p = ra::Params{};
  p.Lq = s->q_len;
  p.Lk = s->kv_len;
  p.seg_len = s->kv_len;
  p.Lb = Lb;
  p.bias_len = s->bias_len;
  p.B = s->batch;
  p.H = s->heads;
  p.D = s->head_dim;
  p.n_ring = n_ring;
  p.ring_rank = s->ring_rank;
  p.bf16 = s->dtype == RA_BF16;
  p.scale = s->scale > 0.f ? s->scale : 1.0f / std::sqrt(static_cast<float>(s->head_dim));
  c->q_elems = HB * s->q_len * s->head_dim;
  c->kv_elems = HB * s->kv_len * s->head_dim;
  c->rows = HB * s->q_len;
  // every grid used is at most (query or key tiles of 64) x B x H workgroups
  const int64_t tiles = (Lb + 63) / 64 * (s->ring_rank < 0 ? n_ring : 1);
  const int64_t ktiles = (Lb + 63) / 64 * n_ring;
  if ((tiles > ktiles ? tiles : ktiles) * HB > 0x7fffffffLL) return fail(RA_ERR_SHAPE, "problem too large for one launch");
  return RA_OK;
}

int check_mask_args(const ra_shape* s, const float* bias, int64_t q_chunk, int64_t k_chunk, int32_t causal,
                    Checked* c) {
  const int64_t Lb = c->p.Lb;
  // causal = 0: no mask; causal = c >= 1: causal block size (1: token-level causal attention)
  if (causal < 0 || causal >= kMaxPos)
    return fail(RA_ERR_ARG, "causal must be 0 or a causal block size in [1, 2^30) (got %d)", causal);
  if (causal > 1 && Lb > 0 && Lb % causal != 0)
    return fail(RA_ERR_ARG, "causal block size %d must divide the ring block length %lld", causal, (long long)Lb);
  if (q_chunk < 1 || k_chunk < 1) return fail(RA_ERR_ARG, "q_chunk and k_chunk must be >= 1");
  if (Lb > 0 && (Lb % q_chunk != 0 || Lb % k_chunk != 0))
    return fail(RA_ERR_ARG, "q_chunk %lld and k_chunk %lld must divide the ring block length %lld",
                (long long)q_chunk, (long long)k_chunk, (long long)Lb);
  if (bias && (s->bias_len < 1 || s->bias_len >= kMaxPos))
    return fail(RA_ERR_ARG, "bias given with bias_len %lld (must be in [1, 2^30))", (long long)s->bias_len);
  c->p.causal = causal;
  if (!bias) c->p.bias_len = 1;
  return RA_OK;
}

int need_ptr(const void* ptr, int64_t elems, const char* name, size_t align) {
  if (elems == 0) return RA_OK;
  if (!ptr) return fail(RA_ERR_ARG, "%s is NULL", name);
  if (!aligned(ptr, align)) return fail(RA_ERR_ARG, "%s is not %zu-byte aligned", name, align);
  return RA_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(RA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

int check_inputs(const Checked& c, const void* q, const void* k, const void* v, const float* bias,
                 const int32_t* seg, const ra_shape* s) {
  RA_TRY(need_ptr(q, c.q_elems, "q", 16));
  RA_TRY(need_ptr(k, c.kv_elems, "k", 16));
  RA_TRY(need_ptr(v, c.kv_elems, "v", 16));
  if (bias && !aligned(bias, 4)) return fail(RA_ERR_ARG, "bias is not 4-byte aligned");
  if (seg && !aligned(seg, 4)) return fail(RA_ERR_ARG, "segment_ids is not 4-byte aligned");
  (void)s;
  return RA_OK;
}

size_t workspace_bytes(const Checked& c) {
  const size_t b = static_cast<size_t>(c.rows) * sizeof(float);
  return (b + 255) / 256 * 256;
}

// bfloat16 runs on the bf16 MFMA kernels; float32 keeps float32 products throughout (float32 MFMA)
int do_bwd_dkdv(const Checked& c, hipStream_t st) {
  return hip_status(c.p.bf16 ? ra::launch_bwd_dkdv_mfma(c.p, st) : ra::launch_bwd_dkdv_f32(c.p, st),
                    "dK/dV launch");
}

int do_bwd_dq(const Checked& c, hipStream_t st) {
  return hip_status(c.p.bf16 ? ra::launch_bwd_dq_mfma(c.p, st) : ra::launch_bwd_dq_f32(c.p, st), "dQ launch");
}

}  // namespace

extern "C" {

int32_t ra_abi_version(void) { return 2; }

static int ffn_check(int64_t tokens, int32_t d_model, int32_t d_ff, int64_t chunk) {
  if (tokens < 0 || tokens >= kMaxPos) return fail(RA_ERR_SHAPE, "tokens must be in [0, 2^30) (got %lld)", (long long)tokens);
  if (d_model < 8 || d_ff < 8 || d_model % 8 || d_ff % 8 || d_model > 65536 || d_ff > 262144)
    return fail(RA_ERR_SHAPE, "d_model and d_ff must be multiples of 8 in [8, 65536] / [8, 262144] (got %d, %d)",
                d_model, d_ff);
  if (chunk < 1) return fail(RA_ERR_ARG, "chunk must be >= 1 (got %lld)", (long long)chunk);
  const int64_t c = tokens < chunk ? tokens : chunk;
  if (static_cast<int64_t>(d_ff) * c >= (int64_t(1) << 31))
    return fail(RA_ERR_SHAPE, "chunk * d_ff must stay below 2^31 (chunk %lld, d_ff %d)", (long long)c, d_ff);
  return RA_OK;
}

size_t ra_blockwise_ffn_workspace_size(int64_t tokens, int32_t d_model, int32_t d_ff, int64_t chunk, int32_t backward) {
  if (tokens < 0 || d_model < 1 || d_ff < 1 || chunk < 1) return 0;
  return ra::ffn_workspace(tokens, d_model, d_ff, chunk, backward != 0).bytes;
}

int ra_blockwise_ffn_fwd(const void* x, const void* w1, const void* w3, const void* w2, void* out, int64_t tokens,
                         int32_t d_model, int32_t d_ff, int64_t chunk, void* workspace, size_t workspace_bytes,
                         void* stream) {
  Range range("ra_blockwise_ffn_fwd tokens=%lld chunk=%lld", (long long)tokens, (long long)chunk);
  RA_TRY(ffn_check(tokens, d_model, d_ff, chunk));
  const int64_t xe = tokens * d_model, we = static_cast<int64_t>(d_ff) * d_model;
  RA_TRY(need_ptr(x, xe, "x", 16));
  RA_TRY(need_ptr(out, xe, "out", 16));
  RA_TRY(need_ptr(w1, we, "w1", 16));
  RA_TRY(need_ptr(w3, we, "w3", 16));
  RA_TRY(need_ptr(w2, we, "w2", 16));
  if (tokens == 0) return ok();
  const size_t need = ra::ffn_workspace(tokens, d_model, d_ff, chunk, false).bytes;
  if (!workspace || workspace_bytes < need)
    return fail(RA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given%s", need, workspace_bytes,
                workspace ? "" : " (NULL)");
  if (!aligned(workspace, 256)) return fail(RA_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  return hip_status(ra::ffn_forward(static_cast<const __bf16*>(x), static_cast<const __bf16*>(w1),
                                    static_cast<const __bf16*>(w3), static_cast<const __bf16*>(w2),
                                    static_cast<__bf16*>(out), tokens, d_model, d_ff, chunk,
                                    static_cast<char*>(workspace), static_cast<hipStream_t>(stream)),
                    "feed-forward launch");
}

int ra_blockwise_ffn_bwd(const void* x, const void* w1, const void* w3, const void* w2, const void* dout, void* dx,
                         float* dw1, float* dw3, float* dw2, int64_t tokens, int32_t d_model, int32_t d_ff,
                         int64_t chunk, void* workspace, size_t workspace_bytes, void* stream) {
  Range range("ra_blockwise_ffn_bwd tokens=%lld chunk=%lld", (long long)tokens, (long long)chunk);
  RA_TRY(ffn_check(tokens, d_model, d_ff, chunk));
  const int64_t xe = tokens * d_model, we = static_cast<int64_t>(d_ff) * d_model;
  RA_TRY(need_ptr(x, xe, "x", 16));
  RA_TRY(need_ptr(dout, xe, "dout", 16));
  RA_TRY(need_ptr(dx, xe, "dx", 16));
  RA_TRY(need_ptr(w1, we, "w1", 16));
  RA_TRY(need_ptr(w3, we, "w3", 16));
  RA_TRY(need_ptr(w2, we, "w2", 16));
  RA_TRY(need_ptr(dw1, we, "dw1", 16));
  RA_TRY(need_ptr(dw3, we, "dw3", 16));
  RA_TRY(need_ptr(dw2, we, "dw2", 16));
  const size_t need = tokens ? ra::ffn_workspace(tokens, d_model, d_ff, chunk, true).bytes : 0;
  if (need && (!workspace || workspace_bytes < need))
    return fail(RA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given%s", need, workspace_bytes,
                workspace ? "" : " (NULL)");
  if (need && !aligned(workspace, 256)) return fail(RA_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  return hip_status(ra::ffn_backward(static_cast<const __bf16*>(x), static_cast<const __bf16*>(w1),
                                     static_cast<const __bf16*>(w3), static_cast<const __bf16*>(w2),
                                     static_cast<const __bf16*>(dout), static_cast<__bf16*>(dx), dw1, dw3, dw2,
                                     tokens, d_model, d_ff, chunk, static_cast<char*>(workspace),
                                     static_cast<hipStream_t>(stream)),
                    "feed-forward backward launch");
}

const char* ra_last_error(void) { return g_last_error.c_str(); }

int ra_blockwise_attn_fwd(const void* q, const void* k, const void* v, const float* bias,
                          const int32_t* segment_ids, int32_t n_ring, int64_t q_chunk, int64_t k_chunk,
                          int32_t causal, void* out, float* lse, const ra_shape* shape, void* stream) {
  Range range("ra_blockwise_attn_fwd n_ring=%d causal=%d", n_ring, causal);
  Checked c;
  RA_TRY(check_shape(shape, n_ring, &c));
  RA_TRY(check_mask_args(shape, bias, q_chunk, k_chunk, causal, &c));
  RA_TRY(check_inputs(c, q, k, v, bias, segment_ids, shape));
  RA_TRY(need_ptr(out, c.q_elems, "out", 16));
  RA_TRY(need_ptr(lse, c.rows, "lse", 4));
  if (c.rows == 0) return ok();
  c.p.q = q;
  c.p.k = k;
  c.p.v = v;
  c.p.bias = bias;
  c.p.seg = segment_ids;
  c.p.out = out;
  c.p.lse = lse;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (c.p.bf16) return hip_status(ra::launch_fwd_mfma(c.p, st), "forward launch");
  return hip_status(ra::launch_fwd_f32(c.p, st), "forward launch");
}

size_t ra_blockwise_attn_bwd_workspace_size(const ra_shape* shape, int32_t n_ring) {
  if (!shape || shape->batch < 0 || shape->heads < 0 || shape->q_len < 0 || n_ring < 1) return 0;
  const size_t rows = static_cast<size_t>(shape->batch) * shape->heads * shape->q_len;
  return (rows * sizeof(float) + 255) / 256 * 256;
}

size_t ra_blockwise_attn_bwd_dbias_workspace_size(const ra_shape* shape) {
  if (!shape || shape->batch < 0 || shape->heads < 0 || shape->q_len < 0 || shape->kv_len < 0) return 0;
  return ra_blockwise_attn_bwd_workspace_size(shape, 1) +
         static_cast<size_t>(shape->batch) * shape->heads * shape->kv_len * sizeof(float);
}

int ra_blockwise_attn_bwd_preprocess(const void* out, const void* dout, float* delta, const ra_shape* shape,
                                     void* stream) {
  Range range("ra_blockwise_attn_bwd_preprocess");
  RA_TRY(check_dims(shape));
  Checked c;
  c.p = ra::Params{};
  c.p.B = shape->batch;
  c.p.H = shape->heads;
  c.p.D = shape->head_dim;
  c.p.Lq = shape->q_len;
  c.p.bf16 = shape->dtype == RA_BF16;
  c.rows = static_cast<int64_t>(shape->batch) * shape->heads * shape->q_len;
  c.q_elems = c.rows * shape->head_dim;
  if ((c.rows + 255) / 256 > 0x7fffffffLL) return fail(RA_ERR_SHAPE, "problem too large for one launch");
  RA_TRY(need_ptr(out, c.q_elems, "out", 16));
  RA_TRY(need_ptr(dout, c.q_elems, "dout", 16));
  RA_TRY(need_ptr(delta, c.rows, "delta", 4));
  if (c.rows == 0) return ok();
  c.p.out = const_cast<void*>(out);
  c.p.dout = dout;
  c.p.delta_out = delta;
  return hip_status(ra::launch_bwd_preprocess(c.p, static_cast<hipStream_t>(stream)), "preprocess launch");
}

static int bwd_common(const void* q, const void* k, const void* v, const float* bias, const int32_t* seg,
                      int32_t n_ring, int64_t q_chunk, int64_t k_chunk, int32_t causal, const float* lse,
                      const void* dout, const ra_shape* shape, Checked* c) {
  RA_TRY(check_shape(shape, n_ring, c));
  RA_TRY(check_mask_args(shape, bias, q_chunk, k_chunk, causal, c));
  RA_TRY(check_inputs(*c, q, k, v, bias, seg, shape));
  RA_TRY(need_ptr(lse, c->rows, "lse", 4));
  RA_TRY(need_ptr(dout, c->q_elems, "dout", 16));
  c->p.q = q;
  c->p.k = k;
  c->p.v = v;
  c->p.bias = bias;
  c->p.seg = seg;
  c->p.lse = const_cast<float*>(lse);
  c->p.dout = dout;
  return RA_OK;
}

int ra_blockwise_attn_bwd_dkdv(const void* q, const void* k, const void* v, const float* bias,
                               const int32_t* segment_ids, int32_t n_ring, int64_t q_chunk, int64_t k_chunk,
                               int32_t causal, const float* lse, const float* delta, const void* dout,
                               void* dk, void* dv, const ra_shape* shape, void* stream) {
  Range range("ra_blockwise_attn_bwd_dkdv n_ring=%d causal=%d", n_ring, causal);
  Checked c;
  RA_TRY(bwd_common(q, k, v, bias, segment_ids, n_ring, q_chunk, k_chunk, causal, lse, dout, shape, &c));
  RA_TRY(need_ptr(delta, c.rows, "delta", 4));
  RA_TRY(need_ptr(dk, c.kv_elems, "dk", 16));
  RA_TRY(need_ptr(dv, c.kv_elems, "dv", 16));
  if (c.kv_elems == 0) return ok();
  c.p.delta = delta;
  c.p.dk = dk;
  c.p.dv = dv;
  return do_bwd_dkdv(c, static_cast<hipStream_t>(stream));
}

int ra_blockwise_attn_bwd_dq(const void* q, const void* k, const void* v, const float* bias,
                             const int32_t* segment_ids, int32_t n_ring, int64_t q_chunk, int64_t k_chunk,
                             int32_t causal, const float* lse, const float* delta, const void* dout, void* dq,
                             const ra_shape* shape, void* stream) {
  Range range("ra_blockwise_attn_bwd_dq n_ring=%d causal=%d", n_ring, causal);
  Checked c;
  RA_TRY(bwd_common(q, k, v, bias, segment_ids, n_ring, q_chunk, k_chunk, causal, lse, dout, shape, &c));
  RA_TRY(need_ptr(delta, c.rows, "delta", 4));
  RA_TRY(need_ptr(dq, c.q_elems, "dq", 16));
  if (c.rows == 0) return ok();
  c.p.delta = delta;
  c.p.dq = dq;
  return do_bwd_dq(c, static_cast<hipStream_t>(stream));
}

// The whole backward: Delta into the workspace, then dK/dV, then dQ; with dbias, the dK/dV kernel
// also leaves per-key sums of dS in the workspace, reduced into dbias afterwards.
static int bwd_full(const void* q, const void* k, const void* v, const float* bias, const int32_t* segment_ids,
                    int32_t n_ring, int64_t q_chunk, int64_t k_chunk, int32_t causal, const void* out,
                    const float* lse, const void* dout, void* dq, void* dk, void* dv, float* dbias, void* workspace,
                    size_t workspace_bytes_given, const ra_shape* shape, void* stream) {
  Checked c;
  RA_TRY(bwd_common(q, k, v, bias, segment_ids, n_ring, q_chunk, k_chunk, causal, lse, dout, shape, &c));
  RA_TRY(need_ptr(out, c.q_elems, "out", 16));
  RA_TRY(need_ptr(dq, c.q_elems, "dq", 16));
  RA_TRY(need_ptr(dk, c.kv_elems, "dk", 16));
  RA_TRY(need_ptr(dv, c.kv_elems, "dv", 16));
  const size_t delta_bytes = workspace_bytes(c);
  size_t need = delta_bytes;
  if (dbias) {
    if (!bias) return fail(RA_ERR_ARG, "dbias needs a bias");
    RA_TRY(need_ptr(dbias, static_cast<int64_t>(shape->heads) * shape->bias_len, "dbias", 4));
    need += static_cast<size_t>(shape->batch) * shape->heads * shape->kv_len * sizeof(float);
  }
  if (need > 0 && (!workspace || workspace_bytes_given < need))
    return fail(RA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given%s", need, workspace_bytes_given,
                workspace ? "" : " (NULL)");
  if (workspace && !aligned(workspace, 4)) return fail(RA_ERR_WORKSPACE, "workspace is not 4-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (c.kv_elems == 0 && c.q_elems == 0) {
    // no pair at all: the bias gradient is zero
    if (dbias)
      RA_TRY(hip_status(ra::launch_fill_zero(dbias, static_cast<int64_t>(shape->heads) * shape->bias_len, st),
                        "dbias clear"));
    return ok();
  }
  c.p.out = const_cast<void*>(out);
  c.p.delta_out = static_cast<float*>(workspace);
  c.p.delta = static_cast<const float*>(workspace);
  c.p.dq = dq;
  c.p.dk = dk;
  c.p.dv = dv;
  c.p.dbias_keys = dbias ? reinterpret_cast<float*>(static_cast<char*>(workspace) + delta_bytes) : nullptr;
  if (c.rows > 0) RA_TRY(hip_status(ra::launch_bwd_preprocess(c.p, st), "preprocess launch"));
  if (c.kv_elems > 0) RA_TRY(do_bwd_dkdv(c, st));
  if (c.rows > 0) RA_TRY(do_bwd_dq(c, st));
  if (dbias) {
    if (c.kv_elems == 0 || c.rows == 0) {
      // nothing visible: dbias is zero (the key sums were not written)
      RA_TRY(hip_status(ra::launch_fill_zero(dbias, static_cast<int64_t>(shape->heads) * shape->bias_len, st),
                        "dbias clear"));
    } else {
      RA_TRY(hip_status(ra::launch_bias_grad(c.p.dbias_keys, dbias, shape->batch, shape->heads, shape->kv_len,
                                             shape->bias_len, st),
                        "dbias launch"));
    }
  }
  return ok();
}

int ra_blockwise_attn_bwd(const void* q, const void* k, const void* v, const float* bias,
                          const int32_t* segment_ids, int32_t n_ring, int64_t q_chunk, int64_t k_chunk,
                          int32_t causal, const void* out, const float* lse, const void* dout, void* dq,
                          void* dk, void* dv, void* workspace, size_t workspace_bytes_given,
                          const ra_shape* shape, void* stream) {
  Range range("ra_blockwise_attn_bwd n_ring=%d causal=%d", n_ring, causal);
  return bwd_full(q, k, v, bias, segment_ids, n_ring, q_chunk, k_chunk, causal, out, lse, dout, dq, dk, dv, nullptr,
                  workspace, workspace_bytes_given, shape, stream);
}

int ra_blockwise_attn_bwd_dbias(const void* q, const void* k, const void* v, const float* bias,
                                const int32_t* segment_ids, int32_t n_ring, int64_t q_chunk, int64_t k_chunk,
                                int32_t causal, const void* out, const float* lse, const void* dout, void* dq,
                                void* dk, void* dv, float* dbias, void* workspace, size_t workspace_bytes_given,
                                const ra_shape* shape, void* stream) {
  Range range("ra_blockwise_attn_bwd_dbias n_ring=%d causal=%d", n_ring, causal);
  if (!dbias) return fail(RA_ERR_ARG, "dbias is NULL");
  return bwd_full(q, k, v, bias, segment_ids, n_ring, q_chunk, k_chunk, causal, out, lse, dout, dq, dk, dv, dbias,
                  workspace, workspace_bytes_given, shape, stream);
}

int ra_blockwise_attn_fwd_step(const void* q, const void* k, const void* v, const float* bias,
                               const int32_t* segment_ids, int64_t seg_len, int64_t q_pos0, int64_t kv_pos0,
                               int32_t causal, float* o_state, float* m_state, float* l_state, int32_t init,
                               const ra_shape* shape, void* stream) {
  Range range("ring step fwd q_pos0=%lld kv_pos0=%lld", (long long)q_pos0, (long long)kv_pos0);
  RA_TRY(check_dims(shape));
  if (shape->dtype != RA_BF16) return fail(RA_ERR_UNSUPPORTED, "ring steps are implemented for RA_BF16 only");
  if (shape->q_len != shape->kv_len)
    return fail(RA_ERR_SHAPE, "a ring step needs equal query and key blocks (q_len %lld, kv_len %lld)",
                (long long)shape->q_len, (long long)shape->kv_len);
  if (q_pos0 < 0 || kv_pos0 < 0) return fail(RA_ERR_ARG, "q_pos0 and kv_pos0 must be >= 0");
  if (q_pos0 + shape->q_len >= kMaxPos || kv_pos0 + shape->kv_len >= kMaxPos)
    return fail(RA_ERR_SHAPE, "global positions must stay below 2^30");
  if (init != 0 && init != 1) return fail(RA_ERR_ARG, "init must be 0 or 1 (got %d)", init);
  ra_shape blk = *shape;
  blk.ring_rank = 0;   // one block: the walk visits the keys held, causal on the global positions below
  Checked c;
  RA_TRY(check_shape(&blk, 1, &c));
  RA_TRY(check_mask_args(&blk, bias, 1, 1, causal, &c));
  RA_TRY(check_inputs(c, q, k, v, bias, segment_ids, &blk));
  if (segment_ids) {
    const int64_t need = (q_pos0 > kv_pos0 ? q_pos0 : kv_pos0) + shape->q_len;
    if (seg_len < need)
      return fail(RA_ERR_SHAPE, "segment_ids rows of %lld positions do not cover position %lld", (long long)seg_len,
                  (long long)(need - 1));
  }
  RA_TRY(need_ptr(o_state, c.q_elems, "o_state", 16));
  RA_TRY(need_ptr(m_state, c.rows, "m_state", 4));
  RA_TRY(need_ptr(l_state, c.rows, "l_state", 4));
  if (c.rows == 0) return ok();
  c.p.q = q;
  c.p.k = k;
  c.p.v = v;
  c.p.bias = bias;
  c.p.seg = segment_ids;
  c.p.seg_len = segment_ids ? seg_len : blk.kv_len;
  c.p.q_pos0 = q_pos0;
  c.p.kv_pos0 = kv_pos0;
  c.p.o_state = o_state;
  c.p.m_state = m_state;
  c.p.l_state = l_state;
  c.p.step_init = init;
  return hip_status(ra::launch_fwd_step_mfma(c.p, static_cast<hipStream_t>(stream)), "ring step launch");
}

int ra_blockwise_attn_bwd_step(const void* q, const void* k, const void* v, const float* bias,
                               const int32_t* segment_ids, int64_t seg_len, int64_t q_pos0, int64_t kv_pos0,
                               int32_t causal, const float* lse, const float* delta, const void* dout, float* dq_acc,
                               float* dk_acc, float* dv_acc, float* dbias_acc, int32_t init_dq, int32_t init_dkv,
                               const ra_shape* shape, void* stream) {
  Range range("ring step bwd q_pos0=%lld kv_pos0=%lld", (long long)q_pos0, (long long)kv_pos0);
  RA_TRY(check_dims(shape));
  if (shape->dtype != RA_BF16) return fail(RA_ERR_UNSUPPORTED, "ring steps are implemented for RA_BF16 only");
  if (shape->q_len != shape->kv_len)
    return fail(RA_ERR_SHAPE, "a ring step needs equal query and key blocks (q_len %lld, kv_len %lld)",
                (long long)shape->q_len, (long long)shape->kv_len);
  if (q_pos0 < 0 || kv_pos0 < 0) return fail(RA_ERR_ARG, "q_pos0 and kv_pos0 must be >= 0");
  if (q_pos0 + shape->q_len >= kMaxPos || kv_pos0 + shape->kv_len >= kMaxPos)
    return fail(RA_ERR_SHAPE, "global positions must stay below 2^30");
  if ((init_dq != 0 && init_dq != 1) || (init_dkv != 0 && init_dkv != 1))
    return fail(RA_ERR_ARG, "init_dq and init_dkv must be 0 or 1 (got %d, %d)", init_dq, init_dkv);
  ra_shape blk = *shape;
  blk.ring_rank = 0;   // one block each of queries and keys, causal on the global positions below
  Checked c;
  RA_TRY(check_shape(&blk, 1, &c));
  RA_TRY(check_mask_args(&blk, bias, 1, 1, causal, &c));
  RA_TRY(check_inputs(c, q, k, v, bias, segment_ids, &blk));
  if (segment_ids) {
    const int64_t need = (q_pos0 > kv_pos0 ? q_pos0 : kv_pos0) + shape->q_len;
    if (seg_len < need)
      return fail(RA_ERR_SHAPE, "segment_ids rows of %lld positions do not cover position %lld", (long long)seg_len,
                  (long long)(need - 1));
  }
  RA_TRY(need_ptr(lse, c.rows, "lse", 4));
  RA_TRY(need_ptr(delta, c.rows, "delta", 4));
  RA_TRY(need_ptr(dout, c.q_elems, "dout", 16));
  RA_TRY(need_ptr(dq_acc, c.q_elems, "dq_acc", 16));
  RA_TRY(need_ptr(dk_acc, c.kv_elems, "dk_acc", 16));
  RA_TRY(need_ptr(dv_acc, c.kv_elems, "dv_acc", 16));
  if (dbias_acc) {
    if (!bias) return fail(RA_ERR_ARG, "dbias_acc needs a bias");
    RA_TRY(need_ptr(dbias_acc, static_cast<int64_t>(shape->batch) * shape->heads * shape->kv_len, "dbias_acc", 4));
  }
  if (c.rows == 0) return ok();
  c.p.q = q;
  c.p.k = k;
  c.p.v = v;
  c.p.bias = bias;
  c.p.seg = segment_ids;
  c.p.seg_len = segment_ids ? seg_len : blk.kv_len;
  c.p.q_pos0 = q_pos0;
  c.p.kv_pos0 = kv_pos0;
  c.p.lse = const_cast<float*>(lse);
  c.p.delta = delta;
  c.p.dout = dout;
  c.p.dq_acc = dq_acc;
  c.p.dk_acc = dk_acc;
  c.p.dv_acc = dv_acc;
  c.p.init_dq = init_dq;
  c.p.init_dkv = init_dkv;
  c.p.dbias_keys = dbias_acc;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  RA_TRY(hip_status(ra::launch_bwd_dkdv_step_mfma(c.p, st), "dK/dV ring step launch"));
  return hip_status(ra::launch_bwd_dq_step_mfma(c.p, st), "dQ ring step launch");
}

int ra_blockwise_attn_bwd_dbias_reduce(const float* key_sums, int64_t kv_pos0, float* dbias, int32_t accumulate,
                                       const ra_shape* shape, void* stream) {
  Range range("ra_blockwise_attn_bwd_dbias_reduce kv_pos0=%lld", (long long)kv_pos0);
  RA_TRY(check_dims(shape));
  if (shape->bias_len < 1 || shape->bias_len >= kMaxPos)
    return fail(RA_ERR_ARG, "bias_len %lld must be in [1, 2^30)", (long long)shape->bias_len);
  if (kv_pos0 < 0 || kv_pos0 + shape->kv_len >= kMaxPos)
    return fail(RA_ERR_ARG, "kv_pos0 must be >= 0 and kv_pos0 + kv_len below 2^30");
  if (accumulate != 0 && accumulate != 1) return fail(RA_ERR_ARG, "accumulate must be 0 or 1 (got %d)", accumulate);
  const int64_t nk = static_cast<int64_t>(shape->batch) * shape->heads * shape->kv_len;
  const int64_t nb = static_cast<int64_t>(shape->heads) * shape->bias_len;
  if ((nb + 255) / 256 > 0x7fffffffLL) return fail(RA_ERR_SHAPE, "problem too large for one launch");
  RA_TRY(need_ptr(key_sums, nk, "key_sums", 4));
  RA_TRY(need_ptr(dbias, nb, "dbias", 4));
  if (nb == 0) return ok();
  return hip_status(ra::launch_bias_grad_block(key_sums, dbias, shape->batch, shape->heads, shape->kv_len, kv_pos0,
                                               shape->bias_len, accumulate, static_cast<hipStream_t>(stream)),
                    "dbias reduce launch");
}

int ra_blockwise_attn_bwd_finalize(const float* dq_acc, const float* dk_acc, const float* dv_acc, void* dq, void* dk,
                                   void* dv, const ra_shape* shape, void* stream) {
  Range range("ra_blockwise_attn_bwd_finalize");
  RA_TRY(check_dims(shape));
  const int64_t HB = static_cast<int64_t>(shape->batch) * shape->heads;
  const int64_t q_elems = HB * shape->q_len * shape->head_dim;
  const int64_t kv_elems = HB * shape->kv_len * shape->head_dim;
  if ((q_elems / 4 + 255) / 256 > 0x7fffffffLL || (kv_elems / 4 + 255) / 256 > 0x7fffffffLL)
    return fail(RA_ERR_SHAPE, "problem too large for one launch");
  RA_TRY(need_ptr(dq_acc, q_elems, "dq_acc", 16));
  RA_TRY(need_ptr(dk_acc, kv_elems, "dk_acc", 16));
  RA_TRY(need_ptr(dv_acc, kv_elems, "dv_acc", 16));
  const size_t el = shape->dtype == RA_BF16 ? 2 : 4;
  RA_TRY(need_ptr(dq, q_elems, "dq", el));
  RA_TRY(need_ptr(dk, kv_elems, "dk", el));
  RA_TRY(need_ptr(dv, kv_elems, "dv", el));
  const float scale = shape->scale > 0.f ? shape->scale : 1.0f / std::sqrt(static_cast<float>(shape->head_dim));
  const bool bf16 = shape->dtype == RA_BF16;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  RA_TRY(hip_status(ra::launch_grad_finalize(dq_acc, scale, dq, q_elems, bf16, st), "dQ finalize launch"));
  RA_TRY(hip_status(ra::launch_grad_finalize(dk_acc, scale, dk, kv_elems, bf16, st), "dK finalize launch"));
  return hip_status(ra::launch_grad_finalize(dv_acc, 1.0f, dv, kv_elems, bf16, st), "dV finalize launch");
}

int ra_blockwise_attn_fwd_finalize(const float* o_state, const float* m_state, const float* l_state, void* out,
                                   float* lse, const ra_shape* shape, void* stream) {
  Range range("ra_blockwise_attn_fwd_finalize");
  RA_TRY(check_dims(shape));
  Checked c;
  c.p = ra::Params{};
  c.p.B = shape->batch;
  c.p.H = shape->heads;
  c.p.D = shape->head_dim;
  c.p.Lq = shape->q_len;
  c.p.bf16 = shape->dtype == RA_BF16;
  c.rows = static_cast<int64_t>(shape->batch) * shape->heads * shape->q_len;
  c.q_elems = c.rows * shape->head_dim;
  if ((c.rows + 255) / 256 > 0x7fffffffLL) return fail(RA_ERR_SHAPE, "problem too large for one launch");
  RA_TRY(need_ptr(o_state, c.q_elems, "o_state", 16));
  RA_TRY(need_ptr(m_state, c.rows, "m_state", 4));
  RA_TRY(need_ptr(l_state, c.rows, "l_state", 4));
  RA_TRY(need_ptr(out, c.q_elems, "out", 16));
  RA_TRY(need_ptr(lse, c.rows, "lse", 4));
  if (c.rows == 0) return ok();
  c.p.o_state = const_cast<float*>(o_state);
  c.p.m_state = const_cast<float*>(m_state);
  c.p.l_state = const_cast<float*>(l_state);
  c.p.out = out;
  c.p.lse = lse;
  return hip_status(ra::launch_fwd_finalize(c.p, static_cast<hipStream_t>(stream)), "finalize launch");
}

int ra_attn_merge(void* out_a, float* lse_a, const void* out_b, const float* lse_b, const ra_shape* shape,
                  void* stream) {
  Range range("ra_attn_merge");
  RA_TRY(check_dims(shape));
  Checked c;
  c.p = ra::Params{};
  c.p.B = shape->batch;
  c.p.H = shape->heads;
  c.p.D = shape->head_dim;
  c.p.Lq = shape->q_len;
  c.p.bf16 = shape->dtype == RA_BF16;
  c.rows = static_cast<int64_t>(shape->batch) * shape->heads * shape->q_len;
  c.q_elems = c.rows * shape->head_dim;
  if ((c.rows + 255) / 256 > 0x7fffffffLL) return fail(RA_ERR_SHAPE, "problem too large for one launch");
  RA_TRY(need_ptr(out_a, c.q_elems, "out_a", 16));
  RA_TRY(need_ptr(lse_a, c.rows, "lse_a", 4));
  RA_TRY(need_ptr(out_b, c.q_elems, "out_b", 16));
  RA_TRY(need_ptr(lse_b, c.rows, "lse_b", 4));
  if (c.rows == 0) return ok();
  c.p.out = out_a;
  c.p.lse = lse_a;
  return hip_status(ra::launch_merge(c.p, out_b, lse_b, static_cast<hipStream_t>(stream)), "merge launch");
}

}  // extern "C"
