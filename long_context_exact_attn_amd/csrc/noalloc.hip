// The backward entry point that allocates nothing, for callers that cannot call hipMalloc or pass
// a workspace (code under HIP graph capture, tight serving loops, harnesses that forbid
// allocation).  Its one scratch buffer, Delta = rowsum(dout * out) of float32 [B, H, Lq], lives in
// a file-scope device array of a fixed size that each GPU holds until the process ends.
//
// Host code never uses the array's name as an address (on the host it names a stand-in, not
// device memory): the device address is looked up once per device with hipGetSymbolAddress, with
// that device current, and kept per device.  Every call on a GPU shares that GPU's array; the
// preprocess kernel writes every Delta row the two gradient kernels read, so nothing in it has to
// start at zero and a call never reads what an earlier call left.  Calls that overlap on one GPU
// (different streams, or threads) race on the array.
#include <mutex>

#include "../../include/ra_attn.h"
#include "ra_common.cuh"

namespace {

constexpr size_t kScratchBytes = size_t(16) << 20;   // 16 MiB: B * H * Lq <= 4,194,304 Delta rows
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mutex;
void* g_scratch[kMaxDevices] = {};   // device address of `scratch` on each device, once looked up

thread_local std::string g_error;

int fail_noalloc(int code, const char* msg) {
  g_error = msg;
  return code;
}

}  // namespace

extern "C" {

size_t ra_blockwise_attn_bwd_noalloc_max_workspace(void) { return kScratchBytes; }

const char* ra_noalloc_last_error(void) { return g_error.c_str(); }

int ra_blockwise_attn_bwd_noalloc(const void* q, const void* k, const void* v, const float* bias,
                                  const int32_t* segment_ids, int32_t n_ring, int64_t q_chunk, int64_t k_chunk,
                                  int32_t causal, const void* out, const float* lse, const void* dout, void* dq,
                                  void* dk, void* dv, const ra_shape* shape, void* stream) {
  g_error.clear();
  if (!shape) return fail_noalloc(RA_ERR_ARG, "shape is NULL");
  const size_t need = ra_blockwise_attn_bwd_workspace_size(shape, n_ring);
  if (need > kScratchBytes)
    return fail_noalloc(RA_ERR_WORKSPACE,
                        "the allocation-free backward holds at most 4,194,304 rows (batch * heads * q_len) of Delta "
                        "in its 16 MiB static scratch; use ra_blockwise_attn_bwd with a workspace");
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail_noalloc(RA_ERR_HIP, "no current HIP device (or its ordinal is 64 or more)");
  void* ptr = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_mutex);
    if (!g_scratch[dev]) {
      // the device is current here, so the address is that device's copy of the array
      const hipError_t e = hipGetSymbolAddress(&g_scratch[dev], HIP_SYMBOL(scratch));
      if (e != hipSuccess || !g_scratch[dev]) {
        g_scratch[dev] = nullptr;
        return fail_noalloc(RA_ERR_HIP, "hipGetSymbolAddress of the static scratch array failed");
      }
    }
    ptr = g_scratch[dev];
  }
  // the workspace path of the ordinary entry point, with the static array as its workspace
  return ra_blockwise_attn_bwd(q, k, v, bias, segment_ids, n_ring, q_chunk, k_chunk, causal, out, lse, dout, dq,
                               dk, dv, ptr, kScratchBytes, shape, stream);
}

}  // extern "C"
