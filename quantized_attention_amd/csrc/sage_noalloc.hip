// sage_noalloc.hip -- the entry point that allocates nothing: sage_quant_qk
// with its column-statistics scratch in a file-scope device array instead
// of a caller workspace (for callers that cannot allocate device memory).
//
// `scratch` is a host-side stand-in in host code: its device address is
// looked up once per device with hipGetSymbolAddress (each GPU holds its own
// copy) and only that pointer is handed to the kernels.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "sage.h"

hipError_t sage_launch_quant_qk(const void* q, const void* k, int bf16, int B, int H, int H_kv,
                                int N, int d, int q_group, int smooth_k, int smooth_q,
                                int8_t* q_i8, float* q_scale, int8_t* k_i8, float* k_scale,
                                float* k_mean, float* q_mean, void* ws, hipStream_t st);
size_t sage_ws_quant_qk_bytes(int B, int H_kv, int N, int d);

// The FP64 per-chunk column sums of K (written in full by every call before
// they are read, so nothing needs clearing between calls).
static __device__ __align__(256) unsigned char scratch[SAGE_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void* g_scratch[kMaxDevices] = {};

// The device address of `scratch` on device `dev` (looked up with that device
// current, once; later calls reuse it).  nullptr on failure.
void* scratch_on(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> g(g_lock);
  if (g_scratch[dev]) return g_scratch[dev];
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return nullptr;
  if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
  void* ptr = nullptr;
  const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (cur != dev) (void)hipSetDevice(cur);
  if (e != hipSuccess || ptr == nullptr) return nullptr;
  g_scratch[dev] = ptr;
  return ptr;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

extern "C" sage_status sage_quant_qk_noalloc(const void* q, const void* k, sage_dtype dtype, int B,
                                             int H, int H_kv, int N, int d, int q_group,
                                             int smooth_k, int smooth_q, int8_t* q_i8,
                                             float* q_scale, int8_t* k_i8, float* k_scale,
                                             float* k_mean, float* q_mean, void* stream) {
  if (!q || !k || !q_i8 || !q_scale || !k_i8 || !k_scale || !k_mean) return SAGE_ERR_NULL;
  if (smooth_q == 1 && !q_mean) return SAGE_ERR_NULL;
  // the same shape rules as every entry point (buffer-size query)
  sage_sizes sz;
  const sage_status st = sage_buffer_sizes(B, H, H_kv, N, d, q_group, &sz);
  if (st != SAGE_OK) return st;
  if (dtype != SAGE_FP16 && dtype != SAGE_BF16) return SAGE_ERR_DTYPE;
  if (smooth_k != 0 && smooth_k != 1) return SAGE_ERR_ARG;
  if (smooth_q != 0 && smooth_q != 1) return SAGE_ERR_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(q_i8) || !aligned16(k_i8)) return SAGE_ERR_ALIGN;
  if (smooth_k && sage_ws_quant_qk_bytes(B, H_kv, N, d) > (size_t)SAGE_SCRATCH_BYTES)
    return SAGE_ERR_SCRATCH;
  int dev = -1;
  if (stream) {
    if (hipStreamGetDevice((hipStream_t)stream, &dev) != hipSuccess) return SAGE_ERR_HIP;
  } else if (hipGetDevice(&dev) != hipSuccess) {
    return SAGE_ERR_HIP;
  }
  void* ws = scratch_on(dev);
  if (!ws) return SAGE_ERR_HIP;
  const hipError_t e = sage_launch_quant_qk(q, k, dtype == SAGE_BF16, B, H, H_kv, N, d, q_group,
                                            smooth_k, smooth_q, q_i8, q_scale, k_i8, k_scale,
                                            k_mean, q_mean, ws, (hipStream_t)stream);
  return e == hipSuccess ? SAGE_OK : SAGE_ERR_HIP;
}
