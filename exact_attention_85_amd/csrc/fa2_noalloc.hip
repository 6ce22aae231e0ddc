// fa2_fwd_splitkv_noalloc: the split-KV forward of fa2_fwd_splitkv with its
// partials in a fixed device array that the library owns, for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc).  It runs the same two kernels over
// the same workspace layout; it calls no allocating routine.
//
// The array `scratch` is file-scope device memory: each GPU the library runs on
// holds its own copy at its own address until the process ends.  In host code
// the name `scratch` is only a host-side stand-in, so the device address of each
// GPU's copy is looked up once per device with hipGetSymbolAddress (with that
// device current) and kept in `g_scratch`; kernels receive that address.
#include <hip/hip_runtime.h>

#include <mutex>

#include "fa2.h"
#include "fa2_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[FA2_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices];  // device address of `scratch` on each device; null until looked up

// The device address of `scratch` on `dev`, looked up on the first call for that
// device (with `dev` made current for the lookup, then the caller's device restored).
int scratch_on(int dev, float** out) {
  if (dev < 0 || dev >= kMaxDevices) return FA2_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_scratch[dev]) {
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return FA2_ERR_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return FA2_ERR_HIP;
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return FA2_ERR_HIP;
    if (e != hipSuccess || !ptr) return FA2_ERR_HIP;
    g_scratch[dev] = ptr;
  }
  *out = static_cast<float*>(g_scratch[dev]);
  return FA2_OK;
}

}  // namespace

extern "C" int fa2_fwd_splitkv_noalloc(const void* Q, const void* K, const void* V, void* O, float* LSE, int B,
                                       int H, int N_q, int N_k, int d, int causal, float scale, int num_splits,
                                       void* stream) {
  // every argument check first, with no HIP call
  int rc = fa2::splitkv_check_args(Q, K, V, O, LSE, B, H, N_q, N_k, d, scale, num_splits);
  if (rc != FA2_OK) return rc;
  if (fa2_splitkv_workspace_bytes(B, H, N_q, d, num_splits) > (size_t)FA2_NOALLOC_SCRATCH_BYTES)
    return FA2_ERR_SCRATCH;
  // the kernels run on the stream's device: use that device's copy of the array
  int dev = 0;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if ((s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev)) != hipSuccess) return FA2_ERR_HIP;
  float* ws = nullptr;
  rc = scratch_on(dev, &ws);
  if (rc != FA2_OK) return rc;
  // every partial slot the merge reads is written by the partial pass first (stream order),
  // so the array needs no clearing between calls
  return fa2::splitkv_run(Q, K, V, O, LSE, B, H, N_q, N_k, d, causal, scale, num_splits, ws, stream);
}
