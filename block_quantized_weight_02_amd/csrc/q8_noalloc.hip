// q8_noalloc.hip -- the product for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc): q8_gemv's default plan and kernels, its split-K
// workspace taken from one fixed device array per GPU instead of an
// allocation.
//
// `scratch` is a file-scope device array; in host code its name is only a
// host-side stand-in, so the device address of each GPU's copy is looked up
// once per device (hipGetSymbolAddress, with that device current) and only
// that address is ever handed to a kernel.  The array keeps the last call's
// contents; the split-K arrival counters at its front must be zero when a
// call starts and every call leaves them zero, so they are cleared once, at
// the first call on each device (a fill kernel on the caller's stream).
// Every call on one GPU shares the array: calls that overlap on one GPU
// (different streams, or different threads without ordering) race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/q8gemv.h"
#include "q8_internal.h"

static __device__ __align__(256) unsigned char scratch[Q8_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_ptr[kMaxDevices];            // each device's address of `scratch`

__global__ void __launch_bounds__(256) clear_words(unsigned *__restrict__ p, unsigned long long n) {
  for (unsigned long long i = (unsigned long long)blockIdx.x * 256 + threadIdx.x; i < n;
       i += (unsigned long long)gridDim.x * 256)
    p[i] = 0u;
}

// The current device's scratch address, set up on its first use.
int device_scratch(hipStream_t stream, void **out) {
  *out = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    return q8::report_error(Q8_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  }
  if (dev < 0 || dev >= kMaxDevices) {
    return q8::report_error(Q8_ERR_HIP, "device %d beyond the %d devices this entry point serves",
                            dev, kMaxDevices);
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      return q8::report_error(Q8_ERR_HIP, "hipGetSymbolAddress(scratch): %s",
                              hipGetErrorString(e));
    }
    (void)hipGetLastError();
    clear_words<<<256, 256, 0, stream>>>(static_cast<unsigned *>(p),
                                          Q8_NOALLOC_SCRATCH_BYTES / 4);
    e = hipGetLastError();
    if (e != hipSuccess) {
      return q8::report_error(Q8_ERR_HIP, "scratch clear launch: %s", hipGetErrorString(e));
    }
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return Q8_OK;
}

}  // namespace

extern "C" {

size_t q8_noalloc_scratch_bytes(void) { return Q8_NOALLOC_SCRATCH_BYTES; }

int q8_gemv_noalloc(const void *x, const int8_t *W_q8, const float *W_q8_scale, float *y,
                    int64_t m, int64_t K, int64_t N, int act_fmt, hipStream_t stream) {
  // the workspace q8_gemv's default plan needs (0: no K split, or a shape
  // the product rejects, which q8_gemv_ws then reports)
  const size_t need = q8_gemv_workspace_bytes(m, K, N, act_fmt);
  if (need > Q8_NOALLOC_SCRATCH_BYTES) {
    return q8::report_error(Q8_ERR_WORKSPACE,
                            "m = %lld, K = %lld, N = %lld needs a %zu-byte split-K workspace, "
                            "more than the %d-byte scratch of q8_gemv_noalloc: use q8_gemv_ws "
                            "with a workspace of that size",
                            (long long)m, (long long)K, (long long)N, need,
                            Q8_NOALLOC_SCRATCH_BYTES);
  }
  void *ws = nullptr;
  if (need > 0) {
    const int st = device_scratch(stream, &ws);
    if (st != Q8_OK) return st;
  }
  return q8_gemv_ws(x, W_q8, W_q8_scale, y, m, K, N, act_fmt, stream, ws,
                    need > 0 ? (size_t)Q8_NOALLOC_SCRATCH_BYTES : 0);
}

}  // extern "C"
