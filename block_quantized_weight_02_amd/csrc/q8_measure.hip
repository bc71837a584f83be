// q8_measure.hip -- the read ceiling the product is judged against: a kernel
// that reads a byte range once with the product's own weight-stream loads
// (16-byte non-temporal buffer loads, a contiguous slice per workgroup, the
// slice's 1 KiB pieces interleaved over the waves) and does no arithmetic
// on what it reads.  The product must move its algorithmic bytes at least
// once (docs.logicaffeine.com, logicaffeine_compile/spatial/passes/
// from_q8.rs, module doc: a decode step is bound by the weight's bytes), so
// the rate this kernel reaches over the same number of bytes is the rate a
// product on this chip can approach; the benchmark reports both.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q8_device.h"
#include "q8_internal.h"

namespace q8 {
namespace {

using namespace dev;

// DEPTH pieces of 1 KiB in flight per wave.  Loads past the slice's extent
// return zero (buffer resource bound), so the loop needs no tail branch.  The
// XOR of everything read is compared with a constant no input of the
// benchmark produces, so the loads stay live and nothing is written.
template <int DEPTH>
__global__ void __launch_bounds__(1024)
stream_read_kernel(const unsigned char *__restrict__ src, unsigned long long bytes,
                   unsigned long long slice, unsigned *__restrict__ sink) {
  const unsigned long long lo = (unsigned long long)blockIdx.x * slice;
  if (lo >= bytes) return;
  const unsigned len = (unsigned)((bytes - lo) < slice ? (bytes - lo) : slice);
  const buf_t r = make_buf(src + lo, len);
  const unsigned lane = threadIdx.x & 63;
  const unsigned wave = threadIdx.x >> 6;
  const unsigned W = blockDim.x >> 6;
  uint4 acc = make_uint4(0u, 0u, 0u, 0u);
  for (unsigned p = wave; p * 1024u < len; p += W * DEPTH) {
    uint4 v[DEPTH];
#pragma unroll
    for (int u = 0; u < DEPTH; ++u) v[u] = buf_ld16(r, (p + u * W) * 1024u + lane * 16u, 0);
#pragma unroll
    for (int u = 0; u < DEPTH; ++u) {
      acc.x ^= v[u].x;
      acc.y ^= v[u].y;
      acc.z ^= v[u].z;
      acc.w ^= v[u].w;
    }
  }
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9e3779b9u && acc.x == 0x7f4a7c15u) sink[0] = acc.y;
}

}  // namespace

hipError_t launch_stream_read(const void *src, unsigned long long bytes, int workgroups,
                              int waves, int depth, unsigned *sink, hipStream_t stream) {
  const unsigned long long pieces = (bytes + 1023) / 1024;
  const unsigned long long slice = (pieces + workgroups - 1) / workgroups * 1024;
  const unsigned char *p = static_cast<const unsigned char *>(src);
  const dim3 grid((unsigned)workgroups), block((unsigned)(64 * waves));
  switch (depth) {
    case 1: stream_read_kernel<1><<<grid, block, 0, stream>>>(p, bytes, slice, sink); break;
    case 2: stream_read_kernel<2><<<grid, block, 0, stream>>>(p, bytes, slice, sink); break;
    case 4: stream_read_kernel<4><<<grid, block, 0, stream>>>(p, bytes, slice, sink); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace q8
