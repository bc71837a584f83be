// q8_kernels.hip -- gfx950 kernels of the Q8_0 weight product.
//
// The product (docs.logicaffeine.com, logicaffeine_compile/spatial/passes/
// from_q8.rs, module doc and fn q8_fold): per Q8_0 block b the int8 block dot
// D = sum_i x[32b+i] * q[32b+i,n], scaled once by the block's fp32 scale and
// folded into an fp32 carry, y[r,n] = sum_b s[b,n] * D[r,b,n]; the weight is
// read once for all m rows.  The pages lower this onto a spatial fabric (a
// work item owns column tiles, K runs in 1024-row chunks) and onto a CUDA
// warp-per-output library; neither tiling is used here.  On gfx950:
//
//   * one 64-lane wave owns one 64-column tile: lane c owns column c, so the
//     activation values a wave needs at any moment are the same for all
//     lanes -- they are loaded once per wave into scalar registers (the
//     scalar cache is the broadcast) and feed the vector ALU as SGPR operands;
//   * each lane reads its column's 32 int8 values of a block as two 16-byte
//     loads; the packed layout makes every wave-wide load one contiguous,
//     fully used 1 KiB (layout in q8_internal.h);
//   * bf16 activations: per block two fp32 FMA chains of 16 (an int8 times a
//     bf16 is exact in fp32), then one FMA with the block's scale;
//     Q8_0 activations: eight v_dot4 int8 ops give the exact int32 block
//     dot, then one FMA with (activation scale * weight scale);
//   * a workgroup's waves split the tile's blocks; their carries meet in LDS
//     in fixed wave order; when K is also split across workgroups the last
//     workgroup to arrive sums the partial carries in fixed split order, so
//     results do not depend on scheduling.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q8_internal.h"

namespace q8 {
namespace {

// ---------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t pair) {  // element 2p
  return __uint_as_float(pair << 16);
}
__device__ __forceinline__ float bf16_hi(uint32_t pair) {  // element 2p+1
  return __uint_as_float(pair & 0xffff0000u);
}

// The four signed bytes of a dword as fp32 (exact); byte j is k = 4d + j.
__device__ __forceinline__ void i8x4_to_f32(uint32_t v, float *f) {
  f[0] = (float)(int8_t)(v);
  f[1] = (float)(int8_t)(v >> 8);
  f[2] = (float)(int8_t)(v >> 16);
  f[3] = (float)((int32_t)v >> 24);
}

// ---------------------------------------------------------------------------
// weight repack / unpack (from_q8.rs, enum Q8Part: the host repacks the
// checkpoint's blocks into the values and scales tensors)
// ---------------------------------------------------------------------------

// One thread per packed 16-byte run; run = ((t*NB + b)*2 + h)*64 + c.
__global__ void __launch_bounds__(256)
repack_kernel(const int8_t *__restrict__ q, const float *__restrict__ s,
              int8_t *__restrict__ wq, float *__restrict__ wsc, int K, int N,
              int NB, long long nruns) {
  const long long run = (long long)blockIdx.x * 256 + threadIdx.x;
  if (run >= nruns) return;
  const int c = (int)(run & 63);
  const int h = (int)((run >> 6) & 1);
  const long long tb = run >> 7;
  const int b = (int)(tb % NB);
  const int t = (int)(tb / NB);
  const int n = t * kTile + c;
  const int k0 = b * kBlock + h * 16;
  uint32_t d[4] = {0u, 0u, 0u, 0u};
  if (n < N) {
#pragma unroll
    for (int j = 0; j < 16; ++j)
      d[j >> 2] |= (uint32_t)(uint8_t)q[(size_t)(k0 + j) * N + n] << (8 * (j & 3));
  }
  *reinterpret_cast<uint4 *>(wq + run * 16) = make_uint4(d[0], d[1], d[2], d[3]);
  if (h == 0) wsc[tb * kTile + c] = (n < N) ? s[(size_t)b * N + n] : 0.0f;
}

__global__ void __launch_bounds__(256)
unpack_kernel(const int8_t *__restrict__ wq, const float *__restrict__ wsc,
              int8_t *__restrict__ q, float *__restrict__ s, int K, int N,
              int NB, long long nruns) {
  const long long run = (long long)blockIdx.x * 256 + threadIdx.x;
  if (run >= nruns) return;
  const int c = (int)(run & 63);
  const int h = (int)((run >> 6) & 1);
  const long long tb = run >> 7;
  const int b = (int)(tb % NB);
  const int t = (int)(tb / NB);
  const int n = t * kTile + c;
  if (n >= N) return;
  const int k0 = b * kBlock + h * 16;
  const uint4 v = *reinterpret_cast<const uint4 *>(wq + run * 16);
  const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int j = 0; j < 16; ++j)
    q[(size_t)(k0 + j) * N + n] = (int8_t)(d[j >> 2] >> (8 * (j & 3)));
  if (h == 0) s[(size_t)b * N + n] = wsc[tb * kTile + c];
}

// ---------------------------------------------------------------------------
// activation quantize (codegen_cuda/lane/plan.rs, const QBLOCK: int8 values
// and one scale per 32).  amax/127 and x/d are each one correctly rounded
// division (done in fp64, rounded once to fp32); ties round away from zero.
// ---------------------------------------------------------------------------

// One thread per element of the flattened m x K activation; a 32-lane group
// is one Q8_0 block (K % 32 == 0 and 256 % 32 == 0).
__global__ void __launch_bounds__(256)
quantize_act_kernel(const uint16_t *__restrict__ x, int8_t *__restrict__ xq,
                    float *__restrict__ dx, long long total) {
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  const bool valid = idx < total;
  const float v = valid ? __uint_as_float((uint32_t)x[idx] << 16) : 0.0f;
  float a = fabsf(v);
#pragma unroll
  for (int o = 16; o > 0; o >>= 1) a = fmaxf(a, __shfl_xor(a, o, 32));
  const float d = (float)((double)a / 127.0);
  int qv = 0;
  if (d != 0.0f) {
    const float quot = (float)((double)v / (double)d);
    float r = roundf(quot);  // half away from zero
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    qv = (int)r;
  }
  if (valid) {
    xq[idx] = (int8_t)qv;
    if ((idx & 31) == 0) dx[idx >> 5] = d;
  }
}

// ---------------------------------------------------------------------------
// the product, VALU form
// ---------------------------------------------------------------------------

// Blocks a wave has in flight per step of its block loop.
constexpr int kUnroll = 4;

template <int MR, int ACT, bool DOTS, int W>
__global__ void __launch_bounds__(64 * W)
gemv_valu_kernel(const void *__restrict__ xv, const int8_t *__restrict__ wq,
                 const float *__restrict__ wsc, float *__restrict__ y,
                 float *__restrict__ partial, unsigned *__restrict__ counters,
                 int32_t *__restrict__ dots, int m, int K, int NB, int Npad,
                 int S, unsigned act_scale_off) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t = blockIdx.x / S;
  const int s = blockIdx.x - t * S;
  const int b_lo = (int)(((long long)NB * s) / S);
  const int b_hi = (int)(((long long)NB * (s + 1)) / S);

  const int8_t *wtile = wq + (size_t)t * NB * kChunkBytes + lane * 16;
  const float *stile = wsc + (size_t)t * NB * kTile + lane;

  float acc[MR];
#pragma unroll
  for (int r = 0; r < MR; ++r) acc[r] = 0.0f;

  for (int b0 = b_lo + wave; b0 < b_hi; b0 += W * kUnroll) {
    uint4 wa[kUnroll], wb[kUnroll];
    float sc[kUnroll];
    // Issue every load of the step first; a block past the range reloads the
    // last block of the range (in bounds) and is not used.
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int b = min(b0 + u * W, b_hi - 1);
      const int8_t *c = wtile + (size_t)b * kChunkBytes;
      wa[u] = *reinterpret_cast<const uint4 *>(c);
      wb[u] = *reinterpret_cast<const uint4 *>(c + kHalfBytes);
      if constexpr (!DOTS) sc[u] = stile[(size_t)b * kTile];
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int b = b0 + u * W;
      if (b >= b_hi) break;
      const uint32_t wd[8] = {wa[u].x, wa[u].y, wa[u].z, wa[u].w,
                              wb[u].x, wb[u].y, wb[u].z, wb[u].w};
      if constexpr (ACT == kActBf16) {
        float wf[32];
#pragma unroll
        for (int d = 0; d < 8; ++d) i8x4_to_f32(wd[d], wf + 4 * d);
        const uint16_t *xb = static_cast<const uint16_t *>(xv);
#pragma unroll
        for (int r = 0; r < MR; ++r) {
          if (r < m) {
            const uint32_t *xr = reinterpret_cast<const uint32_t *>(
                xb + (size_t)r * K + (size_t)b * kBlock);
            float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
            for (int p = 0; p < 8; ++p) {
              const uint32_t lo = xr[p], hi = xr[p + 8];
              p0 = fmaf(bf16_lo(lo), wf[2 * p], p0);
              p0 = fmaf(bf16_hi(lo), wf[2 * p + 1], p0);
              p1 = fmaf(bf16_lo(hi), wf[16 + 2 * p], p1);
              p1 = fmaf(bf16_hi(hi), wf[16 + 2 * p + 1], p1);
            }
            acc[r] = fmaf(sc[u], p0 + p1, acc[r]);
          }
        }
      } else {
        const int8_t *xq = static_cast<const int8_t *>(xv);
        const float *dxp = reinterpret_cast<const float *>(
            static_cast<const char *>(xv) + act_scale_off);
#pragma unroll
        for (int r = 0; r < MR; ++r) {
          if (r < m) {
            const int *xr = reinterpret_cast<const int *>(
                xq + (size_t)r * K + (size_t)b * kBlock);
            int D = 0;
#pragma unroll
            for (int d = 0; d < 8; ++d)
              D = __builtin_amdgcn_sdot4((int)wd[d], xr[d], D, false);
            if constexpr (DOTS) {
              dots[((size_t)r * NB + b) * Npad + (size_t)t * kTile + lane] = D;
            } else {
              const float dxs = dxp[(size_t)r * NB + b];
              acc[r] = fmaf(dxs * sc[u], (float)D, acc[r]);
            }
          }
        }
      }
    }
  }
  if constexpr (DOTS) return;

  // Carries of the W waves meet in LDS, summed in wave order.
  __shared__ float red[W][MR][64];
#pragma unroll
  for (int r = 0; r < MR; ++r) red[wave][r][lane] = acc[r];
  __syncthreads();
  const size_t col0 = (size_t)t * kTile;
  for (int idx = threadIdx.x; idx < MR * 64; idx += 64 * W) {
    const int r = idx >> 6, c = idx & 63;
    if (r < m) {
      float v = red[0][r][c];
#pragma unroll
      for (int w = 1; w < W; ++w) v += red[w][r][c];
      if (S == 1)
        y[(size_t)r * Npad + col0 + c] = v;
      else
        partial[((size_t)s * m + r) * Npad + col0 + c] = v;
    }
  }
  if (S == 1) return;

  // Split K: the last workgroup of the tile to arrive sums the S partial
  // carries in split order and resets the tile's counter for the next call.
  __shared__ int is_last;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0)
    is_last = (atomicAdd(&counters[t], 1u) == (unsigned)(S - 1)) ? 1 : 0;
  __syncthreads();
  if (!is_last) return;
  __threadfence();
  for (int idx = threadIdx.x; idx < MR * 64; idx += 64 * W) {
    const int r = idx >> 6, c = idx & 63;
    if (r < m) {
      float v = partial[(size_t)r * Npad + col0 + c];
      for (int ss = 1; ss < S; ++ss)
        v += partial[((size_t)ss * m + r) * Npad + col0 + c];
      y[(size_t)r * Npad + col0 + c] = v;
    }
  }
  if (threadIdx.x == 0) counters[t] = 0u;
}

template <int MR, int ACT, bool DOTS, int W>
hipError_t launch_valu(const GemvArgs &a, hipStream_t stream) {
  const dim3 grid((unsigned)(a.T * a.split_k));
  const dim3 block(64 * W);
  gemv_valu_kernel<MR, ACT, DOTS, W><<<grid, block, 0, stream>>>(
      a.x, a.wq, a.wsc, a.y, a.partial, a.counters, a.dots, a.m, a.K, a.NB,
      a.Npad, a.split_k, a.act_scale_off);
  return hipGetLastError();
}

using Launcher = hipError_t (*)(const GemvArgs &, hipStream_t);

template <int ACT, bool DOTS, int W>
Launcher pick_valu_rows(int rows) {
  switch (rows) {
    case 1: return &launch_valu<1, ACT, DOTS, W>;
    case 2: return &launch_valu<2, ACT, DOTS, W>;
    case 4: return &launch_valu<4, ACT, DOTS, W>;
    case 8: return &launch_valu<8, ACT, DOTS, W>;
    case 16: return &launch_valu<16, ACT, DOTS, W>;
    case 32: return &launch_valu<32, ACT, DOTS, W>;
    default: return nullptr;
  }
}

template <int W>
Launcher pick_valu(int rows, int act, bool dots) {
  if (act == kActBf16) return dots ? nullptr : pick_valu_rows<kActBf16, false, W>(rows);
  if (act == kActQ8)
    return dots ? pick_valu_rows<kActQ8, true, W>(rows)
                : pick_valu_rows<kActQ8, false, W>(rows);
  return nullptr;
}

Launcher pick(int kernel, int rows, int act, bool dots, int waves) {
  if (kernel == 0) {
    if (waves == 4) return pick_valu<4>(rows, act, dots);
    if (waves == 8 && rows <= 8) return pick_valu<8>(rows, act, dots);
  }
  return nullptr;
}

unsigned blocks_for(long long n) { return (unsigned)((n + 255) / 256); }

}  // namespace

hipError_t launch_repack(const int8_t *q_kn, const float *s_kn, int K, int N,
                         int8_t *wq, float *wsc, hipStream_t stream) {
  const int NB = K / kBlock, T = (N + kTile - 1) / kTile;
  const long long nruns = (long long)T * NB * 128;
  repack_kernel<<<blocks_for(nruns), 256, 0, stream>>>(q_kn, s_kn, wq, wsc, K, N, NB, nruns);
  return hipGetLastError();
}

hipError_t launch_unpack(const int8_t *wq, const float *wsc, int K, int N,
                         int8_t *q_kn, float *s_kn, hipStream_t stream) {
  const int NB = K / kBlock, T = (N + kTile - 1) / kTile;
  const long long nruns = (long long)T * NB * 128;
  unpack_kernel<<<blocks_for(nruns), 256, 0, stream>>>(wq, wsc, q_kn, s_kn, K, N, NB, nruns);
  return hipGetLastError();
}

hipError_t launch_quantize_act(const uint16_t *x, void *x_q8, int m, int K,
                               unsigned scale_off, hipStream_t stream) {
  const long long total = (long long)m * K;
  int8_t *xq = static_cast<int8_t *>(x_q8);
  float *dx = reinterpret_cast<float *>(static_cast<char *>(x_q8) + scale_off);
  quantize_act_kernel<<<blocks_for(total), 256, 0, stream>>>(x, xq, dx, total);
  return hipGetLastError();
}

bool gemv_instantiated(int kernel, int rows, int act, bool write_dots, int waves) {
  return pick(kernel, rows, act, write_dots, waves) != nullptr;
}

hipError_t launch_gemv(int kernel, int rows, int act, bool write_dots,
                       int waves, const GemvArgs &a, hipStream_t stream) {
  Launcher f = pick(kernel, rows, act, write_dots, waves);
  if (!f) return hipErrorInvalidValue;
  return f(a, stream);
}

}  // namespace q8
