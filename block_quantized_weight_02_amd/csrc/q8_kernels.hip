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

#include "q8_device.h"
#include "q8_internal.h"
#include "q8_product.h"

namespace q8 {
namespace {

using namespace dev;

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
  if (h == 0) wsc[tb * kTile + scale_pos(c)] = (n < N) ? s[(size_t)b * N + n] : 0.0f;
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
  if (h == 0) s[(size_t)b * N + n] = wsc[tb * kTile + scale_pos(c)];
}

// ---------------------------------------------------------------------------
// activation quantize (codegen_cuda/lane/plan.rs, const QBLOCK: int8 values
// and one scale per 32).  amax/127 and x/d are each one correctly rounded
// division (done in fp64, rounded once to fp32); ties round away from zero.
// ---------------------------------------------------------------------------

// E (4 or 8) consecutive values a thread: row r = blockIdx.y, values k0 ..
// k0 + E - 1 with k0 = E (blockIdx.x * 256 + threadIdx.x); 32 / E threads are
// one Q8_0 block (K % 32 == 0), whose amax meets over log2(32 / E) lane
// exchanges.  One E*2-byte load and two E-byte stores a thread: the codes
// row-major and in the block-interleaved view, and one scale per block.
// Measured on MI355X against one value a thread (loop us, E = 4 / 8 / 1):
// m=1, K=4096: 1.84 / 2.03 / 1.89; m=16: 2.08 / 2.31 / 1.99; m=32, K=5120:
// 2.11 / 2.32 / 2.20; m=128: 2.39 / 2.54 / 2.92; m=512: 4.26 / 4.19 / 6.66.
template <int E>
__global__ void __launch_bounds__(256)
quantize_act_vec_kernel(const uint16_t *__restrict__ x, int8_t *__restrict__ xq,
                        float *__restrict__ dx, int8_t *__restrict__ xv, int m, int K) {
  constexpr int TPB = 32 / E;   // threads a block
  const int r = blockIdx.y;
  const int k0 = (blockIdx.x * 256 + threadIdx.x) * E;
  const bool valid = k0 < K;
  const size_t idx = (size_t)r * K + k0;
  uint32_t w[E / 2];
  if (valid) {
    if constexpr (E == 8) {
      const uint4 u = *reinterpret_cast<const uint4 *>(x + idx);
      w[0] = u.x; w[1] = u.y; w[2] = u.z; w[3] = u.w;
    } else {
      const uint2 u = *reinterpret_cast<const uint2 *>(x + idx);
      w[0] = u.x; w[1] = u.y;
    }
  } else {
#pragma unroll
    for (int e = 0; e < E / 2; ++e) w[e] = 0u;
  }
  float v[E];
#pragma unroll
  for (int e = 0; e < E / 2; ++e) {
    v[2 * e] = __uint_as_float(w[e] << 16);
    v[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
  }
  float a = 0.0f;
#pragma unroll
  for (int e = 0; e < E; ++e) a = fmaxf(a, fabsf(v[e]));
#pragma unroll
  for (int o = TPB / 2; o > 0; o >>= 1) a = fmaxf(a, __shfl_xor(a, o, TPB));
  const float d = q8_scale_of(a);
  if (valid) {
    uint32_t c[E / 4];
#pragma unroll
    for (int j = 0; j < E / 4; ++j) {
      uint32_t p = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) p |= (uint32_t)(uint8_t)q8_code_of(v[4 * j + e], d) << (8 * e);
      c[j] = p;
    }
    int8_t *dv = xv + ((size_t)(k0 >> 5) * m + r) * 32 + (k0 & 31);
    if constexpr (E == 8) {
      *reinterpret_cast<uint2 *>(xq + idx) = make_uint2(c[0], c[1]);
      *reinterpret_cast<uint2 *>(dv) = make_uint2(c[0], c[1]);
    } else {
      *reinterpret_cast<uint32_t *>(xq + idx) = c[0];
      *reinterpret_cast<uint32_t *>(dv) = c[0];
    }
    if ((k0 & 31) == 0) dx[idx >> 5] = d;
  }
}

// The two-word form (one value a thread): the first word and the scale as
// above, the second word
// round_half_away(128 * (quot - hi)) of the correctly rounded fp32 quotient
// quot = v / d.
// quot - hi is exact in fp32 (hi is quot rounded, within a factor of two of
// it or zero) and the scaling by 128 is exact, so the second word is unique.
__global__ void __launch_bounds__(256)
quantize_act_two_words_kernel(const uint16_t *__restrict__ x, int8_t *__restrict__ hi,
                              int8_t *__restrict__ lo, float *__restrict__ dx,
                              long long total) {
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  const bool valid = idx < total;
  const float v = valid ? __uint_as_float((uint32_t)x[idx] << 16) : 0.0f;
  float a = fabsf(v);
#pragma unroll
  for (int o = 16; o > 0; o >>= 1) a = fmaxf(a, __shfl_xor(a, o, 32));
  const float d = q8_scale_of(a);
  if (valid) {
    int h = 0, l = 0;
    if (d != 0.0f) {
      const float quot = q8_quot(v, d);
      const float rh = fminf(fmaxf(roundf(quot), -127.0f), 127.0f);
      h = (int)rh;
      l = (int)roundf((quot - rh) * 128.0f);
    }
    hi[idx] = (int8_t)h;
    lo[idx] = (int8_t)l;
    if ((idx & 31) == 0) dx[idx >> 5] = d;
  }
}

// ---------------------------------------------------------------------------
// the product, VALU form: lane = column, activation in scalar registers
// ---------------------------------------------------------------------------

// Blocks a wave loads per stage; two stages are in flight (double buffer).
#ifndef Q8_VALU_UNROLL
#define Q8_VALU_UNROLL 1
#endif
constexpr int kUnroll = Q8_VALU_UNROLL;

// Rows whose activation is prefetched with the stage (scalar registers): one
// bf16 row is 16 dwords a block, an int8 row 8 dwords and its scale (two-word
// rows: 8 dwords of each word); more rows than two would overflow the scalar
// registers.
template <int MR, int ACT>
struct ValuX {
  static constexpr bool kPrefetch = MR <= 2;
  static constexpr int kRows = kPrefetch ? MR : 1;
  static constexpr int kWords = (ACT == kActQ8) ? 8 : 16;
};

template <int MR, int ACT, bool DOTS>
struct ValuStage {
  uint4 wa[kUnroll], wb[kUnroll];
  float sc[kUnroll];
  uint32_t x[kUnroll][ValuX<MR, ACT>::kRows][ValuX<MR, ACT>::kWords];
  float dx[kUnroll][ValuX<MR, ACT>::kRows];
};

// Where a wave's tile comes from: buffer resources (wave-uniform base and
// extent in scalar registers; a loop with them needs no per-lane 64-bit
// addresses), or plain pointers where the scalar registers are taken by the
// prefetched activation (two rows).  lw, ls: the lane's byte offsets.
template <int MR>
struct ValuSrc {
  static constexpr bool kBuf = MR != 2;
  buf_t wr, sr;
  const int8_t *wp;
  const float *sp;
  unsigned lw, ls;
};

// Issue the loads of the stage's blocks b0 + u*W; a block past the range
// reloads the range's last block (in bounds) and is not used.
template <int MR, int ACT, bool DOTS, int W>
__device__ __forceinline__ void valu_load(ValuStage<MR, ACT, DOTS> &st, const ValuSrc<MR> &src,
                                          int b0, int b_hi, const void *__restrict__ xv, int m,
                                          int K, int NB, unsigned act_scale_off) {
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int b = min(b0 + u * W, b_hi - 1);
    if constexpr (ValuSrc<MR>::kBuf) {
      const unsigned wb = (unsigned)b * kChunkBytes, sb = (unsigned)b * (kTile * 4);
      st.wa[u] = buf_ld16(src.wr, src.lw, wb);
      st.wb[u] = buf_ld16(src.wr, src.lw + kHalfBytes, wb);
      if constexpr (!DOTS) st.sc[u] = buf_ld4f(src.sr, src.ls, sb);
    } else {
      const int8_t *c = src.wp + (size_t)b * kChunkBytes + src.lw;
      st.wa[u] = ld_stream16(c);
      st.wb[u] = ld_stream16(c + kHalfBytes);
      if constexpr (!DOTS)
        st.sc[u] = ld_scale4f(reinterpret_cast<const float *>(
            reinterpret_cast<const char *>(src.sp) + (size_t)b * (kTile * 4) + src.ls));
    }
    if constexpr (ValuX<MR, ACT>::kPrefetch) {
#pragma unroll
      for (int r = 0; r < MR; ++r) {
        const int rr = min(r, m - 1);   // rows past m reload row m-1, unused
        if constexpr (ACT == kActBf16) {
          const uint32_t *xr = reinterpret_cast<const uint32_t *>(
              static_cast<const uint16_t *>(xv) + (size_t)rr * K + (size_t)b * kBlock);
#pragma unroll
          for (int p = 0; p < 16; ++p) st.x[u][r][p] = xr[p];
        } else {
          const uint32_t *xr = reinterpret_cast<const uint32_t *>(
              static_cast<const int8_t *>(xv) + (size_t)rr * K + (size_t)b * kBlock);
#pragma unroll
          for (int p = 0; p < 8; ++p) st.x[u][r][p] = xr[p];
          if constexpr (ACT == kActQ8x2) {   // the second words: rows m .. 2m-1
            const uint32_t *xl = reinterpret_cast<const uint32_t *>(
                static_cast<const int8_t *>(xv) + ((size_t)m + rr) * K + (size_t)b * kBlock);
#pragma unroll
            for (int p = 0; p < 8; ++p) st.x[u][r][8 + p] = xl[p];
          }
          if constexpr (!DOTS)
            st.dx[u][r] = reinterpret_cast<const float *>(static_cast<const char *>(xv) +
                                                          act_scale_off)[(size_t)rr * NB + b];
        }
      }
    }
  }
}

template <int MR, int ACT, bool DOTS, int W>
__device__ __forceinline__ void valu_compute(const ValuStage<MR, ACT, DOTS> &st, float *acc,
                                             int b0, int b_hi, const void *__restrict__ xv,
                                             int32_t *__restrict__ dots, int m, int K, int NB,
                                             int Npad, int t, int lane,
                                             unsigned act_scale_off) {
  constexpr bool kPre = ValuX<MR, ACT>::kPrefetch;
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int b = b0 + u * W;
    if (b >= b_hi) break;
    const uint32_t wd[8] = {st.wa[u].x, st.wa[u].y, st.wa[u].z, st.wa[u].w,
                            st.wb[u].x, st.wb[u].y, st.wb[u].z, st.wb[u].w};
    if constexpr (ACT == kActBf16) {
      float wf[32];
#pragma unroll
      for (int d = 0; d < 8; ++d) i8x4_to_f32(wd[d], wf + 4 * d);
      const uint16_t *xb = static_cast<const uint16_t *>(xv);
#pragma unroll
      for (int r = 0; r < MR; ++r) {
        if (r < m) {
          const uint32_t *xr =
              reinterpret_cast<const uint32_t *>(xb + (size_t)r * K + (size_t)b * kBlock);
          float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
          for (int p = 0; p < 8; ++p) {
            uint32_t lo, hi;
            if constexpr (kPre) {
              lo = st.x[u][r][p];
              hi = st.x[u][r][p + 8];
            } else {
              lo = xr[p];
              hi = xr[p + 8];
            }
            p0 = fmaf(bf16_lo(lo), wf[2 * p], p0);
            p0 = fmaf(bf16_hi(lo), wf[2 * p + 1], p0);
            p1 = fmaf(bf16_lo(hi), wf[16 + 2 * p], p1);
            p1 = fmaf(bf16_hi(hi), wf[16 + 2 * p + 1], p1);
          }
          acc[r] = fmaf(st.sc[u], p0 + p1, acc[r]);
        }
      }
    } else {
      const int8_t *xq = static_cast<const int8_t *>(xv);
      const float *dxp =
          reinterpret_cast<const float *>(static_cast<const char *>(xv) + act_scale_off);
#pragma unroll
      for (int r = 0; r < MR; ++r) {
        if (r < m) {
          const int *xr = reinterpret_cast<const int *>(xq + (size_t)r * K + (size_t)b * kBlock);
          int D = 0;
#pragma unroll
          for (int d = 0; d < 8; ++d)
            D = __builtin_amdgcn_sdot4((int)wd[d], kPre ? (int)st.x[u][r][d] : xr[d], D, false);
          if constexpr (ACT == kActQ8x2) {
            // The second words' dot, joined with the first exactly in int32
            // (|128 D_hi + D_lo| < 2^27), then one FMA with the block's scales.
            const int *xl =
                reinterpret_cast<const int *>(xq + ((size_t)m + r) * K + (size_t)b * kBlock);
            int Dl = 0;
#pragma unroll
            for (int d = 0; d < 8; ++d)
              Dl = __builtin_amdgcn_sdot4((int)wd[d], kPre ? (int)st.x[u][r][8 + d] : xl[d], Dl,
                                          false);
            const float dxv = kPre ? st.dx[u][r] : dxp[(size_t)r * NB + b];
            acc[r] = fmaf(dxv * st.sc[u], (float)(D * 128 + Dl) * 0.0078125f, acc[r]);
          } else if constexpr (DOTS) {
            dots[((size_t)r * NB + b) * Npad + (size_t)t * kTile + lane] = D;
          } else {
            const float dxv = kPre ? st.dx[u][r] : dxp[(size_t)r * NB + b];
            acc[r] = fmaf(dxv * st.sc[u], (float)D, acc[r]);
          }
        }
      }
    }
  }
}

template <int MR, int ACT, bool DOTS, int W, bool PAIR, bool PARTS>
__global__ void __launch_bounds__(64 * W)
gemv_valu_kernel(const void *__restrict__ xv, const int8_t *__restrict__ wq,
                 const float *__restrict__ wsc, float *__restrict__ y,
                 float *__restrict__ partial, unsigned *__restrict__ counters,
                 int32_t *__restrict__ dots, int m, int K, int NB, int Npad,
                 int S, int split_q, int split_r, unsigned act_scale_off, Epi ep) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // unit tv: a tile of the product, of a gated pair's weight (the pair's two
  // weights are adjacent units), or of one part of a parts launch; the grid
  // is units x splits
  const int tv = blockIdx.x;
  const int s = blockIdx.y;
  const int wsel = PAIR ? (tv & 1) : 0;
  int t = PAIR ? (tv >> 1) : tv;
  const int8_t *wbase = wsel ? ep.wq_u : wq;
  const float *sbase = wsel ? ep.wsc_u : wsc;
  TileOut out{y, Npad, (size_t)t * kTile, (size_t)t * kTile, Npad, (unsigned)t};
  Epi uep = ep;
  if constexpr (PARTS) {
    const PartUnit u = part_unit(ep, tv, (int)gridDim.x);
    t = u.t;
    wbase = u.wq;
    sbase = u.wsc;
    out = u.out;
    uep = u.ep;
  }
  int b_lo, b_hi;
  split_range(s, split_q, split_r, b_lo, b_hi);

  // the tile's values and scales; each lane adds its own byte offset
  ValuSrc<MR> src;
  src.wp = wbase + (size_t)t * NB * kChunkBytes;
  src.sp = sbase + (size_t)t * NB * kTile;
  if constexpr (ValuSrc<MR>::kBuf) {
    src.wr = make_buf(src.wp, (unsigned)NB * kChunkBytes);
    src.sr = make_buf(src.sp, (unsigned)NB * kTile * 4);
  }
  src.lw = (unsigned)lane * 16u;
  src.ls = (unsigned)scale_pos(lane) * 4u;

  float acc[MR];
#pragma unroll
  for (int r = 0; r < MR; ++r) acc[r] = 0.0f;

  // Two stages in flight: the next stage's loads are issued before the
  // current stage is computed, so HBM is never idle while the wave computes.
  // Each path issues its prefetch unconditionally just before the compute it
  // overlaps, which lets the compiler wait only for the older stage.
  constexpr int step = W * kUnroll;
  int b = b_lo + wave;
  if (b < b_hi) {
    ValuStage<MR, ACT, DOTS> A, B;
    valu_load<MR, ACT, DOTS, W>(A, src, b, b_hi, xv, m, K, NB, act_scale_off);
    while (true) {
      if (b + step >= b_hi) {
        valu_compute<MR, ACT, DOTS, W>(A, acc, b, b_hi, xv, dots, m, K, NB, Npad, t, lane,
                                       act_scale_off);
        break;
      }
      valu_load<MR, ACT, DOTS, W>(B, src, b + step, b_hi, xv, m, K, NB, act_scale_off);
      valu_compute<MR, ACT, DOTS, W>(A, acc, b, b_hi, xv, dots, m, K, NB, Npad, t, lane,
                                     act_scale_off);
      b += step;
      if (b + step >= b_hi) {
        valu_compute<MR, ACT, DOTS, W>(B, acc, b, b_hi, xv, dots, m, K, NB, Npad, t, lane,
                                       act_scale_off);
        break;
      }
      valu_load<MR, ACT, DOTS, W>(A, src, b + step, b_hi, xv, m, K, NB, act_scale_off);
      valu_compute<MR, ACT, DOTS, W>(B, acc, b, b_hi, xv, dots, m, K, NB, Npad, t, lane,
                                     act_scale_off);
      b += step;
    }
  }
  if constexpr (DOTS) return;

  __shared__ float red[W * MR * 64];
#pragma unroll
  for (int r = 0; r < MR; ++r) red[(wave * MR + r) * 64 + lane] = acc[r];
  __syncthreads();
  finish_tile<MR, W, PAIR>(red, out, partial, counters, m, s, S, wsel, uep);
}

// ---------------------------------------------------------------------------
// the product, MFMA forms: 16x16x32 matrix-core block dots
// ---------------------------------------------------------------------------
//
// One block of one 16-column group is one MFMA per 16 activation rows:
// D[r, c] = sum_{k<32} x[r, 32b+k] * q[32b+k, c], which is exactly the
// per-block dot the method scales, so the scale is still applied once per
// block, on the vector ALU, to D.  The 32-deep K of the instruction is one
// Q8_0 block: blocks with different scales never mix.
//
// Lane l (i = l % 16, quarter j = l / 16) feeds A with row i's k = 8j..8j+7
// and B with column i's k = 8j..8j+7, and receives D rows 4j..4j+3 of
// column i.
//
// Work split.  A wave owns one 16-column group g of a tile; KW waves split
// the blocks of the workgroup's K range between them (wave kw takes blocks
// kw, kw+KW, ...) and meet in LDS at the end of the tile; P groups of 4*KW
// waves ("slots") work on P tiles side by side.  The workgroup's activation
// rows for its K range are staged into LDS once (bf16: 64 B per row and
// block; int8: 32 B plus the fp32 block scale; rows m..MR-1 zero) and serve
// every tile the workgroup then walks through: tiles j*P + slot, stepping by
// G*P over the grid's G workgroups per K split.

// Blocks per stage (two stages in flight): the block-interleaved kernel
// loads four 16-column groups per block, the column-group kernel one.
#ifndef Q8_MFMA_UNROLL
#define Q8_MFMA_UNROLL 1
#endif
#ifndef Q8_COLS_UNROLL
#define Q8_COLS_UNROLL 2
#endif
constexpr int kMfmaUnroll = Q8_MFMA_UNROLL;
constexpr int kColsUnroll = Q8_COLS_UNROLL;

struct ColsStage {
  uint2 w[kColsUnroll];    // 8 values of the lane's column, k = 8j..8j+7
  float sc[kColsUnroll];   // the lane's column scale
};

template <bool DOTS, int KW>
__device__ __forceinline__ void cols_load(ColsStage &st, const int8_t *wcol, const float *scol,
                                          int b0, int b_hi) {
#pragma unroll
  for (int u = 0; u < kColsUnroll; ++u) {
    const int b = min(b0 + u * KW, b_hi - 1);
    st.w[u] = ld_stream8(wcol + (size_t)b * kChunkBytes);
    if constexpr (!DOTS) st.sc[u] = ld_scale4f(scol + (size_t)b * kTile);
  }
}

// The epilogue for the column-group kernel's layout, all loads first:
// v[rg][e][h] (and vu, the gated pair's second sums) is row
// row0 + 16rg + 4j + e, column col0 + 16h + i of lane (i, j); H column groups
// (1 or 2).  On return v holds the final values (final_value's arithmetic).
template <int RG, int H, bool PAIR>
__device__ __forceinline__ void epi_final_groups(const Epi &ep, int Npad, int m, int row0,
                                                 size_t col0, int lane, float (&v)[RG][4][H],
                                                 const float (&vu)[RG][4][H]) {
  const int li = lane & 15, lj = lane >> 4;
  float b[H], bu[H], rv[RG][4][H];
#pragma unroll
  for (int h = 0; h < H; ++h) {
    const size_t col = col0 + 16 * h + li;
    b[h] = (ep.bias && (int)col < ep.N) ? ep.bias[col] : 0.0f;
    bu[h] = (PAIR && ep.bias_u && (int)col < ep.N) ? ep.bias_u[col] : 0.0f;
  }
#pragma unroll
  for (int rg = 0; rg < RG; ++rg)
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int h = 0; h < H; ++h) {
        const int r = row0 + rg * 16 + lj * 4 + e;
        const size_t col = col0 + 16 * h + li;
        rv[rg][e][h] = (!PAIR && ep.residual && r < m) ? ep.residual[(size_t)r * Npad + col]
                                                       : 0.0f;
      }
#pragma unroll
  for (int rg = 0; rg < RG; ++rg)
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int h = 0; h < H; ++h) {
        const size_t col = col0 + 16 * h + li;
        float z = v[rg][e][h];
        if constexpr (PAIR) {
          if (ep.bias) z += b[h];
          float u = vu[rg][e][h];
          if (ep.bias_u) u += bu[h];
          z = silu(z) * u;
        } else {
          if (ep.bias) z += b[h];
          if (ep.residual) z += rv[rg][e][h];
        }
        v[rg][e][h] = ((int)col < ep.N) ? z : 0.0f;
      }
}

// The column-group kernel's partial carries: one record per (split, unit,
// 16-column group) of MR * 16 floats, lane-major: lane l's carries of row
// group rg (rows 16rg + 4j + e, e = 0..3; column 16g + i) are the four floats
// at rg * 256 + 4l, so a wave writes and reads whole 1 KiB runs.
// T: the launch's units.
template <int MR>
__device__ __forceinline__ buf_t cols_record(float *partial, int T, int s, int tv, int g) {
  const size_t rec = ((size_t)s * T + tv) * 4 + g;
  return make_buf(partial + rec * (16 * MR), 16 * MR * 4);
}

// Sums over the S splits (in split order) of unit tv's partial carries for
// v[0][e][h]'s places (row group rg: rows 16rg + 4j + e; column group g0 + h).
// The loads of four splits are issued together (a place past the last split
// reloads the last one, unused); the additions keep split order.
template <int MR, int H>
__device__ __forceinline__ void cols_sum_partials(float *partial, int T, int S, int tv, int g0,
                                                  int rg, int lane, float (&v)[1][4][H]) {
  constexpr int kBatch = 4;
  const unsigned off = (unsigned)(rg * 256 + lane * 4) * 4u;
  for (int s0 = 0; s0 < S; s0 += kBatch) {
    float4 a[kBatch][H];
#pragma unroll
    for (int q = 0; q < kBatch; ++q)
#pragma unroll
      for (int h = 0; h < H; ++h)
        a[q][h] = buf_ld16_sys(cols_record<MR>(partial, T, min(s0 + q, S - 1), tv, g0 + h), off);
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      if (s0 + q >= S) break;
#pragma unroll
      for (int h = 0; h < H; ++h) {
        if (s0 + q == 0) {
          v[0][0][h] = a[q][h].x;
          v[0][1][h] = a[q][h].y;
          v[0][2][h] = a[q][h].z;
          v[0][3][h] = a[q][h].w;
        } else {
          v[0][0][h] += a[q][h].x;
          v[0][1][h] += a[q][h].y;
          v[0][2][h] += a[q][h].z;
          v[0][3][h] += a[q][h].w;
        }
      }
    }
  }
}

// The last arrival's finish of H adjacent 16-column groups (columns col0 +
// 16h + i), one 16-row group at a time (a rolled loop keeps the registers of
// this path below the main loop's): sums of the partials, the epilogue, y,
// and with QUANT the quantized output (H == 2: a row's 32 values are two per
// lane across 16 lanes).
// tv0: the unit of the (first) weight; g0: the first column group, at
// column col0 of y.
template <int RG, int H, bool QUANT, bool PAIR>
__device__ __forceinline__ void cols_finish(const Epi &ep, float *__restrict__ y, float *partial,
                                            int m, int Npad, int T, int S, int tv0, int g0,
                                            size_t col0, int lane) {
  const int li = lane & 15, lj = lane >> 4;
  // The row stride as an opaque value, so the addresses below are formed
  // here and not hoisted into registers held across the caller's main loop.
  asm volatile("" : "+s"(Npad));
#pragma unroll 1
  for (int rg = 0; rg < RG; ++rg) {
    const int row0 = rg * 16;
    if (row0 >= m) break;
    float v[1][4][H], vu[1][4][H];
    cols_sum_partials<RG * 16, H>(partial, T, S, tv0, g0, rg, lane, v);
    if constexpr (PAIR) {
      cols_sum_partials<RG * 16, H>(partial, T, S, tv0 + 1, g0, rg, lane, vu);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int h = 0; h < H; ++h) vu[0][e][h] = 0.0f;
    }
    // every bias and residual value is read before any y is written (the
    // residual may be y itself)
    epi_final_groups<1, H, PAIR>(ep, Npad, m, row0, col0, lane, v, vu);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = row0 + lj * 4 + e;
      if (r >= m) continue;   // uniform over the 16 lanes of one j
      if (ep.write_y) {
#pragma unroll
        for (int h = 0; h < H; ++h) y[(size_t)r * Npad + col0 + 16 * h + li] = v[0][e][h];
      }
      if constexpr (QUANT) {
        static_assert(H == 2, "a quantized block is 32 columns");
        float amax = fmaxf(fabsf(v[0][e][0]), fabsf(v[0][e][1]));
#pragma unroll
        for (int o = 8; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 16));
        const float d = q8_scale_of(amax);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int8_t c = q8_code_of(v[0][e][h], d);
          ep.yq[(size_t)r * Npad + col0 + 16 * h + li] = c;
          ep.yq_view[((col0 / 32) * m + r) * 32 + 16 * h + li] = c;
        }
        if (li == 0) ep.yq_scale[(size_t)r * (Npad / 32) + col0 / 32] = d;
      }
    }
  }
}

// One 16-column group complete in one wave (one split, one weight): the
// epilogue and y (column col0 + i of lane (i, j)).
template <int RG>
__device__ __forceinline__ void cols_store_group(const Epi &ep, float *__restrict__ y, int Npad,
                                                 int m, size_t col0, int lane,
                                                 float (&v)[RG][4][1]) {
  const int li = lane & 15, lj = lane >> 4;
  if (ep.bias || ep.residual || (int)(col0 + 16) > ep.N) {
    float vu[RG][4][1] = {};
    epi_final_groups<RG, 1, false>(ep, Npad, m, 0, col0, lane, v, vu);
  }
  if (!ep.write_y) return;
#pragma unroll
  for (int rg = 0; rg < RG; ++rg)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = rg * 16 + lj * 4 + e;
      if (r < m) y[(size_t)r * Npad + col0 + li] = v[rg][e][0];
    }
}

template <int MR, int ACT, bool DOTS, int KW, int P, bool QO, bool PAIR>
__global__ void __launch_bounds__(256 * KW * P)
gemv_mfma_cols_kernel(const void *__restrict__ xv, const int8_t *__restrict__ wq,
                      const float *__restrict__ wsc, float *__restrict__ y,
                      float *__restrict__ partial, unsigned *__restrict__ counters,
                      int32_t *__restrict__ dots, int m, int K, int NB, int Npad, int T,
                      int S, int split_q, int split_r, int G, int nblk_max,
                      unsigned act_scale_off, Epi ep) {
  constexpr int W = 4 * KW * P;
  constexpr int RG = MR / 16;
  constexpr int kRowBytes = (ACT == kActBf16) ? 64 : 32;   // one row of one block in LDS
  extern __shared__ __attribute__((aligned(16))) char lds[];

  const int lane = threadIdx.x & 63;
  const int li = lane & 15, lj = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = wave & 3;
  const int kw = (wave >> 2) % KW;
  const int slot = wave / (4 * KW);
  const int s = blockIdx.y;
  const int jwg = blockIdx.x;
  int b_lo, b_hi;
  split_range(s, split_q, split_r, b_lo, b_hi);
  const int nblk = b_hi - b_lo;
  const int col_in_tile = 16 * g + li;
  // lane's bytes in a chunk: half j/2, column 16g+i, k offset 8*(j%2)
  const size_t lane_off = (size_t)(lj >> 1) * kHalfBytes + (size_t)col_in_tile * 16 + (lj & 1) * 8;

  constexpr int step = KW * kColsUnroll;
  // Units tv = (tile, weight), T of them: a gated pair's two weights are
  // adjacent units.
  constexpr bool pair = PAIR;
  constexpr int NW = PAIR ? 2 : 1;
  const int tv0 = jwg * P + slot;
  ColsStage A, B;
  // First stage of the first tile in flight while the activation is staged.
  if (tv0 < T && b_lo + kw < b_hi) {
    const int t0 = pair ? tv0 >> 1 : tv0, w0 = pair ? (tv0 & 1) : 0;
    cols_load<DOTS, KW>(A, (w0 ? ep.wq_u : wq) + (size_t)t0 * NB * kChunkBytes + lane_off,
                        (w0 ? ep.wsc_u : wsc) + (size_t)t0 * NB * kTile + scale_pos(col_in_tile),
                        b_lo + kw, b_hi);
  }

  stage_activation<MR, ACT, 64 * W>(lds, xv, m, K, NB, b_lo, nblk, act_scale_off);
  __syncthreads();
  const float *dxs = reinterpret_cast<const float *>(lds + (size_t)nblk * MR * kRowBytes);
  float *red = reinterpret_cast<float *>(lds + mfma_stage_bytes(MR, ACT, nblk_max));

  for (int tv = tv0; tv < T; tv += G * P) {
    const int t = pair ? tv >> 1 : tv, wsel = pair ? (tv & 1) : 0;
    const int8_t *wcol = (wsel ? ep.wq_u : wq) + (size_t)t * NB * kChunkBytes + lane_off;
    const float *scol = (wsel ? ep.wsc_u : wsc) + (size_t)t * NB * kTile + scale_pos(col_in_tile);
    f32x4_t acc[RG];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) acc[rg] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    auto compute = [&](const ColsStage &st, int b0) {
#pragma unroll
      for (int u = 0; u < kColsUnroll; ++u) {
        const int bb = b0 + u * KW;
        if (bb >= b_hi) break;
        const int lb = bb - b_lo;
        if constexpr (ACT == kActBf16) {
          const bf16x8_t bw = i8x8_to_bf16(st.w[u]);
#pragma unroll
          for (int rg = 0; rg < RG; ++rg) {
            const bf16x8_t a = *reinterpret_cast<const bf16x8_t *>(
                lds + ((size_t)lb * MR + rg * 16 + li) * kRowBytes + lj * 16);
            const f32x4_t d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                a, bw, f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[rg][e] = fmaf(st.sc[u], d[e], acc[rg][e]);
          }
        } else {
          const long bw = __builtin_bit_cast(long, st.w[u]);
#pragma unroll
          for (int rg = 0; rg < RG; ++rg) {
            const long a = *reinterpret_cast<const long *>(
                lds + ((size_t)lb * MR + rg * 16 + li) * kRowBytes + lj * 8);
            const i32x4_t d = __builtin_amdgcn_mfma_i32_16x16x32_i8(a, bw, i32x4_t{0, 0, 0, 0},
                                                                   0, 0, 0);
            if constexpr (DOTS) {
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int r = rg * 16 + lj * 4 + e;
                if (r < m)
                  dots[((size_t)r * NB + bb) * Npad + (size_t)t * kTile + col_in_tile] = d[e];
              }
            } else {
              const float4 dx4 =
                  *reinterpret_cast<const float4 *>(dxs + (size_t)lb * MR + rg * 16 + lj * 4);
              const float dxv[4] = {dx4.x, dx4.y, dx4.z, dx4.w};
#pragma unroll
              for (int e = 0; e < 4; ++e)
                acc[rg][e] = fmaf(dxv[e] * st.sc[u], (float)d[e], acc[rg][e]);
            }
          }
        }
      }
    };

    int b = b_lo + kw;
    if (b < b_hi) {
      if (tv != tv0)   // the first tile's first stage is already in flight
        cols_load<DOTS, KW>(A, wcol, scol, b, b_hi);
      // One compute site: the next stage is loaded into B while A is
      // computed, then copied into A (the copy waits for B, which the next
      // compute needs anyway).
      while (true) {
        if (b + step >= b_hi) {
          compute(A, b);
          break;
        }
        cols_load<DOTS, KW>(B, wcol, scol, b + step, b_hi);
        __builtin_amdgcn_sched_barrier(0);   // keep the prefetch ahead of the compute
        compute(A, b);
        A = B;
        b += step;
      }
    }
    if constexpr (DOTS) continue;

    if constexpr (KW > 1) {
      // The KW waves of a column group meet in LDS, summed in kw order.
#pragma unroll
      for (int rg = 0; rg < RG; ++rg)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          red[(kw * MR + rg * 16 + lj * 4 + e) * 64 + col_in_tile] = acc[rg][e];
      __syncthreads();
      if (kw == 0) {
#pragma unroll
        for (int rg = 0; rg < RG; ++rg)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float v = acc[rg][e];
#pragma unroll
            for (int w2 = 1; w2 < KW; ++w2) v += red[(w2 * MR + rg * 16 + lj * 4 + e) * 64 + col_in_tile];
            acc[rg][e] = v;
          }
      }
      __syncthreads();   // red is free again for the next tile
      if (kw != 0) continue;
    }

    // This wave's 16 columns are final for its split and weight: store, or
    // publish the partial and let the last arrival sum the partials in split
    // order (the protocol of finish_tile, per 16-column group, inside one
    // wave).
    const size_t col = (size_t)t * kTile + col_in_tile;
    const int arrivals = S * NW;
    if (arrivals == 1) {
      float v[RG][4][1];
#pragma unroll
      for (int rg = 0; rg < RG; ++rg)
#pragma unroll
        for (int e = 0; e < 4; ++e) v[rg][e][0] = acc[rg][e];
      cols_store_group<RG>(ep, y, Npad, m, col - li, lane, v);
      continue;
    }
    {
      const buf_t rec = cols_record<MR>(partial, T, s, tv, g);
#pragma unroll
      for (int rg = 0; rg < RG; ++rg)
        buf_st16_sys(rec, (unsigned)(rg * 256 + lane * 4) * 4u,
                     make_float4(acc[rg][0], acc[rg][1], acc[rg][2], acc[rg][3]));
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    // The output quantizer's 32-column blocks span the column-group pair
    // (g & 2, g | 1): then the pair shares one counter and the last of its
    // arrivals finishes all 32 columns.
    unsigned *counter = counters + (size_t)t * 4 + (QO ? (g & 2) : g);
    const unsigned last = (unsigned)(arrivals * (QO ? 2 : 1) - 1);
    unsigned prev = 0;
    if (lane == 0)
      prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    prev = __builtin_amdgcn_readfirstlane(prev);
    if (prev != last) continue;
    const int tv0 = pair ? (tv & ~1) : tv;   // the unit of the pair's first weight
    if constexpr (QO) {
      cols_finish<RG, 2, true, PAIR>(ep, y, partial, m, Npad, T, S, tv0, g & 2,
                                     (size_t)t * kTile + 16 * (g & 2), lane);
    } else if constexpr (PAIR) {
      cols_finish<RG, 1, false, true>(ep, y, partial, m, Npad, T, S, tv0, g, col - li, lane);
    } else {
      // one weight, no quantizer: the split sums in place (this form keeps
      // the main loop's register allocation of the plain build)
      float v[RG][4][1];
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) {
        float w[1][4][1];
        cols_sum_partials<MR, 1>(partial, T, S, tv, g, rg, lane, w);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[rg][e][0] = w[0][e][0];
      }
      cols_store_group<RG>(ep, y, Npad, m, col - li, lane, v);
    }
    if (lane == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  }
}

// ---------------------------------------------------------------------------
// the product, MFMA form with block-interleaved waves
// ---------------------------------------------------------------------------
//
// Every wave covers all 64 columns of the tile (four 16-column MFMAs per row
// group and block) and the W waves split the blocks of the workgroup's K range
// (wave w takes blocks w, w+W, ...), so one activation fragment read from LDS
// serves four MFMAs.  The carries of the W waves meet in LDS at the end of
// each tile.  The activation rows of the workgroup's K range are staged once
// and serve every tile the workgroup walks through (tiles j, j+G, ...).

struct MfmaStage {
  uint2 w[kMfmaUnroll][4];   // 8 values of column 16g + i, k = 8j..8j+7
  float4 sc[kMfmaUnroll];    // scales of columns i + 16g, g = 0..3
};

template <bool DOTS, int W>
__device__ __forceinline__ void mfma_load(MfmaStage &st, const int8_t *wlane,
                                          const float4 *slane, int b0, int b_hi) {
#pragma unroll
  for (int u = 0; u < kMfmaUnroll; ++u) {
    const int b = min(b0 + u * W, b_hi - 1);
    const int8_t *c = wlane + (size_t)b * kChunkBytes;
#pragma unroll
    for (int g = 0; g < 4; ++g) st.w[u][g] = ld_stream8(c + g * 256);
    if constexpr (!DOTS) st.sc[u] = ld_scale16f(slane + (size_t)b * (kTile / 4));
  }
}

template <int MR, int ACT, bool DOTS, int W, bool PAIR, bool PARTS>
__global__ void __launch_bounds__(64 * W)
gemv_mfma_kernel(const void *__restrict__ xv, const int8_t *__restrict__ wq,
                 const float *__restrict__ wsc, float *__restrict__ y,
                 float *__restrict__ partial, unsigned *__restrict__ counters,
                 int32_t *__restrict__ dots, int m, int K, int NB, int Npad, int T,
                 int S, int split_q, int split_r, int G, int nblk_max, int red_on_stage,
                 unsigned act_scale_off, Epi ep) {
  constexpr int RG = MR / 16;
  constexpr int kRowBytes = (ACT == kActBf16) ? 64 : 32;
  extern __shared__ __attribute__((aligned(16))) char lds[];

  const int lane = threadIdx.x & 63;
  const int li = lane & 15, lj = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int s = blockIdx.y;
  const int jwg = blockIdx.x;
  int b_lo, b_hi;
  split_range(s, split_q, split_r, b_lo, b_hi);
  const int nblk = b_hi - b_lo;
  // lane's bytes in a chunk: half j/2, column i (+16g), k offset 8*(j%2)
  const size_t lane_off = (size_t)(lj >> 1) * kHalfBytes + li * 16 + (lj & 1) * 8;

  // Units tv, T of them: the product's tiles, the parts' tiles side by side,
  // or the gated pair's output tiles, whose two weights the workgroup's two
  // halves of waves stream together (waves 0 .. W/2-1 the gate, the rest the
  // up weight), so the pair meets in LDS.  WH waves split each weight's
  // blocks.
  constexpr int WH = PAIR ? W / 2 : W;
  const int wsel_w = PAIR ? wave / WH : 0;   // the weight this wave streams
  const int wave_in = PAIR ? wave - wsel_w * WH : wave;
  constexpr int step = WH * kMfmaUnroll;
  MfmaStage A, B;
  // unit tv's weight and scales (for this wave), and its tile within its
  // product
  auto unit_src = [&](int tv, const int8_t *&wb, const float *&sb, int &tt) {
    if constexpr (PARTS) {
      const int p = part_of(ep.parts, tv);
      tt = tv - ep.parts.cum[p];
      wb = ep.parts.wq[p];
      sb = ep.parts.wsc[p];
    } else {
      tt = tv;
      wb = wsel_w ? ep.wq_u : wq;
      sb = wsel_w ? ep.wsc_u : wsc;
    }
  };
  if (jwg < T && b_lo + wave_in < b_hi) {
    const int8_t *wb;
    const float *sb;
    int t0;
    unit_src(jwg, wb, sb, t0);
    mfma_load<DOTS, WH>(A, wb + (size_t)t0 * NB * kChunkBytes + lane_off,
                        reinterpret_cast<const float4 *>(sb + (size_t)t0 * NB * kTile) + li,
                        b_lo + wave_in, b_hi);
  }
  stage_activation<MR, ACT, 64 * W>(lds, xv, m, K, NB, b_lo, nblk, act_scale_off);
  __syncthreads();
  const float *dxs = reinterpret_cast<const float *>(lds + (size_t)nblk * MR * kRowBytes);
  // The carries' area: after the stage, or (when every workgroup has at most
  // one tile, G >= T) on top of the stage, which is no longer read by then.
  float *red = reinterpret_cast<float *>(
      lds + (red_on_stage ? (size_t)0 : mfma_stage_bytes(MR, ACT, nblk_max)));

  for (int tv = jwg; tv < T; tv += G) {
    const int8_t *wb;
    const float *sb;
    int t;
    unit_src(tv, wb, sb, t);
    const int8_t *wlane = wb + (size_t)t * NB * kChunkBytes + lane_off;
    const float4 *slane = reinterpret_cast<const float4 *>(sb + (size_t)t * NB * kTile) + li;
    f32x4_t acc[RG][4];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
      for (int g = 0; g < 4; ++g) acc[rg][g] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    auto compute = [&](const MfmaStage &st, int b0) {
#pragma unroll
      for (int u = 0; u < kMfmaUnroll; ++u) {
        const int bb = b0 + u * WH;
        if (bb >= b_hi) break;
        const int lb = bb - b_lo;
        if constexpr (ACT == kActBf16) {
          bf16x8_t a[RG];
#pragma unroll
          for (int rg = 0; rg < RG; ++rg)
            a[rg] = *reinterpret_cast<const bf16x8_t *>(
                lds + ((size_t)lb * MR + rg * 16 + li) * kRowBytes + lj * 16);
          const float scs[4] = {st.sc[u].x, st.sc[u].y, st.sc[u].z, st.sc[u].w};
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const bf16x8_t bw = i8x8_to_bf16(st.w[u][g]);
#pragma unroll
            for (int rg = 0; rg < RG; ++rg) {
              const f32x4_t d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  a[rg], bw, f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
#pragma unroll
              for (int e = 0; e < 4; ++e) acc[rg][g][e] = fmaf(scs[g], d[e], acc[rg][g][e]);
            }
          }
        } else if constexpr (ACT == kActQ8x2) {
          // First words in rows 0-15, second words in rows 16-31: one int8
          // MFMA each, and the two passes' dots meet exactly in int32
          // (|128 D_hi + D_lo| <= 128 * 516128 + 64 * 127 * 32 < 2^27).
          const long ahi = *reinterpret_cast<const long *>(
              lds + ((size_t)lb * MR + li) * kRowBytes + lj * 8);
          const long alo = *reinterpret_cast<const long *>(
              lds + ((size_t)lb * MR + 16 + li) * kRowBytes + lj * 8);
          const float4 dx4 = *reinterpret_cast<const float4 *>(dxs + (size_t)lb * MR + lj * 4);
          const float dxv[4] = {dx4.x, dx4.y, dx4.z, dx4.w};
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const long bw = __builtin_bit_cast(long, st.w[u][g]);
            const i32x4_t dh =
                __builtin_amdgcn_mfma_i32_16x16x32_i8(ahi, bw, i32x4_t{0, 0, 0, 0}, 0, 0, 0);
            const i32x4_t dl =
                __builtin_amdgcn_mfma_i32_16x16x32_i8(alo, bw, i32x4_t{0, 0, 0, 0}, 0, 0, 0);
            const float scg = (g == 0) ? st.sc[u].x : (g == 1) ? st.sc[u].y
                            : (g == 2) ? st.sc[u].z : st.sc[u].w;
#pragma unroll
            for (int e = 0; e < 4; ++e)
              acc[0][g][e] = fmaf(dxv[e] * scg, (float)(dh[e] * 128 + dl[e]) * 0.0078125f,
                                  acc[0][g][e]);
          }
        } else {
          long a[RG];
          float4 dx4[RG];
#pragma unroll
          for (int rg = 0; rg < RG; ++rg) {
            a[rg] = *reinterpret_cast<const long *>(
                lds + ((size_t)lb * MR + rg * 16 + li) * kRowBytes + lj * 8);
            if constexpr (!DOTS)
              dx4[rg] = *reinterpret_cast<const float4 *>(dxs + (size_t)lb * MR + rg * 16 + lj * 4);
          }
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const long bw = __builtin_bit_cast(long, st.w[u][g]);
#pragma unroll
            for (int rg = 0; rg < RG; ++rg) {
              const i32x4_t d = __builtin_amdgcn_mfma_i32_16x16x32_i8(
                  a[rg], bw, i32x4_t{0, 0, 0, 0}, 0, 0, 0);
              if constexpr (DOTS) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  const int r = rg * 16 + lj * 4 + e;
                  if (r < m)
                    dots[((size_t)r * NB + bb) * Npad + (size_t)t * kTile + g * 16 + li] = d[e];
                }
              } else {
                const float scg = (g == 0) ? st.sc[u].x : (g == 1) ? st.sc[u].y
                                : (g == 2) ? st.sc[u].z : st.sc[u].w;
                const float dxv[4] = {dx4[rg].x, dx4[rg].y, dx4[rg].z, dx4[rg].w};
#pragma unroll
                for (int e = 0; e < 4; ++e)
                  acc[rg][g][e] = fmaf(dxv[e] * scg, (float)d[e], acc[rg][g][e]);
              }
            }
          }
        }
      }
    };

    int b = b_lo + wave_in;
    if (b < b_hi) {
      if (tv != jwg) mfma_load<DOTS, WH>(A, wlane, slane, b, b_hi);
      // One compute site: the next stage is loaded into B while A is
      // computed, then copied into A (the copy waits for B, which the next
      // compute needs anyway).
      while (true) {
        if (b + step >= b_hi) {
          compute(A, b);
          break;
        }
        mfma_load<DOTS, WH>(B, wlane, slane, b + step, b_hi);
        __builtin_amdgcn_sched_barrier(0);   // keep the prefetch ahead of the compute
        compute(A, b);
        A = B;
        b += step;
      }
    }
    if constexpr (DOTS) continue;

    // The W waves meet in LDS, then the tile is stored (or its split-K
    // partial published and combined by the last split to arrive).
    if (red_on_stage) __syncthreads();   // every wave is done reading the stage
    // the two-word form carries its rows in the first row group only
    constexpr int kOutRG = ACT == kActQ8x2 ? 1 : RG;
#pragma unroll
    for (int rg = 0; rg < kOutRG; ++rg)
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          red[(wave * MR + rg * 16 + lj * 4 + e) * 64 + g * 16 + li] = acc[rg][g][e];
    __syncthreads();
    if constexpr (PARTS) {
      const PartUnit u = part_unit(ep, tv, T);
      finish_tile<MR, W, false>(red, u.out, partial, counters, m, s, S, 0, u.ep);
    } else if constexpr (PAIR) {
      finish_pair_tile<MR, W>(red, TileOut{y, Npad, (size_t)t * kTile, (size_t)t * kTile, Npad,
                                           (unsigned)t},
                              partial, counters, m, s, S, ep);
    } else {
      finish_tile<MR, W, false>(red, TileOut{y, Npad, (size_t)t * kTile, (size_t)t * kTile, Npad,
                                             (unsigned)t},
                                partial, counters, m, s, S, 0, ep);
    }
    __syncthreads();   // red is free again for the next tile
  }
}

// Dynamic LDS bytes of a block-interleaved MFMA launch: the staged activation
// of the largest split and the W waves' carries of one tile, the carries
// either after the stage or (one tile per workgroup) on top of it.
size_t mfma_stage_of(int rows, int act, int NB, int S) {
  return mfma_stage_bytes(rows, act, (NB + S - 1) / S);
}
size_t mfma_red_of(int rows, int waves) { return (size_t)waves * rows * 64 * 4; }
size_t mfma_lds_bytes_of(int rows, int act, int waves, int NB, int S) {
  // the smaller form; the launch takes the larger one when it fits and pays
  const size_t st = mfma_stage_of(rows, act, NB, S), rd = mfma_red_of(rows, waves);
  return st > rd ? st : rd;
}

// Dynamic LDS bytes of a column-group MFMA launch: the staged activation of
// the largest split, plus the KW-way carries of a tile when KW > 1.
size_t cols_lds_bytes_of(int rows, int act, int kslices, int NB, int S) {
  const int nblk = (NB + S - 1) / S;
  const size_t red = kslices > 1 ? (size_t)kslices * rows * 64 * 4 : 0;
  return mfma_stage_bytes(rows, act, nblk) + red;
}

template <int MR, int ACT, bool DOTS, int W, bool PAIR, bool PARTS>
hipError_t launch_valu_k(const GemvArgs &a, hipStream_t stream) {
  const dim3 grid((unsigned)a.tiles(), (unsigned)a.split_k);
  gemv_valu_kernel<MR, ACT, DOTS, W, PAIR, PARTS><<<grid, dim3(64 * W), 0, stream>>>(
      a.x, a.wq, a.wsc, a.y, a.partial, a.counters, a.dots, a.m, a.K, a.NB,
      a.Npad, a.split_k, a.NB / a.split_k, a.NB % a.split_k, a.act_scale_off, a.ep);
  return hipGetLastError();
}

// Each kernel is built for one weight and for the gated pair, so the single
// product carries none of the pair's code.
template <int MR, int ACT, bool DOTS, int W>
hipError_t launch_valu(const GemvArgs &a, hipStream_t stream) {
  if constexpr (!DOTS) {
    if (a.ep.nw == 2) return launch_valu_k<MR, ACT, DOTS, W, true, false>(a, stream);
    if (a.ep.parts.n > 0) return launch_valu_k<MR, ACT, DOTS, W, false, true>(a, stream);
  }
  return launch_valu_k<MR, ACT, DOTS, W, false, false>(a, stream);
}

template <int MR, int ACT, bool DOTS, int W, bool PAIR, bool PARTS>
hipError_t launch_mfma_k(const GemvArgs &a, hipStream_t stream) {
  const int nblk_max = (a.NB + a.split_k - 1) / a.split_k;
  const size_t st = mfma_stage_of(MR, ACT, a.NB, a.split_k), rd = mfma_red_of(MR, W);
  const size_t lds_alias = st > rd ? st : rd;   // carries on top of the stage
  const size_t lds_sep = st + rd;               // carries after the stage
  auto kern = gemv_mfma_kernel<MR, ACT, DOTS, W, PAIR, PARTS>;
  static size_t granted = 64 * 1024;
  int dev = 0, max_lds = 0;
  (void)hipGetDevice(&dev);
  if (hipDeviceGetAttribute(&max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) !=
      hipSuccess)
    max_lds = 64 * 1024;
  // One tile per workgroup when all of them fit on the device at once (the
  // carries then reuse the stage); otherwise a persistent grid that stages
  // once and walks tiles j, j+G, ... (carries apart), if that fits in LDS.
  hipError_t e = grant_lds(kern, lds_alias, granted);
  if (e != hipSuccess) return e;
  // units: output tiles (the pair's two weights share a workgroup)
  const int units = PAIR ? a.T : a.tiles();
  int G = units, red_on_stage = 1;
  size_t lds = lds_alias;
  const int fit_alias = resident_workgroups(kern, 64 * W, lds_alias) / a.split_k;
  if (fit_alias < units && lds_sep + 1024 <= (size_t)max_lds) {
    e = grant_lds(kern, lds_sep, granted);
    if (e != hipSuccess) return e;
    G = balanced_grid(resident_workgroups(kern, 64 * W, lds_sep) / a.split_k, units);
    red_on_stage = 0;
    lds = lds_sep;
  }
  (void)hipGetLastError();
  kern<<<dim3((unsigned)G, (unsigned)a.split_k), dim3(64 * W), lds, stream>>>(
      a.x, a.wq, a.wsc, a.y, a.partial, a.counters, a.dots, a.m, a.K, a.NB, a.Npad, units,
      a.split_k, a.NB / a.split_k, a.NB % a.split_k, G, nblk_max, red_on_stage,
      a.act_scale_off, a.ep);
  return hipGetLastError();
}

template <int MR, int ACT, bool DOTS, int W>
hipError_t launch_mfma(const GemvArgs &a, hipStream_t stream) {
  if constexpr (!DOTS) {
    if (a.ep.nw == 2) return launch_mfma_k<MR, ACT, DOTS, W, true, false>(a, stream);
    if (a.ep.parts.n > 0) return launch_mfma_k<MR, ACT, DOTS, W, false, true>(a, stream);
  }
  return launch_mfma_k<MR, ACT, DOTS, W, false, false>(a, stream);
}

template <int MR, int ACT, bool DOTS, int KW, int P, bool QO, bool PAIR>
hipError_t launch_cols_k(const GemvArgs &a, hipStream_t stream) {
  constexpr int W = 4 * KW * P;
  const int nblk_max = (a.NB + a.split_k - 1) / a.split_k;
  const size_t lds = cols_lds_bytes_of(MR, ACT, KW, a.NB, a.split_k);
  auto kern = gemv_mfma_cols_kernel<MR, ACT, DOTS, KW, P, QO, PAIR>;
  static size_t granted = 64 * 1024;
  hipError_t e = grant_lds(kern, lds, granted);
  if (e != hipSuccess) return e;
  // G workgroups per K split, each walking tiles j*P + slot, step G*P.
  const int want = (a.tiles() + P - 1) / P;
  const int G = balanced_grid(resident_workgroups(kern, 64 * W, lds) / a.split_k, want);
  (void)hipGetLastError();
  kern<<<dim3((unsigned)G, (unsigned)a.split_k), dim3(64 * W), lds, stream>>>(
      a.x, a.wq, a.wsc, a.y, a.partial, a.counters, a.dots, a.m, a.K, a.NB, a.Npad, a.tiles(),
      a.split_k, a.NB / a.split_k, a.NB % a.split_k, G, nblk_max, a.act_scale_off, a.ep);
  return hipGetLastError();
}

// The column-group kernel is built with and without the output quantizer
// in its split-K finish, and for one weight or the gated pair: each build
// keeps only the registers its own finish needs (the main loop runs at the
// register limit of 16 waves).
template <int MR, int ACT, bool DOTS, int KW, int P>
hipError_t launch_cols(const GemvArgs &a, hipStream_t stream) {
  if constexpr (!DOTS) {
    const bool qo = a.ep.yq != nullptr, pair = a.ep.nw == 2;
    if (qo && pair) return launch_cols_k<MR, ACT, DOTS, KW, P, true, true>(a, stream);
    if (qo) return launch_cols_k<MR, ACT, DOTS, KW, P, true, false>(a, stream);
    if (pair) return launch_cols_k<MR, ACT, DOTS, KW, P, false, true>(a, stream);
  }
  return launch_cols_k<MR, ACT, DOTS, KW, P, false, false>(a, stream);
}

using Launcher = hipError_t (*)(const GemvArgs &, hipStream_t);

// VALU instantiations: 16 waves up to 4 rows, 8 waves up to 8 rows (more rows
// would exceed the VGPRs the larger workgroups allow), 4 waves for any row count.
template <int ACT, bool DOTS, int W>
Launcher pick_valu_rows(int rows) {
  switch (rows) {
    case 1: return &launch_valu<1, ACT, DOTS, W>;
    case 2: return &launch_valu<2, ACT, DOTS, W>;
    case 4: return &launch_valu<4, ACT, DOTS, W>;
    default: break;
  }
  if constexpr (W <= 8) {
    if (rows == 8) return &launch_valu<8, ACT, DOTS, W>;
  }
  if constexpr (W <= 4) {
    if (rows == 16) return &launch_valu<16, ACT, DOTS, W>;
    if (rows == 32) return &launch_valu<32, ACT, DOTS, W>;
  }
  return nullptr;
}

template <int ACT, bool DOTS, int W>
Launcher pick_mfma_rows(int rows) {
  switch (rows) {
    case 16: return &launch_mfma<16, ACT, DOTS, W>;
    case 32: return &launch_mfma<32, ACT, DOTS, W>;
    default: return nullptr;
  }
}

template <int W>
Launcher pick_mfma(int rows, int act, bool dots) {
  if (act == kActBf16) return dots ? nullptr : pick_mfma_rows<kActBf16, false, W>(rows);
  if (act == kActQ8)
    return dots ? pick_mfma_rows<kActQ8, true, W>(rows) : pick_mfma_rows<kActQ8, false, W>(rows);
  // two words: the first words fill rows 0-15 and the second rows 16-31
  if (act == kActQ8x2 && !dots && rows == 32) return &launch_mfma<32, kActQ8x2, false, W>;
  return nullptr;
}

// Column-group MFMA instantiations: (k-slices, tile slots) in {(1,1), (1,2),
// (1,4), (2,1), (4,1)}, i.e. 4, 8 or 16 waves.
template <int ACT, bool DOTS, int KW, int P>
Launcher pick_cols_rows(int rows) {
  switch (rows) {
    case 16: return &launch_cols<16, ACT, DOTS, KW, P>;
    case 32: return &launch_cols<32, ACT, DOTS, KW, P>;
    default: return nullptr;
  }
}

template <int KW, int P>
Launcher pick_cols(int rows, int act, bool dots) {
  if (act == kActBf16) return dots ? nullptr : pick_cols_rows<kActBf16, false, KW, P>(rows);
  if (act == kActQ8)
    return dots ? pick_cols_rows<kActQ8, true, KW, P>(rows)
                : pick_cols_rows<kActQ8, false, KW, P>(rows);
  return nullptr;
}

template <int W>
Launcher pick_valu(int rows, int act, bool dots) {
  if (act == kActBf16) return dots ? nullptr : pick_valu_rows<kActBf16, false, W>(rows);
  if (act == kActQ8)
    return dots ? pick_valu_rows<kActQ8, true, W>(rows) : pick_valu_rows<kActQ8, false, W>(rows);
  // two words: up to 4 rows (two sdot4 passes per block and row)
  if (act == kActQ8x2 && !dots) {
    switch (rows) {
      case 1: return &launch_valu<1, kActQ8x2, false, W>;
      case 2: return &launch_valu<2, kActQ8x2, false, W>;
      case 4: return &launch_valu<4, kActQ8x2, false, W>;
      default: return nullptr;
    }
  }
  return nullptr;
}

Launcher pick(int kernel, int rows, int act, bool dots, int waves, int kslices) {
  if (kernel == 0) {
    switch (waves) {
      case 4: return pick_valu<4>(rows, act, dots);
      case 8: return pick_valu<8>(rows, act, dots);
      case 16: return pick_valu<16>(rows, act, dots);
      default: return nullptr;
    }
  }
  if (kernel == 1) {
    switch (waves) {
      case 4: return pick_mfma<4>(rows, act, dots);
      case 8: return pick_mfma<8>(rows, act, dots);
      case 16: return pick_mfma<16>(rows, act, dots);
      default: return nullptr;
    }
  }
  if (kernel == 2) {
    if (waves == 4 && kslices == 1) return pick_cols<1, 1>(rows, act, dots);
    if (waves == 8 && kslices == 1) return pick_cols<1, 2>(rows, act, dots);
    if (waves == 16 && kslices == 1) return pick_cols<1, 4>(rows, act, dots);
    if (waves == 8 && kslices == 2) return pick_cols<2, 1>(rows, act, dots);
    if (waves == 16 && kslices == 4) return pick_cols<4, 1>(rows, act, dots);
  }
  return nullptr;
}

unsigned blocks_for(long long n) { return (unsigned)((n + 255) / 256); }

// Values a thread of the activation quantizer takes (measured at its kernel).
constexpr int kQuantizeE = 4;

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
                               size_t scale_off, size_t view_off, hipStream_t stream) {
  int8_t *xq = static_cast<int8_t *>(x_q8);
  float *dx = reinterpret_cast<float *>(static_cast<char *>(x_q8) + scale_off);
  int8_t *xv = static_cast<int8_t *>(x_q8) + view_off;
  quantize_act_vec_kernel<kQuantizeE><<<dim3(blocks_for(K / kQuantizeE), (unsigned)m), 256, 0,
                                          stream>>>(x, xq, dx, xv, m, K);
  return hipGetLastError();
}

hipError_t launch_quantize_act_two_words(const uint16_t *x, void *x_q8x2, int m, int K,
                                         unsigned scale_off, hipStream_t stream) {
  const long long total = (long long)m * K;
  int8_t *hi = static_cast<int8_t *>(x_q8x2);
  int8_t *lo = hi + total;
  float *dx = reinterpret_cast<float *>(static_cast<char *>(x_q8x2) + scale_off);
  quantize_act_two_words_kernel<<<blocks_for(total), 256, 0, stream>>>(x, hi, lo, dx, total);
  return hipGetLastError();
}

size_t gemv_lds_bytes(int kernel, int rows, int act, int waves, int kslices, int NB,
                      int split_k) {
  if (kernel == 1) return mfma_lds_bytes_of(rows, act, waves, NB, split_k);
  if (kernel >= 3 && kernel <= 5) return mfma32_lds_bytes(kernel, waves, kslices, NB, split_k);
  if (kernel == 6) return tile16_lds_bytes(rows, act, waves, NB, split_k);
  if (kernel == 2) return cols_lds_bytes_of(rows, act, kslices, NB, split_k);
  return 0;
}

bool gemv_instantiated(int kernel, int rows, int act, bool write_dots, int waves, int kslices) {
  if (kernel >= 3 && kernel <= 5)
    return mfma32_instantiated(kernel, rows, act, write_dots, waves, kslices);
  if (kernel == 6) return tile16_instantiated(rows, act, write_dots, waves, kslices);
  return pick(kernel, rows, act, write_dots, waves, kslices) != nullptr;
}

hipError_t launch_gemv(int kernel, int rows, int act, bool write_dots, int waves, int kslices,
                       const GemvArgs &a, hipStream_t stream) {
  if (kernel >= 3 && kernel <= 5) {
    if (!mfma32_instantiated(kernel, rows, act, write_dots, waves, kslices))
      return hipErrorInvalidValue;
    return launch_gemv_mfma32(kernel, waves, kslices, write_dots, a, stream);
  }
  if (kernel == 6) {
    if (!tile16_instantiated(rows, act, write_dots, waves, kslices)) return hipErrorInvalidValue;
    return launch_gemv_tile16(rows, act, waves, kslices, write_dots, a, stream);
  }
  Launcher f = pick(kernel, rows, act, write_dots, waves, kslices);
  if (!f) return hipErrorInvalidValue;
  return f(a, stream);
}

}  // namespace q8
