// q8_mfma32.hip -- the product for 17-32 rows of a Q8_0 activation on the
// 32x32x32 int8 matrix core.
//
// The product (docs.logicaffeine.com, logicaffeine_compile/spatial/passes/
// from_q8.rs, module doc and fn q8_fold): per Q8_0 block b the exact int32
// dot D[r,n] = sum_i xq[r,32b+i] * q[32b+i,n], scaled once by the block's
// scales and folded into an fp32 carry.  One v_mfma_i32_32x32x32_i8 is
// exactly that dot for 32 rows and 32 columns of one block: its K of 32 is
// one Q8_0 block, so blocks with different scales never mix in the matrix
// core, and the scale is applied once per block to D on the vector ALU
// (acc = fma(dx[r,b] * s[b,n], float(D), acc); D is exact in fp32).
//
// Operand mapping (lane l, h = l / 32, j = l % 32):
//   A (activation): row j, k = 16h .. 16h+15 of the block -- 16 bytes of the
//     staged rows in LDS;
//   B (weight): column j of the 32-column group, k = 16h .. 16h+15 -- in the
//     packed layout that is 16 bytes at half h, column j: the two groups of a
//     64-column tile are two 16-byte loads per lane, and each load
//     instruction reads two whole 512-byte runs (a wave reads the block's
//     2 KiB chunk in two instructions);
//   D: element v of lane l is row 8(v/4) + 4h + v%4, column j.
//
// Work split: a workgroup of W = KW * P waves works on P tiles side by side;
// the KW waves of a tile split the blocks of the workgroup's K range (wave kw
// takes blocks kw, kw+KW, ...).  The activation rows of the K range are
// staged into LDS once and serve every tile the workgroup walks (tile groups
// j, j+G, ...).  A tile's KW carries meet in LDS in kw order; its first wave
// then finishes the tile from registers: the epilogue and y, or the split-K
// partial published as a lane-major record, the last of the tile's S
// arrivals summing the records in split order (the protocol of the other
// product kernels: write-through stores, completion awaited, a system-scope
// arrival counter; no device-scope fence).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q8_device.h"
#include "q8_internal.h"
#include "q8_product.h"

namespace q8 {
namespace {

using namespace dev;

typedef __attribute__((ext_vector_type(16))) int i32x16_t;
typedef __attribute__((ext_vector_type(4))) int i32x4v_t;

template <int U, bool AG>
struct M32Stage {
  uint4 w0[U], w1[U];   // 16 values of columns j and 32 + j, k = 16h .. 16h+15
  float s0[U], s1[U];   // their scales
  uint4 a[AG ? U : 1];  // direct form: the activation fragment (row j, k = 16h ..)
};

// Place of row r's scale of block lb in the stage below: [block][row], the
// row's group of four (r / 4) stored at group (r / 4) ^ (lb % 8).  The
// stage's writes go down a column (consecutive blocks of one row), which
// unswizzled all fall into one LDS bank (a 128-byte stride); the swizzle
// spreads them over eight.  A group stays whole, so a reader's float4 of
// rows 4g .. 4g+3 is still one 16-byte load.
__device__ __forceinline__ int dx_slot(int lb, int r) {
  return lb * 32 + ((((r >> 2) ^ (lb & 7)) << 2) | (r & 3));
}

// The direct form's stage of the activation scales of blocks [b_lo, b_lo +
// nblk) into LDS (dx_slot order), rows m..31 zero.
// Consecutive threads read consecutive blocks of one row (the buffer's
// scales are row-major), so the loads are coalesced; the LDS write is the
// transpose.
template <int NTHREADS>
__device__ __forceinline__ void stage_act_scales(float *dxs, const void *__restrict__ xv, int m,
                                                 int NB, int b_lo, int nblk,
                                                 unsigned act_scale_off) {
  const float *dxp =
      reinterpret_cast<const float *>(static_cast<const char *>(xv) + act_scale_off);
  for (int p = threadIdx.x; p < nblk * 32; p += NTHREADS) {
    const int r = p / nblk, bb = p - r * nblk;
    dxs[dx_slot(bb, r)] = (r < m) ? dxp[(size_t)r * NB + b_lo + bb] : 0.0f;
  }
}

// Bytes of the 32-row int8 activation stage of nblk blocks (the direct form:
// its scales only), and of the carries of the waves past the first of each
// tile.
template <bool AG>
constexpr size_t m32_stage_bytes(int nblk) { return (size_t)nblk * 32 * (AG ? 4 : 36); }
constexpr size_t m32_red_bytes(int kw, int p) { return (size_t)(kw - 1) * p * 32 * 64 * 4; }

// A tile's split-K partial: one 8 KiB record per (split, tile), 8 pieces of
// 16 bytes per lane, piece k of lane l at k * 1024 + 16 l (acc0[0..3], then
// acc1[0..3]), so every piece is one contiguous KiB of the wave.
__device__ __forceinline__ buf_t m32_record(float *partial, int T, int s, int t) {
  return make_buf(partial + ((size_t)s * T + t) * 2048, 8192);
}

// The finish of tile t by one wave holding its complete sums v0 (column j)
// and v1 (column 32 + j), rows 8q + 4h + e: bias and residual (in that
// order), the pad columns' zero, y, and the quantized output (a row's 32
// columns of one group are the 32 lanes of one h).
__device__ __forceinline__ void m32_store(const Epi &ep, float *__restrict__ y, int Npad, int m,
                                          int t, int lane, f32x4_t (&v0)[4], f32x4_t (&v1)[4]) {
  const int h = lane >> 5, j = lane & 31;
  const size_t c0 = (size_t)t * kTile + j, c1 = c0 + 32;
  const float b0 = (ep.bias && (int)c0 < ep.N) ? ep.bias[c0] : 0.0f;
  const float b1 = (ep.bias && (int)c1 < ep.N) ? ep.bias[c1] : 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 8 * q + 4 * h + e;
      float z0 = v0[q][e], z1 = v1[q][e];
      if (ep.bias) {
        z0 += b0;
        z1 += b1;
      }
      if (ep.residual && r < m) {
        z0 += ep.residual[(size_t)r * Npad + c0];
        z1 += ep.residual[(size_t)r * Npad + c1];
      }
      v0[q][e] = ((int)c0 < ep.N) ? z0 : 0.0f;
      v1[q][e] = ((int)c1 < ep.N) ? z1 : 0.0f;
    }
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 8 * q + 4 * h + e;
      if (r >= m) continue;   // uniform over the 32 lanes of one h
      if (ep.write_y) {
        y[(size_t)r * Npad + c0] = v0[q][e];
        y[(size_t)r * Npad + c1] = v1[q][e];
      }
      if (ep.yq) {
        float a0 = fabsf(v0[q][e]), a1 = fabsf(v1[q][e]);
#pragma unroll
        for (int o = 16; o > 0; o >>= 1) {
          a0 = fmaxf(a0, __shfl_xor(a0, o, 32));
          a1 = fmaxf(a1, __shfl_xor(a1, o, 32));
        }
        const float d0 = q8_scale_of(a0), d1 = q8_scale_of(a1);
        const int8_t k0 = q8_code_of(v0[q][e], d0), k1 = q8_code_of(v1[q][e], d1);
        ep.yq[(size_t)r * Npad + c0] = k0;
        ep.yq[(size_t)r * Npad + c1] = k1;
        ep.yq_view[((c0 / 32) * m + r) * 32 + j] = k0;
        ep.yq_view[((c1 / 32) * m + r) * 32 + j] = k1;
        if (j == 0) {
          ep.yq_scale[(size_t)r * (Npad / 32) + c0 / 32] = d0;
          ep.yq_scale[(size_t)r * (Npad / 32) + c1 / 32] = d1;
        }
      }
    }
}

// AG (the direct form): the activation fragments are loaded from memory with
// each weight stage (16 bytes a lane; rows past m read as zero through the
// buffer's extent) and only the activation scales are staged, so the K range
// of a workgroup is not bounded by the LDS.
// The finish of tile t by one wave holding its sums over the workgroup's K
// range: stored directly with one split; otherwise published as the split's
// record, and the last of the tile's S arrivals sums the records in split
// order and stores.
__device__ __forceinline__ void m32_finish(const Epi &ep, float *__restrict__ y, float *partial,
                                           unsigned *__restrict__ counters, int m, int Npad,
                                           int T, int s, int S, int t, int lane,
                                           f32x4_t (&acc0)[4], f32x4_t (&acc1)[4]) {
  if (S == 1) {
    m32_store(ep, y, Npad, m, t, lane, acc0, acc1);
    return;
  }
  {
    const buf_t rec = m32_record(partial, T, s, t);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      buf_st16_sys(rec, (unsigned)(q * 1024 + lane * 16),
                   make_float4(acc0[q][0], acc0[q][1], acc0[q][2], acc0[q][3]));
      buf_st16_sys(rec, (unsigned)((4 + q) * 1024 + lane * 16),
                   make_float4(acc1[q][0], acc1[q][1], acc1[q][2], acc1[q][3]));
    }
  }
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  unsigned *counter = counters + (size_t)t * 4;
  unsigned prev = 0;
  if (lane == 0)
    prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  prev = __builtin_amdgcn_readfirstlane(prev);
  if (prev != (unsigned)(S - 1)) return;
  // the last arrival: the S records summed in split order, half a record
  // (four pieces) of four splits in flight at a time
  constexpr int kBatch = 4;
#pragma unroll
  for (int k0 = 0; k0 < 8; k0 += 4) {
    for (int s0 = 0; s0 < S; s0 += kBatch) {
      float4 rv[kBatch][4];
#pragma unroll
      for (int qq = 0; qq < kBatch; ++qq) {
        const buf_t rec = m32_record(partial, T, min(s0 + qq, S - 1), t);
#pragma unroll
        for (int k = 0; k < 4; ++k)
          rv[qq][k] = buf_ld16_sys(rec, (unsigned)((k0 + k) * 1024 + lane * 16));
      }
#pragma unroll
      for (int qq = 0; qq < kBatch; ++qq) {
        if (s0 + qq >= S) break;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const f32x4_t p = {rv[qq][k].x, rv[qq][k].y, rv[qq][k].z, rv[qq][k].w};
          f32x4_t &acc = k0 == 0 ? acc0[k] : acc1[k];
          acc = (s0 + qq == 0) ? p : acc + p;
        }
      }
    }
  }
  m32_store(ep, y, Npad, m, t, lane, acc0, acc1);
  if (lane == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

template <int KW, int P, int U, bool DOTS, bool AG>
__global__ void __launch_bounds__(64 * KW * P)
gemv_mfma32_kernel(const void *__restrict__ xv, const int8_t *__restrict__ wq,
                   const float *__restrict__ wsc, float *__restrict__ y,
                   float *__restrict__ partial, unsigned *__restrict__ counters,
                   int32_t *__restrict__ dots, int m, int K, int NB, int Npad, int T, int S,
                   int split_q, int split_r, int G, unsigned act_scale_off, Epi ep) {
  constexpr int MR = 32;
  constexpr int W = KW * P;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5, j = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kw = wave % KW, slot = wave / KW;
  const int s = blockIdx.y;
  const int jwg = blockIdx.x;
  int b_lo, b_hi;
  split_range(s, split_q, split_r, b_lo, b_hi);
  const int nblk = b_hi - b_lo;
  // the lane's bytes in a chunk (group 1: 512 further) and its two scales'
  // places in the chunk's scale row (columns j and 32 + j)
  const unsigned voff = (unsigned)h * kHalfBytes + (unsigned)j * 16u;
  const unsigned soff0 = (unsigned)scale_pos(j) * 4u;
  const unsigned soff1 = (unsigned)scale_pos(32 + j) * 4u;

  // stage u holds block b + u*KW (a block past the range reloads the
  // range's last one, unused)
  // the direct form's activation: m rows of K int8 values
  const buf_t xr = make_buf(xv, (unsigned)m * (unsigned)K);
  const unsigned xoff = (unsigned)j * (unsigned)K + (unsigned)h * 16u;
  auto load = [&](M32Stage<U, AG> &st, buf_t wr, buf_t sr, int b) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int bu = min(b + u * KW, b_hi - 1);
      const unsigned wb = (unsigned)bu * kChunkBytes;
      st.w0[u] = buf_ld16(wr, voff, wb);
      st.w1[u] = buf_ld16(wr, voff + 512u, wb);
      if constexpr (AG) {
        const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(xr, xoff, (unsigned)bu * 32u, 0);
        st.a[u] = make_uint4(v.x, v.y, v.z, v.w);
      }
      if constexpr (!DOTS) {
        const unsigned sb = (unsigned)min(b + u * KW, b_hi - 1) * (kTile * 4);
        st.s0[u] = buf_ld4f(sr, soff0, sb);
        st.s1[u] = buf_ld4f(sr, soff1, sb);
      }
    }
  };
  auto tile_bufs = [&](int t, buf_t &wr, buf_t &sr) {
    wr = make_buf(wq + (size_t)t * NB * kChunkBytes, (unsigned)NB * kChunkBytes);
    if constexpr (DOTS)
      sr = wr;   // unused
    else
      sr = make_buf(wsc + (size_t)t * NB * kTile, (unsigned)NB * kTile * 4);
  };

  constexpr int step = KW * U;
  M32Stage<U, AG> A, B;
  const int t0 = jwg * P + slot;
  // the first tile's first stage in flight while the activation is staged
  if (t0 < T && b_lo + kw < b_hi) {
    buf_t wr, sr;
    tile_bufs(t0, wr, sr);
    load(A, wr, sr, b_lo + kw);
  }
  const int nblk_max = split_q + (split_r > 0 ? 1 : 0);
  if constexpr (AG)
    stage_act_scales<64 * W>(reinterpret_cast<float *>(lds), xv, m, NB, b_lo, nblk,
                             act_scale_off);
  else
    stage_activation<MR, kActQ8, 64 * W>(lds, xv, m, K, NB, b_lo, nblk, act_scale_off);
  __syncthreads();
  const float *dxs =
      reinterpret_cast<const float *>(lds + (AG ? (size_t)0 : (size_t)nblk * MR * 32));
  float *red = reinterpret_cast<float *>(lds + m32_stage_bytes<AG>(nblk_max));

  for (int tg = jwg; tg * P < T; tg += G) {
    const int t = tg * P + slot;
    const bool live = t < T;
    buf_t wr, sr;
    if (live) tile_bufs(t, wr, sr);
    f32x4_t acc0[4], acc1[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc0[q] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      acc1[q] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }

    auto compute = [&](const M32Stage<U, AG> &st, int b0) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int bb = b0 + u * KW;
        if (bb >= b_hi) break;
        const int lb = bb - b_lo;
        i32x4v_t a;
        if constexpr (AG)
          a = __builtin_bit_cast(i32x4v_t, st.a[u]);
        else
          a = *reinterpret_cast<const i32x4v_t *>(lds + ((size_t)lb * MR + j) * 32 +
                                                  (size_t)h * 16);
        const i32x16_t d0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(
            a, __builtin_bit_cast(i32x4v_t, st.w0[u]), i32x16_t{}, 0, 0, 0);
        const i32x16_t d1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(
            a, __builtin_bit_cast(i32x4v_t, st.w1[u]), i32x16_t{}, 0, 0, 0);
        if constexpr (DOTS) {
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int r = 8 * (v >> 2) + 4 * h + (v & 3);
            if (r < m) {
              int32_t *dr = dots + ((size_t)r * NB + bb) * Npad + (size_t)t * kTile + j;
              dr[0] = d0[v];
              dr[32] = d1[v];
            }
          }
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float4 dx4 = *reinterpret_cast<const float4 *>(
                dxs + (AG ? (size_t)dx_slot(lb, 8 * q + 4 * h) : (size_t)lb * MR + 8 * q + 4 * h));
            const float dxv[4] = {dx4.x, dx4.y, dx4.z, dx4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              acc0[q][e] = fmaf(dxv[e] * st.s0[u], (float)d0[4 * q + e], acc0[q][e]);
              acc1[q][e] = fmaf(dxv[e] * st.s1[u], (float)d1[4 * q + e], acc1[q][e]);
            }
          }
        }
      }
    };

    int b = b_lo + kw;
    if (live && b < b_hi) {
      if (tg != jwg) load(A, wr, sr, b);
      // one compute site: the next stage is loaded into B while A is
      // computed, then moved into A
      while (true) {
        if (b + step >= b_hi) {
          compute(A, b);
          break;
        }
        load(B, wr, sr, b + step);
        __builtin_amdgcn_sched_barrier(0);   // keep the prefetch ahead of the compute
        compute(A, b);
        A = B;
        b += step;
      }
    }
    if constexpr (DOTS) continue;

    if constexpr (KW > 1) {
      // the tile's waves past the first hand their carries to the first
      if (kw > 0) {
        float *rw = red + ((size_t)slot * (KW - 1) + (kw - 1)) * 2048;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          *reinterpret_cast<f32x4_t *>(rw + q * 256 + lane * 4) = acc0[q];
          *reinterpret_cast<f32x4_t *>(rw + (4 + q) * 256 + lane * 4) = acc1[q];
        }
      }
      __syncthreads();
      if (kw == 0) {
#pragma unroll
        for (int k2 = 1; k2 < KW; ++k2) {
          const float *rw = red + ((size_t)slot * (KW - 1) + (k2 - 1)) * 2048;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            acc0[q] += *reinterpret_cast<const f32x4_t *>(rw + q * 256 + lane * 4);
            acc1[q] += *reinterpret_cast<const f32x4_t *>(rw + (4 + q) * 256 + lane * 4);
          }
        }
      }
      __syncthreads();   // red is free again for the next tile group
      if (kw != 0) continue;
    }
    if (!live) continue;
    m32_finish(ep, y, partial, counters, m, Npad, T, s, S, t, lane, acc0, acc1);
  }
}

template <int KW, int P, int U, bool DOTS, bool AG>
hipError_t launch_m32(const GemvArgs &a, hipStream_t stream) {
  constexpr int W = KW * P;
  const int nblk_max = (a.NB + a.split_k - 1) / a.split_k;
  const size_t lds = m32_stage_bytes<AG>(nblk_max) + (DOTS ? 0 : m32_red_bytes(KW, P));
  auto kern = gemv_mfma32_kernel<KW, P, U, DOTS, AG>;
  static size_t granted = 64 * 1024;
  hipError_t e = grant_lds(kern, lds, granted);
  if (e != hipSuccess) return e;
  // G workgroups per K split, each walking tile groups j, j+G, ... of P
  // tiles: the fewest rounds of the resident workgroups, balanced
  const int groups = (a.T + P - 1) / P;
  const int G = balanced_grid(resident_workgroups(kern, 64 * W, lds) / a.split_k, groups);
  (void)hipGetLastError();
  kern<<<dim3((unsigned)G, (unsigned)a.split_k), dim3(64 * W), lds, stream>>>(
      a.x, a.wq, a.wsc, a.y, a.partial, a.counters, a.dots, a.m, a.K, a.NB, a.Npad, a.T,
      a.split_k, a.NB / a.split_k, a.NB % a.split_k, G, a.act_scale_off, a.ep);
  return hipGetLastError();
}

// Blocks per stage of the product (two stages in flight).
#ifndef Q8_M32_UNROLL
#define Q8_M32_UNROLL 1
#endif

template <int KW, int P, bool AG>
hipError_t launch_m32_u(bool dots, const GemvArgs &a, hipStream_t stream) {
  if (dots) return launch_m32<KW, P, 1, true, AG>(a, stream);
  return launch_m32<KW, P, Q8_M32_UNROLL, false, AG>(a, stream);
}

template <bool AG>
hipError_t launch_m32_shape(int waves, int kslices, bool dots, const GemvArgs &a,
                            hipStream_t stream) {
  if (waves == 4 && kslices == 1) return launch_m32_u<1, 4, AG>(dots, a, stream);
  if (waves == 4 && kslices == 2) return launch_m32_u<2, 2, AG>(dots, a, stream);
  if (waves == 4 && kslices == 4) return launch_m32_u<4, 1, AG>(dots, a, stream);
  if (waves == 8 && kslices == 1) return launch_m32_u<1, 8, AG>(dots, a, stream);
  if (waves == 8 && kslices == 2) return launch_m32_u<2, 4, AG>(dots, a, stream);
  if (waves == 8 && kslices == 4) return launch_m32_u<4, 2, AG>(dots, a, stream);
  if (waves == 8 && kslices == 8) return launch_m32_u<8, 1, AG>(dots, a, stream);
  return hipErrorInvalidValue;
}


// ---------------------------------------------------------------------------
// the tile-per-workgroup form (kernel 5): the weight stream of the VALU
// kernel, the block dots on the 32x32x32 matrix core
// ---------------------------------------------------------------------------
//
// One workgroup per (tile, K split); its W waves take blocks w, w+W, ... of
// the split.  Lane c loads column c's two 16-byte halves of a block, so each
// load instruction reads one contiguous KiB (the access pattern that reaches
// the read ceiling here); one v_permlane32_swap per dword then hands lanes
// 32-63 the first 32 columns' second halves and lanes 0-31 the last 32
// columns' first halves, which is the matrix core's B operand of the two
// 32-column groups.  The swap of the lane's own scale with itself gives
// every lane both groups' scales of its column j.  The activation fragment
// (row j, k = 16h .. 16h+15) is loaded from memory with the weights, from the
// quantized activation's block-interleaved view, where one block's rows are
// one contiguous run (the row-major rows would put every lane of a load in a
// different cache line; measured on MI355X at m=32, K=5120, N=32000: 44.2
// against 37.3 us); the activation scales of the split are staged in LDS.
// The waves' carries meet by halves in LDS (wave w + half into wave w, half =
// W/2, W/4, .., 1); the tile's sums then go through LDS once more so that
// every wave takes a share of the finish (epilogue, stores, split-K combine).

template <int W>
constexpr size_t m32w_lds_bytes(int nblk) {
  return (size_t)nblk * 32 * 4 + (size_t)(W / 2) * 2048 * 4;
}

// TP: column tiles a wave covers (1 or 2).  With two, each activation
// fragment serves four MFMAs instead of two (half the activation loads per
// weight byte), for products wide enough that half as many workgroups still
// keep every CU streaming.
template <int W, bool DOTS, int TP>
__global__ void __launch_bounds__(64 * W)
gemv_mfma32w_kernel(const void *__restrict__ xv, const int8_t *__restrict__ wq,
                    const float *__restrict__ wsc, float *__restrict__ y,
                    float *__restrict__ partial, unsigned *__restrict__ counters,
                    int32_t *__restrict__ dots, int m, int K, int NB, int Npad, int T, int S,
                    int split_q, int split_r, unsigned act_scale_off, unsigned act_view_off,
                    Epi ep) {
  constexpr int MR = 32;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5, j = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t0 = blockIdx.x * TP, s = blockIdx.y;
  int b_lo, b_hi;
  split_range(s, split_q, split_r, b_lo, b_hi);
  const int nblk = b_hi - b_lo;
  const int nblk_max = split_q + (split_r > 0 ? 1 : 0);

  // tile t0 + tp; a second tile past the last (T odd) streams the first
  // again and is not stored
  buf_t wr[TP], sr[TP];
#pragma unroll
  for (int tp = 0; tp < TP; ++tp) {
    const int tt = t0 + tp < T ? t0 + tp : t0;
    wr[tp] = make_buf(wq + (size_t)tt * NB * kChunkBytes, (unsigned)NB * kChunkBytes);
    sr[tp] = DOTS ? wr[tp] : make_buf(wsc + (size_t)tt * NB * kTile, (unsigned)NB * kTile * 4);
  }
  // the activation's block-interleaved view: block b's rows are m * 32
  // consecutive bytes; lanes of rows past m read zero
  const buf_t xr = make_buf(static_cast<const char *>(xv) + act_view_off,
                            (unsigned)m * (unsigned)K);
  const unsigned lw = (unsigned)lane * 16u, ls = (unsigned)scale_pos(lane) * 4u;
  const bool row_live = j < m;
  const unsigned xoff = (unsigned)(row_live ? j : 0) * 32u + (unsigned)h * 16u;

  struct Stage {
    uint4 lo[TP], hi[TP];   // column `lane`'s k = 0..15 and 16..31 of the block
    uint4 a;                // activation row j, k = 16h .. 16h+15
    float sc[TP];           // column `lane`'s scale
  };
  auto load = [&](Stage &st, int b) {
    const unsigned wb = (unsigned)b * kChunkBytes;
#pragma unroll
    for (int tp = 0; tp < TP; ++tp) {
      st.lo[tp] = buf_ld16(wr[tp], lw, wb);
      st.hi[tp] = buf_ld16(wr[tp], lw + kHalfBytes, wb);
    }
    const u32x4_t v =
        __builtin_amdgcn_raw_buffer_load_b128(xr, xoff, (unsigned)b * (unsigned)m * 32u, 0);
    st.a = row_live ? make_uint4(v.x, v.y, v.z, v.w) : make_uint4(0u, 0u, 0u, 0u);
    if constexpr (!DOTS) {
#pragma unroll
      for (int tp = 0; tp < TP; ++tp) st.sc[tp] = buf_ld4f(sr[tp], ls, (unsigned)b * (kTile * 4));
    }
  };

  Stage A, B;
  if (b_lo + wave < b_hi) load(A, b_lo + wave);
  float *dxs = reinterpret_cast<float *>(lds);
  float *red = reinterpret_cast<float *>(lds + (size_t)nblk_max * MR * 4);
  if constexpr (!DOTS) {
    stage_act_scales<64 * W>(dxs, xv, m, NB, b_lo, nblk, act_scale_off);
    __syncthreads();
  }

  f32x4_t acc0[TP][4], acc1[TP][4];
#pragma unroll
  for (int tp = 0; tp < TP; ++tp)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc0[tp][q] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      acc1[tp][q] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }
  auto compute = [&](const Stage &st, int bb) {
    const i32x4v_t a = __builtin_bit_cast(i32x4v_t, st.a);
#pragma unroll
    for (int tp = 0; tp < TP; ++tp) {
      // the B operands of the tile's two 32-column groups
      uint32_t g0[4], g1[4];
      const uint32_t lo[4] = {st.lo[tp].x, st.lo[tp].y, st.lo[tp].z, st.lo[tp].w};
      const uint32_t hi[4] = {st.hi[tp].x, st.hi[tp].y, st.hi[tp].z, st.hi[tp].w};
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const auto r = __builtin_amdgcn_permlane32_swap(lo[d], hi[d], false, false);
        g0[d] = r[0];
        g1[d] = r[1];
      }
      const i32x16_t d0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(
          a, i32x4v_t{(int)g0[0], (int)g0[1], (int)g0[2], (int)g0[3]}, i32x16_t{}, 0, 0, 0);
      const i32x16_t d1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(
          a, i32x4v_t{(int)g1[0], (int)g1[1], (int)g1[2], (int)g1[3]}, i32x16_t{}, 0, 0, 0);
      if constexpr (DOTS) {
        if (t0 + tp < T) {
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int r = 8 * (v >> 2) + 4 * h + (v & 3);
            if (r < m) {
              int32_t *dr = dots + ((size_t)r * NB + bb) * Npad + (size_t)(t0 + tp) * kTile + j;
              dr[0] = d0[v];
              dr[32] = d1[v];
            }
          }
        }
      } else {
        const unsigned scu = __float_as_uint(st.sc[tp]);
        const auto sp = __builtin_amdgcn_permlane32_swap(scu, scu, false, false);
        const float s0 = __uint_as_float(sp[0]), s1 = __uint_as_float(sp[1]);
        const int lb = bb - b_lo;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 dx4 =
              *reinterpret_cast<const float4 *>(dxs + dx_slot(lb, 8 * q + 4 * h));
          const float dxv[4] = {dx4.x, dx4.y, dx4.z, dx4.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc0[tp][q][e] = fmaf(dxv[e] * s0, (float)d0[4 * q + e], acc0[tp][q][e]);
            acc1[tp][q][e] = fmaf(dxv[e] * s1, (float)d1[4 * q + e], acc1[tp][q][e]);
          }
        }
      }
    }
  };

  int b = b_lo + wave;
  if (b < b_hi) {
    while (true) {
      if (b + W >= b_hi) {
        compute(A, b);
        break;
      }
      load(B, b + W);
      __builtin_amdgcn_sched_barrier(0);   // keep the prefetch ahead of the compute
      compute(A, b);
      A = B;
      b += W;
    }
  }
  if constexpr (DOTS) return;

#pragma unroll
  for (int tp = 0; tp < TP; ++tp) {
    // carries meet by halves: wave w + half adds into wave w
#pragma unroll
    for (int half = W / 2; half >= 1; half /= 2) {
      if (wave >= half && wave < 2 * half) {
        float *rw = red + (size_t)(wave - half) * 2048;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          *reinterpret_cast<f32x4_t *>(rw + q * 256 + lane * 4) = acc0[tp][q];
          *reinterpret_cast<f32x4_t *>(rw + (4 + q) * 256 + lane * 4) = acc1[tp][q];
        }
      }
      __syncthreads();
      if (wave < half) {
        const float *rw = red + (size_t)wave * 2048;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc0[tp][q] += *reinterpret_cast<const f32x4_t *>(rw + q * 256 + lane * 4);
          acc1[tp][q] += *reinterpret_cast<const f32x4_t *>(rw + (4 + q) * 256 + lane * 4);
        }
      }
      __syncthreads();
    }
    // wave 0 holds the tile's sums: into LDS row-major, and every wave takes
    // a share of the epilogue, the stores and the split-K combine
    if (wave == 0) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 8 * q + 4 * h + e;
          red[r * 64 + j] = acc0[tp][q][e];
          red[r * 64 + 32 + j] = acc1[tp][q][e];
        }
    }
    __syncthreads();
    const int t = t0 + tp;
    if (t < T)
      finish_tile<MR, 1, false, 64 * W>(
          red, TileOut{y, Npad, (size_t)t * kTile, (size_t)t * kTile, Npad, (unsigned)t},
          partial, counters, m, s, S, 0, ep);
    if (TP > 1) __syncthreads();   // red is read by the finish before the next tile's carries
  }
}

template <int W, bool DOTS, int TP>
hipError_t launch_m32w(const GemvArgs &a, hipStream_t stream) {
  const int nblk_max = (a.NB + a.split_k - 1) / a.split_k;
  const size_t lds = m32w_lds_bytes<W>(nblk_max);
  auto kern = gemv_mfma32w_kernel<W, DOTS, TP>;
  static size_t granted = 64 * 1024;
  hipError_t e = grant_lds(kern, lds, granted);
  if (e != hipSuccess) return e;
  (void)hipGetLastError();
  kern<<<dim3((unsigned)((a.T + TP - 1) / TP), (unsigned)a.split_k), dim3(64 * W), lds, stream>>>(
      a.x, a.wq, a.wsc, a.y, a.partial, a.counters, a.dots, a.m, a.K, a.NB, a.Npad, a.T,
      a.split_k, a.NB / a.split_k, a.NB % a.split_k, a.act_scale_off, a.act_view_off, a.ep);
  return hipGetLastError();
}

template <int W>
hipError_t launch_m32w_tp(int tp, bool dots, const GemvArgs &a, hipStream_t stream) {
  if (tp == 2)
    return dots ? launch_m32w<W, true, 2>(a, stream) : launch_m32w<W, false, 2>(a, stream);
  return dots ? launch_m32w<W, true, 1>(a, stream) : launch_m32w<W, false, 1>(a, stream);
}

}  // namespace

// Kernels 3 and 4, (waves, kslices) built: waves = kslices x tiles side by
// side.  Kernel 5: 4, 8 or 16 waves; kslices = column tiles a wave covers
// (1, or 2 with 4 or 8 waves).
bool mfma32_instantiated(int kernel, int rows, int act, bool write_dots, int waves,
                         int kslices) {
  (void)write_dots;
  if (rows != 32 || act != kActQ8) return false;
  if (kernel == 5)
    return (kslices == 1 && (waves == 4 || waves == 8 || waves == 16)) ||
           (kslices == 2 && (waves == 4 || waves == 8));
  return (waves == 4 && (kslices == 1 || kslices == 2 || kslices == 4)) ||
         (waves == 8 && (kslices == 1 || kslices == 2 || kslices == 4 || kslices == 8));
}

size_t mfma32_lds_bytes(int kernel, int waves, int kslices, int NB, int split_k) {
  const int nblk = (NB + split_k - 1) / split_k;
  if (kernel == 5) {
    return waves == 4 ? m32w_lds_bytes<4>(nblk)
         : waves == 8 ? m32w_lds_bytes<8>(nblk) : m32w_lds_bytes<16>(nblk);
  }
  const int p = kslices > 0 ? waves / kslices : 1;
  return (kernel == 4 ? m32_stage_bytes<true>(nblk) : m32_stage_bytes<false>(nblk)) +
         m32_red_bytes(kslices, p);
}

hipError_t launch_gemv_mfma32(int kernel, int waves, int kslices, bool write_dots,
                              const GemvArgs &a, hipStream_t stream) {
  if (a.ep.nw != 1 || a.ep.parts.n > 0) return hipErrorInvalidValue;
  if (kernel == 5) {
    switch (waves) {
      case 4: return launch_m32w_tp<4>(kslices, write_dots, a, stream);
      case 8: return launch_m32w_tp<8>(kslices, write_dots, a, stream);
      case 16:
        if (kslices != 1) return hipErrorInvalidValue;
        return write_dots ? launch_m32w<16, true, 1>(a, stream)
                          : launch_m32w<16, false, 1>(a, stream);
      default: return hipErrorInvalidValue;
    }
  }
  return kernel == 4 ? launch_m32_shape<true>(waves, kslices, write_dots, a, stream)
                     : launch_m32_shape<false>(waves, kslices, write_dots, a, stream);
}

}  // namespace q8
