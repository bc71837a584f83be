// q8_product.h -- device pieces shared by the product kernels (q8_kernels.hip,
// q8_mfma32.hip): split ranges, the epilogue arithmetic, the split-K combine
// of a finished tile, the activation stage into LDS, and the host's
// occupancy and LDS helpers for persistent grids.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q8_device.h"
#include "q8_internal.h"

namespace q8 {
namespace {

using namespace dev;
// ---------------------------------------------------------------------------
// the product: shared pieces
// ---------------------------------------------------------------------------

// The workgroup's range of blocks [b_lo, b_hi) of split s: NB = S*q + r
// blocks, the first r splits one block longer (q and r come from the host,
// so a workgroup starts its stream without an integer division).
__device__ __forceinline__ void split_range(int s, int q, int r, int &b_lo, int &b_hi) {
  b_lo = s * q + min(s, r);
  b_hi = b_lo + q + (s < r ? 1 : 0);
}

// SiLU, g * sigmoid(g), in fp32 (the gate of the pages' GemvGlu launch).
__device__ __forceinline__ float silu(float g) { return g / (1.0f + expf(-g)); }

// z of output element (r, col) from its sums over K: vg of the (first) weight
// and, for the gated pair, vu of the second.  Single weight: bias and
// residual added in that order; pair: silu(vg + bias) * (vu + bias_u).  Pad
// columns are exactly 0.
template <bool PAIR>
__device__ __forceinline__ float final_value(const Epi &ep, int Npad, int r, size_t col, float vg,
                                             float vu) {
  if ((int)col >= ep.N) return 0.0f;
  if constexpr (PAIR) {
    if (ep.bias) vg += ep.bias[col];
    if (ep.bias_u) vu += ep.bias_u[col];
    return silu(vg) * vu;
  }
  if (ep.bias) vg += ep.bias[col];
  if (ep.residual) vg += ep.residual[(size_t)r * Npad + col];
  return vg;
}

// Stores z of output element (r, col): y when asked, and its quantized form.
// The quantizer reduces over 32 consecutive columns, so all 32 lanes of the
// caller's 32-lane half-wave must call together, for one row and the 32
// columns of one 32-column block (in lane order).
__device__ __forceinline__ void store_final(const Epi &ep, float *__restrict__ y, int Npad, int m,
                                            int r, size_t col, float z) {
  if (ep.write_y) y[(size_t)r * Npad + col] = z;
  if (ep.yq) {
    float a = fabsf(z);
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) a = fmaxf(a, __shfl_xor(a, o, 32));
    const float d = q8_scale_of(a);
    const int8_t c = q8_code_of(z, d);
    ep.yq[(size_t)r * Npad + col] = c;
    ep.yq_view[((col / 32) * m + r) * 32 + (col & 31)] = c;
    if ((col & 31) == 0) ep.yq_scale[(size_t)r * (Npad / 32) + col / 32] = d;
  }
}

// Sum over the S splits of weight `wsel`'s partial carries of (r, col), in
// split order.  partial holds [wsel][split][row][column] carries.  The loads
// go out eight at a time (a place past the last split reloads the last one,
// unused), so the last arrival waits about one memory round trip per eight
// splits rather than one per split; the additions keep split order, so the
// sum has the bits of the plain serial one.
__device__ __forceinline__ float sum_partials(const float *__restrict__ partial, int m, int Npad,
                                              int S, int wsel, int r, size_t col) {
  constexpr int kBatch = 8;
  const float *p = partial + ((size_t)wsel * S * m + r) * Npad + col;
  const size_t stride = (size_t)m * Npad;
  float v = 0.0f;
  for (int s0 = 0; s0 < S; s0 += kBatch) {
    float t[kBatch];
#pragma unroll
    for (int q = 0; q < kBatch; ++q)
      t[q] = __hip_atomic_load(p + (size_t)min(s0 + q, S - 1) * stride, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_SYSTEM);
#pragma unroll
    for (int q = 0; q < kBatch; ++q)
      if (s0 + q < S) v = (s0 + q == 0) ? t[q] : v + t[q];
  }
  return v;
}

// Where a unit's finished tile goes: its product's output y (row stride
// Npad) at columns col0 .., its partial carries' columns pcol0 .. in rows of
// pstride, and its arrival counter.
struct TileOut {
  float *y;
  int Npad;
  size_t col0;
  size_t pcol0;
  int pstride;
  unsigned cidx;
};

// The part that unit tv of a parts launch belongs to.
__device__ __forceinline__ int part_of(const Parts &pt, int tv) {
  int p = 0;
#pragma unroll
  for (int i = 1; i < kMaxParts; ++i)
    if (i < pt.n && tv >= pt.cum[i]) p = i;
  return p;
}

// Unit tv of a parts launch (units in all): its weight, where its tile goes,
// its epilogue (the part's bias and width), and its tile within the part.
struct PartUnit {
  const int8_t *wq;
  const float *wsc;
  TileOut out;
  Epi ep;
  int t;
};
__device__ __forceinline__ PartUnit part_unit(const Epi &ep, int tv, int units) {
  const Parts &pt = ep.parts;
  const int p = part_of(pt, tv);
  PartUnit u;
  u.t = tv - pt.cum[p];
  u.wq = pt.wq[p];
  u.wsc = pt.wsc[p];
  const int np = (pt.N[p] + kTile - 1) / kTile * kTile;
  u.out = TileOut{pt.y[p], np, (size_t)u.t * kTile, (size_t)tv * kTile, units * kTile,
                  (unsigned)tv};
  u.ep = ep;
  u.ep.bias = pt.bias[p];
  u.ep.N = pt.N[p];
  return u;
}

// Epilogue of both kernels.  red[w][r][c] holds wave w's fp32 carry of row r,
// tile column c of weight `wsel` (already written, __syncthreads() done by the
// caller).  Sums the waves in order; when the tile's value is complete here
// (one split, one weight) stores it, otherwise publishes the partial and the
// last of the tile's S * nw arrivals sums each weight's S partials in split
// order and stores the final values.
//
// The partial carries are written and read with system-scope relaxed atomic
// stores and loads, which go through to memory and bypass the per-XCD L2s;
// their completion is awaited (s_waitcnt 0) before the arrival count is
// bumped.  So no workgroup needs a device-scope fence, whose L2 write-back and
// invalidate would cost each workgroup microseconds.
// NT: the workgroup's threads (by default the W waves' 64 W).
template <int MR, int W, bool PAIR, int NT = 64 * W>
__device__ __forceinline__ void finish_tile(const float *red, const TileOut &o,
                                            float *__restrict__ partial,
                                            unsigned *__restrict__ counters, int m, int s, int S,
                                            int wsel, const Epi &ep) {
  const int arrivals = S * (PAIR ? 2 : 1);
  if (!PAIR && arrivals == 1) {
    // One split, one weight: the bias and residual of all the thread's
    // elements are loaded first, so that their round trips overlap rather
    // than one per element (the stores in between may alias them for the
    // compiler); the additions keep final_value's order.
    constexpr int kIt = (MR * 64 + NT - 1) / NT;
    float bz[kIt], rz[kIt];
#pragma unroll
    for (int k = 0; k < kIt; ++k) {
      const int idx = (int)threadIdx.x + k * NT;
      const int r = idx >> 6;
      const size_t col = o.col0 + (idx & 63);
      const bool live = idx < MR * 64 && r < m && (int)col < ep.N;
      bz[k] = (live && ep.bias) ? ep.bias[col] : 0.0f;
      rz[k] = (live && ep.residual) ? ep.residual[(size_t)r * o.Npad + col] : 0.0f;
    }
#pragma unroll
    for (int k = 0; k < kIt; ++k) {
      const int idx = (int)threadIdx.x + k * NT;
      const int r = idx >> 6, c = idx & 63;
      if (idx < MR * 64 && r < m) {
        float v = red[idx];
#pragma unroll
        for (int w = 1; w < W; ++w) v += red[w * MR * 64 + idx];
        const size_t col = o.col0 + c;
        float z = 0.0f;
        if ((int)col < ep.N) {
          z = v;
          if (ep.bias) z += bz[k];
          if (ep.residual) z += rz[k];
        }
        store_final(ep, o.y, o.Npad, m, r, col, z);
      }
    }
    return;
  }
  for (int idx = threadIdx.x; idx < MR * 64; idx += NT) {
    const int r = idx >> 6, c = idx & 63;
    if (r < m) {
      float v = red[idx];
#pragma unroll
      for (int w = 1; w < W; ++w) v += red[w * MR * 64 + idx];
      if (arrivals == 1)
        store_final(ep, o.y, o.Npad, m, r, o.col0 + c,
                    final_value<PAIR>(ep, o.Npad, r, o.col0 + c, v, 0.0f));
      else
        __hip_atomic_store(&partial[(((size_t)wsel * S + s) * m + r) * o.pstride + o.pcol0 + c],
                           v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
  }
  if (arrivals == 1) return;
  __shared__ int is_last;
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  if (threadIdx.x == 0)
    is_last = (__hip_atomic_fetch_add(&counters[o.cidx], 1u, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_SYSTEM) == (unsigned)(arrivals - 1))
                  ? 1 : 0;
  __syncthreads();
  if (!is_last) return;
  for (int idx = threadIdx.x; idx < MR * 64; idx += NT) {
    const int r = idx >> 6, c = idx & 63;
    if (r < m) {
      const float vg = sum_partials(partial, m, o.pstride, S, 0, r, o.pcol0 + c);
      const float vu = PAIR ? sum_partials(partial, m, o.pstride, S, 1, r, o.pcol0 + c) : 0.0f;
      store_final(ep, o.y, o.Npad, m, r, o.col0 + c,
                  final_value<PAIR>(ep, o.Npad, r, o.col0 + c, vg, vu));
    }
  }
  if (threadIdx.x == 0)
    __hip_atomic_store(&counters[o.cidx], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// The gated pair's epilogue when one workgroup holds both weights of its
// tile (the block-interleaved MFMA kernel): red[w][r][c] holds the gate's
// carries in waves 0 .. W/2-1 and the up weight's in waves W/2 .. W-1
// (written, __syncthreads() done by the caller).  Each weight's waves are
// summed in order; with one split the gate is applied here, otherwise both
// weights' partials are published and the last of the tile's S arrivals sums
// each weight's S partials in split order (the protocol of finish_tile).
template <int MR, int W>
__device__ __forceinline__ void finish_pair_tile(const float *red, const TileOut &o,
                                                 float *__restrict__ partial,
                                                 unsigned *__restrict__ counters, int m, int s,
                                                 int S, const Epi &ep) {
  constexpr int WH = W / 2;
  for (int idx = threadIdx.x; idx < MR * 64; idx += 64 * W) {
    const int r = idx >> 6, c = idx & 63;
    if (r < m) {
      float vg = red[idx], vu = red[WH * MR * 64 + idx];
#pragma unroll
      for (int w = 1; w < WH; ++w) {
        vg += red[w * MR * 64 + idx];
        vu += red[(WH + w) * MR * 64 + idx];
      }
      if (S == 1) {
        store_final(ep, o.y, o.Npad, m, r, o.col0 + c,
                    final_value<true>(ep, o.Npad, r, o.col0 + c, vg, vu));
      } else {
        __hip_atomic_store(&partial[((size_t)s * m + r) * o.pstride + o.pcol0 + c], vg,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        __hip_atomic_store(&partial[(((size_t)S + s) * m + r) * o.pstride + o.pcol0 + c], vu,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      }
    }
  }
  if (S == 1) return;
  __shared__ int is_last_pair;
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  if (threadIdx.x == 0)
    is_last_pair = (__hip_atomic_fetch_add(&counters[o.cidx], 1u, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_SYSTEM) == (unsigned)(S - 1))
                       ? 1 : 0;
  __syncthreads();
  if (!is_last_pair) return;
  for (int idx = threadIdx.x; idx < MR * 64; idx += 64 * W) {
    const int r = idx >> 6, c = idx & 63;
    if (r < m) {
      const float vg = sum_partials(partial, m, o.pstride, S, 0, r, o.pcol0 + c);
      const float vu = sum_partials(partial, m, o.pstride, S, 1, r, o.pcol0 + c);
      store_final(ep, o.y, o.Npad, m, r, o.col0 + c,
                  final_value<true>(ep, o.Npad, r, o.col0 + c, vg, vu));
    }
  }
  if (threadIdx.x == 0)
    __hip_atomic_store(&counters[o.cidx], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Bytes of the activation stage of one workgroup (largest split).
__host__ __device__ constexpr size_t mfma_stage_bytes(int rows, int act, int nblk) {
  return (size_t)nblk * rows * (act == kActBf16 ? 64 : 36);
}

// Stage the activation rows of blocks [b_lo, b_lo + nblk) into LDS:
// [block][row][kRowBytes], then (int8) the fp32 block scales [block][row].
// Eight 16-byte pieces in flight per thread; the loads are unconditional
// (indices clamped in bounds) and values past the range or past row m-1 are
// replaced by zero at the LDS write.
template <int MR, int ACT, int NTHREADS>
__device__ __forceinline__ void stage_activation(char *lds, const void *__restrict__ xv, int m,
                                                 int K, int NB, int b_lo, int nblk,
                                                 unsigned act_scale_off) {
  constexpr int kRowBytes = (ACT == kActBf16) ? 64 : 32;
  constexpr int kBatch = 8;
  constexpr int ppr = kRowBytes / 16;
  const int total = nblk * MR * ppr;
  const char *xbase = static_cast<const char *>(xv);
  // Two-word form (MR = 32, m <= 16): LDS rows 0-15 take the first words of
  // rows 0-15, rows 16-31 the second words (buffer rows m .. 2m-1).
  constexpr bool kTwo = ACT == kActQ8x2;
  for (int p0 = threadIdx.x; p0 < total; p0 += NTHREADS * kBatch) {
    uint4 v[kBatch];
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      const int p = min(p0 + q * NTHREADS, total - 1);
      const int piece = p % ppr;
      const int r = (p / ppr) % MR;
      const int bb = p / (ppr * MR);
      const int src = kTwo ? min(r & 15, m - 1) + (r >= 16 ? m : 0) : min(r, m - 1);
      v[q] = *reinterpret_cast<const uint4 *>(
          xbase + ((size_t)src * K + (size_t)(b_lo + bb) * kBlock) * (kRowBytes / 32) +
          piece * 16);
    }
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      const int p = p0 + q * NTHREADS;
      const int r = (p / ppr) % MR;
      if (p < total)
        *reinterpret_cast<uint4 *>(lds + (size_t)p * 16) =
            ((kTwo ? (r & 15) : r) < m) ? v[q] : make_uint4(0u, 0u, 0u, 0u);
    }
  }
  if constexpr (ACT != kActBf16) {
    float *dxs = reinterpret_cast<float *>(lds + (size_t)nblk * MR * kRowBytes);
    const float *dxp = reinterpret_cast<const float *>(xbase + act_scale_off);
    const int nd = nblk * MR;
    for (int p0 = threadIdx.x; p0 < nd; p0 += NTHREADS * kBatch) {
      float v[kBatch];
#pragma unroll
      for (int q = 0; q < kBatch; ++q) {
        const int p = min(p0 + q * NTHREADS, nd - 1);
        const int r = kTwo ? (p % MR) & 15 : p % MR;
        v[q] = dxp[(size_t)min(r, m - 1) * NB + b_lo + p / MR];
      }
#pragma unroll
      for (int q = 0; q < kBatch; ++q) {
        const int p = p0 + q * NTHREADS;
        const int r = kTwo ? (p % MR) & 15 : p % MR;
        if (p < nd) dxs[p] = (r < m) ? v[q] : 0.0f;
      }
    }
  }
}

// Workgroups of a launch that fit on the device at once (per CU, from the
// runtime's occupancy query for this kernel and LDS size, times the CUs).
template <typename Kern>
int resident_workgroups(Kern kern, int threads, size_t lds) {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, threads, lds) != hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  int dev = 0, cus = 0;
  (void)hipGetDevice(&dev);
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1)
    cus = 256;
  return per_cu * cus;
}

// Workgroups of a persistent grid over `units` units of work when at most
// `fit` are resident: the fewest rounds, then the fewest workgroups that
// finish in that many rounds, so every workgroup walks the same number of
// units (448 units on 256 resident: 224 workgroups of 2, not 256 of 1 or 2).
inline int balanced_grid(int fit, int units) {
  if (fit < 1) fit = 1;
  if (units < 1) return 1;
  const int rounds = (units + fit - 1) / fit;
  return (units + rounds - 1) / rounds;
}

// Grants the dynamic LDS above the default 64 KiB (once per size increase).
template <typename Kern>
hipError_t grant_lds(Kern kern, size_t lds, size_t &granted) {
  if (lds <= granted) return hipSuccess;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e == hipSuccess) granted = lds;
  return e;
}

}  // namespace
}  // namespace q8
