// q8_tile16.hip -- the product for few activation rows (bf16, or the Q8_0
// form) on the 16x16x32 matrix core, one workgroup per column tile: 16, 32
// or 64 rows a wave (RG row groups of 16, each block's weight turned into B
// operands once for all of them), more rows in chunks of 64 (grid z), and
// the parts' tiles side by side (a parts launch).
//
// The product (docs.logicaffeine.com, logicaffeine_compile/spatial/passes/
// from_q8.rs, module doc and fn q8_fold): per Q8_0 block b the dot
// D[r,n] = sum_i x[r,32b+i] * q[32b+i,n], scaled once by the block's scale
// and folded into an fp32 carry.  One 16x16x32 MFMA is exactly that dot for
// 16 rows and 16 columns of one block (its K of 32 is one block), in bf16
// (an int8 weight is exact in bf16 and every product exact in the fp32
// accumulator) or in int8 (exact int32).
//
// The weight stream is the VALU kernel's: lane c loads column c's two
// 16-byte halves of a block, so each load instruction reads one contiguous
// KiB.  The MFMA's B operand of 16-column group g wants, in quarter q of the
// wave (lanes 16q .. 16q+15), the 8 values k = 8q .. 8q+7 of column 16g + i
// (i = lane % 16): a 4 x 4 transpose of (quarter, 8-byte piece), done in
// registers with two v_permlane32_swap and two v_permlane16_swap per dword
// pair.  The scale row's place 4i .. 4i+3 holds the scales of columns i,
// i+16, i+32, i+48 -- the four groups of the lane -- as one 16-byte load.
// The activation fragment (row i, k = 8q .. 8q+7) is loaded with the weights:
// int8 from the quantized activation's block-interleaved view (a block's
// rows are one run; W waves take blocks w, w+W, ...); bf16 either straight
// from the rows, one block a stage, or two blocks a stage (a wave takes pairs
// 2w, 2w+1, then 2w+2W, ...) with the rows' 128 bytes of the pair read as
// whole cache lines and handed to the MFMA layout through a per-wave LDS
// scratch (one block of 16 rows touches 16 half-used lines a load); the
// rows past m are loaded too (their rows of D are never read).  Two stages
// are in flight, taking turns in two register sets.  The waves' carries meet
// by halves in LDS and every wave takes a share of the finish (epilogue,
// stores, split-K combine).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q8_device.h"
#include "q8_internal.h"
#include "q8_product.h"

namespace q8 {
namespace {

using namespace dev;

typedef __attribute__((ext_vector_type(2))) unsigned u32x2v_t;

// LDS: int8, the split's activation scales of the chunk's rows; bf16, a 2 KiB
// scratch per wave and row group (the activation transpose); then the
// carries' halves.
template <int ACT, int W, int RG>
constexpr size_t t16_lds_bytes(int nblk) {
  return (ACT == kActQ8 ? (size_t)nblk * 16 * RG * 4 : (size_t)W * 2048 * RG) +
         (size_t)(W / 2) * 1024 * 4 * RG;
}


// A 16-byte load of the scale row with the default cache policy.
__device__ __forceinline__ float4 buf_ld16f(buf_t r, unsigned voff, unsigned soff) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z),
                     __uint_as_float(v.w));
}

// RG: row groups of 16 a wave covers (MR = 16 RG rows; RG > 1 serves the
// many-row product's smaller chunks, up to 64 rows): each block's weight is
// turned into B operands once and meets RG activation fragments.
template <int ACT, int W, bool DOTS, bool PAIRS, int RG>
__global__ void __launch_bounds__(64 * W)
gemv_tile16_kernel(const void *__restrict__ xv, const int8_t *__restrict__ wq,
                   const float *__restrict__ wsc, float *__restrict__ y,
                   float *__restrict__ partial, unsigned *__restrict__ counters,
                   int32_t *__restrict__ dots, int m, int K, int NB, int Npad, int T, int S,
                   int split_q, int split_r, unsigned act_scale_off, unsigned act_view_off,
                   Epi ep) {
  constexpr int MR = 16 * RG;
  constexpr bool kQ8 = ACT == kActQ8;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int lane = threadIdx.x & 63;
  const int q = lane >> 4, i = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t = blockIdx.x, s = blockIdx.y;
  // rows r0 .. r0 + mz - 1 of the activation: a chunk of MR rows (grid z)
  const int r0 = blockIdx.z * MR;
  const int mz = min(m - r0, MR);
  int b_lo, b_hi;
  split_range(s, split_q, split_r, b_lo, b_hi);
  const int nblk = b_hi - b_lo;
  const int nblk_max = split_q + (split_r > 0 ? 1 : 0);

  // a parts launch: the workgroup's tile t is tile tt of one part's weight
  const int8_t *wt = wq;
  const float *stt = wsc;
  int tt = t;
  if (!DOTS && ep.parts.n > 0) {
    const int p = part_of(ep.parts, t);
    tt = t - ep.parts.cum[p];
    wt = ep.parts.wq[p];
    stt = ep.parts.wsc[p];
  }
  const buf_t wr = make_buf(wt + (size_t)tt * NB * kChunkBytes, (unsigned)NB * kChunkBytes);
  const buf_t sr = DOTS ? wr : make_buf(stt + (size_t)tt * NB * kTile, (unsigned)NB * kTile * 4);
  const unsigned lw = (unsigned)lane * 16u, ls = (unsigned)i * 16u;
  // the activation: the chunk's bf16 rows, or the int8 view (block b's m
  // rows at b*m*32; row r0 + r of the chunk).  Lanes of rows past the chunk
  // load its first row (or, for the pair's whole lines, read zero past the
  // buffer's extent): those rows of D are never read, and an unconditional
  // load keeps the stage's loads out of branches.
  int ri[RG];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg)
    ri[rg] = (kQ8 ? r0 : 0) + (16 * rg + i < mz ? 16 * rg + i : 0);
  const buf_t xr = kQ8 ? make_buf(static_cast<const char *>(xv) + act_view_off,
                                  (unsigned)m * (unsigned)K)
                       : make_buf(static_cast<const char *>(xv) + (size_t)r0 * K * 2,
                                  (unsigned)mz * (unsigned)K * 2u);
  // int8: the view, 8 bytes a lane (row i, k = 8q ..).  bf16 single blocks:
  // 16 bytes a lane (row i, k = 8q ..) from the rows.  bf16 pairs: a stage
  // holds two consecutive blocks; its activation is read as whole cache lines
  // (lane L of load v: row 8v + L/8, bytes 16 (L%8) of the two blocks' 128)
  // and handed to the MFMA layout through the wave's LDS scratch.
  constexpr int U = PAIRS ? 2 : 1;
  const int lrow = lane >> 3;
  unsigned xoff[RG];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg)
    xoff[rg] = kQ8      ? (unsigned)ri[rg] * 32u + (unsigned)q * 8u
               : PAIRS ? (unsigned)(16 * rg + lrow) * (unsigned)K * 2u + (unsigned)(lane & 7) * 16u
                       : (unsigned)ri[rg] * (unsigned)K * 2u + (unsigned)q * 16u;
  const unsigned xoff8 = (unsigned)8 * (unsigned)K * 2u;   // rows 8 .. 15

  struct Stage {
    uint4 lo[U], hi[U];   // column `lane`'s k = 0..15 and 16..31 of each block
    float4 sc[U];         // scales of columns i, i+16, i+32, i+48
    uint4 a[PAIRS ? 2 * RG : (RG > 1 ? RG : 2)];   // row group rg's fragment (int8: .xy);
                                                   // pairs: row group rg's two loads
  };
  auto load = [&](Stage &st, int bv) {
    const int b = __builtin_amdgcn_readfirstlane(bv);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int bu = min(b + u, b_hi - 1);
      const unsigned wb = (unsigned)bu * kChunkBytes;
      st.lo[u] = buf_ld16(wr, lw, wb);
      st.hi[u] = buf_ld16(wr, lw + kHalfBytes, wb);
      if constexpr (!DOTS) st.sc[u] = buf_ld16f(sr, ls, (unsigned)bu * (kTile * 4));
    }
    if constexpr (kQ8) {
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) {
        const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(xr, xoff[rg],
                                                               (unsigned)b * (unsigned)m * 32u, 0);
        st.a[rg] = make_uint4(v.x, v.y, 0u, 0u);
      }
    } else if constexpr (!PAIRS) {
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) {
        const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(xr, xoff[rg], (unsigned)b * 64u, 0);
        st.a[rg] = make_uint4(v.x, v.y, v.z, v.w);
      }
    } else {
      // (a pair never starts at the rows' last block: the host allows
      // two-block stages only where the last split has an even number of
      // blocks, so no read runs past the last row's end)
#pragma unroll
      for (int rg = 0; rg < RG; ++rg)
#pragma unroll
        for (int v2 = 0; v2 < 2; ++v2) {
          const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(
              xr, xoff[rg] + (unsigned)v2 * xoff8, (unsigned)b * 64u, 0);
          st.a[2 * rg + v2] = make_uint4(v.x, v.y, v.z, v.w);
        }
    }
  };

  Stage A, B;
  if (b_lo + U * wave < b_hi) load(A, b_lo + U * wave);
  float *dxs = reinterpret_cast<float *>(lds);
  char *scr = lds + (size_t)wave * 2048 * RG;   // bf16: this wave's transpose scratch
  float *red = reinterpret_cast<float *>(lds + (kQ8 ? (size_t)nblk_max * MR * 4
                                                     : (size_t)W * 2048 * RG));
  if constexpr (kQ8 && !DOTS) {
    // the split's activation scales of the chunk's rows, [block][row], rows
    // past the chunk zero
    const float *dxp =
        reinterpret_cast<const float *>(static_cast<const char *>(xv) + act_scale_off);
    for (int p = threadIdx.x; p < nblk * MR; p += 64 * W) {
      const int r = p / nblk, bb = p - r * nblk;
      dxs[bb * MR + r] = (r < mz) ? dxp[(size_t)(r0 + r) * NB + b_lo + bb] : 0.0f;
    }
    __syncthreads();
  }

  f32x4_t acc[RG][4];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg)
#pragma unroll
    for (int g = 0; g < 4; ++g) acc[rg][g] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // one block of a stage: u its place in the stage, bb the block, afrag the
  // row groups' activation fragments
  auto compute1 = [&](const Stage &st, int u, int bb, const uint4 (&afrag)[RG]) {
    // pieces: quarter Q holds column 16Q + i, piece p = k 8p .. 8p+7; after
    // the transpose R[g] holds, in quarter q, column 16g + i's piece q
    uint32_t R[4][2] = {{st.lo[u].x, st.lo[u].y}, {st.lo[u].z, st.lo[u].w},
                        {st.hi[u].x, st.hi[u].y}, {st.hi[u].z, st.hi[u].w}};
    opaque_copy(R);
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      const auto a02 = __builtin_amdgcn_permlane32_swap(R[0][d], R[2][d], false, false);
      const auto a13 = __builtin_amdgcn_permlane32_swap(R[1][d], R[3][d], false, false);
      const auto b01 = __builtin_amdgcn_permlane16_swap(a02[0], a13[0], false, false);
      const auto b23 = __builtin_amdgcn_permlane16_swap(a02[1], a13[1], false, false);
      R[0][d] = b01[0];
      R[1][d] = b01[1];
      R[2][d] = b23[0];
      R[3][d] = b23[1];
    }
    const float scs[4] = {st.sc[u].x, st.sc[u].y, st.sc[u].z, st.sc[u].w};
    if constexpr (kQ8) {
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) {
        const long a = __builtin_bit_cast(long, make_uint2(afrag[rg].x, afrag[rg].y));
        float4 dx4 = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        if constexpr (!DOTS)
          dx4 = *reinterpret_cast<const float4 *>(dxs + (bb - b_lo) * MR + 16 * rg + 4 * q);
        const float dxv[4] = {dx4.x, dx4.y, dx4.z, dx4.w};
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const long bw = __builtin_bit_cast(long, make_uint2(R[g][0], R[g][1]));
          const i32x4_t d =
              __builtin_amdgcn_mfma_i32_16x16x32_i8(a, bw, i32x4_t{0, 0, 0, 0}, 0, 0, 0);
          if constexpr (DOTS) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 16 * rg + 4 * q + e;
              if (r < mz)
                dots[((size_t)(r0 + r) * NB + bb) * Npad + (size_t)t * kTile + 16 * g + i] = d[e];
            }
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              acc[rg][g][e] = fmaf(dxv[e] * scs[g], (float)d[e], acc[rg][g][e]);
          }
        }
      }
    } else {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const bf16x8_t bw = i8x8_to_bf16(make_uint2(R[g][0], R[g][1]));
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
          const bf16x8_t a = __builtin_bit_cast(bf16x8_t, afrag[rg]);
          const f32x4_t d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              a, bw, f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[rg][g][e] = fmaf(scs[g], d[e], acc[rg][g][e]);
        }
      }
    }
  };

  auto compute = [&](const Stage &st, int b0) {
    if constexpr (!PAIRS) {
      uint4 af[RG];
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) af[rg] = st.a[rg];
      compute1(st, 0, b0, af);
    } else {
      // the pair's rows through LDS: row r's 128 bytes at r * 128, then the
      // MFMA fragment of block u (row i, k = 8q ..) at i * 128 + 64u + 16q
#pragma unroll
      for (int rg = 0; rg < RG; ++rg)
#pragma unroll
        for (int v2 = 0; v2 < 2; ++v2)
          *reinterpret_cast<uint4 *>(scr + rg * 2048 + (8 * v2 + lrow) * 128 + (lane & 7) * 16) =
              st.a[2 * rg + v2];
      __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the writes are done
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (b0 + u >= b_hi) break;
        uint4 af[RG];
#pragma unroll
        for (int rg = 0; rg < RG; ++rg)
          af[rg] = *reinterpret_cast<const uint4 *>(scr + rg * 2048 + i * 128 + 64 * u + 16 * q);
        compute1(st, u, b0 + u, af);
      }
    }
  };

  // Two stages in flight, taking turns: each path issues the next stage's
  // loads just before computing the older one, and no registers are copied
  // between stages, so the compiler waits only for the older stage.
  constexpr int step = W * U;
  int b = b_lo + U * wave;
  if (b < b_hi) {
    while (true) {
      if (b + step >= b_hi) {
        compute(A, b);
        break;
      }
      load(B, b + step);
      compute(A, b);
      b += step;
      if (b + step >= b_hi) {
        compute(B, b);
        break;
      }
      load(A, b + step);
      compute(B, b);
      b += step;
    }
  }
  if constexpr (DOTS) return;

  // carries meet by halves: wave w + half adds into wave w
#pragma unroll
  for (int half = W / 2; half >= 1; half /= 2) {
    if (wave >= half && wave < 2 * half) {
      float *rw = red + (size_t)(wave - half) * 1024 * RG;
#pragma unroll
      for (int rg = 0; rg < RG; ++rg)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<f32x4_t *>(rw + (rg * 4 + g) * 256 + lane * 4) = acc[rg][g];
    }
    __syncthreads();
    if (wave < half) {
      const float *rw = red + (size_t)wave * 1024 * RG;
#pragma unroll
      for (int rg = 0; rg < RG; ++rg)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          acc[rg][g] += *reinterpret_cast<const f32x4_t *>(rw + (rg * 4 + g) * 256 + lane * 4);
    }
    __syncthreads();
  }
  // wave 0 holds the tile's sums: into LDS row-major, then every wave takes a
  // share of the finish
  if (wave == 0) {
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e) red[(16 * rg + 4 * q + e) * 64 + 16 * g + i] = acc[rg][g][e];
  }
  __syncthreads();
  // the chunk's rows of the output (a launch of several chunks has one split
  // and a plain epilogue)
  if (ep.parts.n > 0) {
    PartUnit u = part_unit(ep, t, T);
    u.out.y += (size_t)r0 * u.out.Npad;
    finish_tile<MR, 1, false, 64 * W>(red, u.out, partial, counters, mz, s, S, 0, u.ep);
  } else {
    finish_tile<MR, 1, false, 64 * W>(
        red, TileOut{y + (size_t)r0 * Npad, Npad, (size_t)t * kTile, (size_t)t * kTile, Npad,
                     (unsigned)t},
        partial, counters, mz, s, S, 0, ep);
  }
}

template <int ACT, int W, bool DOTS, bool PAIRS, int RG>
hipError_t launch_t16_k(const GemvArgs &a, hipStream_t stream) {
  const int nblk_max = (a.NB + a.split_k - 1) / a.split_k;
  const size_t lds = t16_lds_bytes<ACT, W, RG>(nblk_max);
  auto kern = gemv_tile16_kernel<ACT, W, DOTS, PAIRS, RG>;
  static size_t granted = 64 * 1024;
  hipError_t e = grant_lds(kern, lds, granted);
  if (e != hipSuccess) return e;
  (void)hipGetLastError();
  const unsigned chunks = (unsigned)((a.m + 16 * RG - 1) / (16 * RG));
  kern<<<dim3((unsigned)a.T, (unsigned)a.split_k, chunks), dim3(64 * W), lds, stream>>>(
      a.x, a.wq, a.wsc, a.y, a.partial, a.counters, a.dots, a.m, a.K, a.NB, a.Npad, a.T,
      a.split_k, a.NB / a.split_k, a.NB % a.split_k, a.act_scale_off, a.act_view_off, a.ep);
  return hipGetLastError();
}

// Instantiated: 16 rows with 4, 8 or 16 waves (bf16 also with two-block
// stages); 32 rows with 4, 8 or 16 waves (bf16 two-block stages with 4 or 8);
// 64 rows with 4 or 8 waves (their accumulators and stages do not fit 16
// waves' registers; with two-block stages not even 8 waves').
template <int ACT, bool DOTS>
hipError_t launch_t16_rw(int rows, int waves, bool pairs, const GemvArgs &a, hipStream_t stream) {
  if (rows == 16 && pairs && ACT == kActBf16) {
    switch (waves) {
      case 4: return launch_t16_k<ACT, 4, DOTS, true, 1>(a, stream);
      case 8: return launch_t16_k<ACT, 8, DOTS, true, 1>(a, stream);
      case 16: return launch_t16_k<ACT, 16, DOTS, true, 1>(a, stream);
      default: return hipErrorInvalidValue;
    }
  }
  if (rows == 32 && pairs && ACT == kActBf16) {
    switch (waves) {
      case 4: return launch_t16_k<ACT, 4, DOTS, true, 2>(a, stream);
      case 8: return launch_t16_k<ACT, 8, DOTS, true, 2>(a, stream);
      default: return hipErrorInvalidValue;
    }
  }
  if (pairs) return hipErrorInvalidValue;
  if (rows == 16) {
    switch (waves) {
      case 4: return launch_t16_k<ACT, 4, DOTS, false, 1>(a, stream);
      case 8: return launch_t16_k<ACT, 8, DOTS, false, 1>(a, stream);
      case 16: return launch_t16_k<ACT, 16, DOTS, false, 1>(a, stream);
      default: return hipErrorInvalidValue;
    }
  }
  if (rows == 32) {
    switch (waves) {
      case 4: return launch_t16_k<ACT, 4, DOTS, false, 2>(a, stream);
      case 8: return launch_t16_k<ACT, 8, DOTS, false, 2>(a, stream);
      case 16: return launch_t16_k<ACT, 16, DOTS, false, 2>(a, stream);
      default: return hipErrorInvalidValue;
    }
  }
  if (rows == 64) {
    switch (waves) {
      case 4: return launch_t16_k<ACT, 4, DOTS, false, 4>(a, stream);
      case 8: return launch_t16_k<ACT, 8, DOTS, false, 4>(a, stream);
      default: return hipErrorInvalidValue;
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool tile16_instantiated(int rows, int act, bool write_dots, int waves, int kslices) {
  const bool w = rows == 64 ? (waves == 4 || waves == 8)
                            : (rows == 16 || rows == 32) && (waves == 4 || waves == 8 || waves == 16);
  if (!w) return false;
  if (act == kActQ8) return kslices == 1;
  return act == kActBf16 && !write_dots &&
         (kslices == 1 || (kslices == 2 && (rows == 16 || (rows == 32 && waves <= 8))));
}

size_t tile16_lds_bytes(int rows, int act, int waves, int NB, int split_k) {
  const int nblk = (NB + split_k - 1) / split_k;
  const int rg = rows / 16;
  const size_t first = act == kActQ8 ? (size_t)nblk * 16 * rg * 4 : (size_t)waves * 2048 * rg;
  return first + (size_t)(waves / 2) * 1024 * 4 * rg;
}

hipError_t launch_gemv_tile16(int rows, int act, int waves, int kslices, bool write_dots,
                              const GemvArgs &a, hipStream_t stream) {
  if (a.ep.nw != 1 || (a.ep.parts.n > 0 && write_dots)) return hipErrorInvalidValue;
  // more rows than a wave covers: chunks of rows in grid z, one split and no
  // row-wise epilogue (residual, output quantizer)
  if (a.m > rows && (a.split_k != 1 || a.ep.residual || a.ep.yq))
    return hipErrorInvalidValue;
  if (!tile16_instantiated(rows, act, write_dots, waves, kslices)) return hipErrorInvalidValue;
  if (act == kActQ8)
    return write_dots ? launch_t16_rw<kActQ8, true>(rows, waves, false, a, stream)
                      : launch_t16_rw<kActQ8, false>(rows, waves, false, a, stream);
  return launch_t16_rw<kActBf16, false>(rows, waves, kslices == 2, a, stream);
}

}  // namespace q8
