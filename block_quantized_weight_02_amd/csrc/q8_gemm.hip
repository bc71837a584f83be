// q8_gemm.hip -- the Q8_0 weight product for many activation rows (a prefill
// chunk): a matrix-core GEMM over the packed weight.
//
// What it computes is the product of q8_kernels.hip for any m:
//   y[r,n] = sum_b s[b,n] * D[r,b,n],  D[r,b,n] = sum_i x[r,32b+i] * q[32b+i,n]
// (int8 activations: x = dx[r,b] * xq), carried in fp32.  The pages' CUDA
// planner takes the product to its tensor-core GEMM above the GEMV's rows,
// with the activation quantized and the Q8_0 scale arrays read beside the
// values (codegen_cuda/lane/plan.rs, Launch::on_tensor_cores and
// gemm_blk_rows).
//
// gfx950 design:
//   * a workgroup of 4 waves owns a BM x BN output tile (BM = 64: 1 x 4 waves,
//     BN = 256; BM = 128: 2 x 2 waves, BN = 128); each wave a 64 x 64 piece:
//     4 row groups x 4 column groups of 16 = 16 MFMAs per Q8_0 block;
//   * one 16x16x32 MFMA is exactly one Q8_0 block (K = 32), so every D is a
//     single block's dot and takes its own scale on the vector ALU:
//     acc += s[b,n] * D (int8: (dx[r,b] * s[b,n]) * D);
//   * the activation rows and the weight chunks of kGemmCB blocks are staged
//     in LDS by the whole workgroup (16-byte pieces, coalesced), double
//     buffered: the next stage's global loads are in flight while the current
//     stage is computed.  The weight's packed chunks are copied as they are:
//     their byte order already is the MFMA B-operand order;
//   * workgroups are numbered so that each XCD walks a contiguous range of
//     (row block, column block) pairs with the row block fastest: the row
//     blocks that read one weight tile run together on one XCD, and its L2
//     serves the weight to all of them.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q8_device.h"
#include "q8_internal.h"

namespace q8 {
namespace {

using namespace dev;

constexpr int kGemmCB = 2;        // Q8_0 blocks per LDS stage
constexpr int kGemmThreads = 256;

template <int ACT, int BM>
struct GemmShape {
  static constexpr int WM = BM / 64;            // waves along M
  static constexpr int WN = 4 / WM;             // waves along N, one 64-column tile each
  static constexpr int BN = 64 * WN;
  static constexpr int kRowB = ACT == kActBf16 ? 64 : 32;   // activation bytes, one row x block
  // staged activation rows: the two-word form stages its BM rows' first
  // words, then the same rows' second words
  static constexpr int kRowsA = ACT == kActQ8x2 ? 2 * BM : BM;
  static constexpr int kA = kGemmCB * kRowsA * kRowB;       // activation bytes per stage
  static constexpr int kDx = ACT == kActBf16 ? 0 : kGemmCB * BM * 4;   // int8 row scales
  static constexpr int kW = WN * kGemmCB * kChunkBytes;     // weight values per stage (global)
  // in LDS the bf16 form holds the values as bf16 (converted once, at staging)
  static constexpr int kWElt = ACT == kActBf16 ? 2 : 1;
  static constexpr int kWL = kW * kWElt;                    // weight values per stage (LDS)
  static constexpr int kS = WN * kGemmCB * kTile * 4;       // weight scales per stage
  static constexpr int kStage = kA + kDx + kWL + kS;
  static constexpr int kPieces = (kA + kW + kS) / 16;       // 16-byte staging pieces
  static constexpr int kPer = (kPieces + kGemmThreads - 1) / kGemmThreads;
  static constexpr int kDxPer = (kGemmCB * BM + kGemmThreads - 1) / kGemmThreads;
  static_assert(kA % (16 * 64) == 0 && kW % (16 * 64) == 0 && kS % (16 * 64) == 0,
                "each wave's staging pieces fall in one region");
};

// Byte offset, within one row's staged activation, of 16-byte part `unit`
// of row r (bf16), or of 8-byte unit `unit` (int8).  The parts of a row are
// permuted by a function of r % 16 so that the MFMA operand read (lane
// (i, j) reads part j of row i, 16 bytes) does not stall on LDS banks.  The
// bf16 parts are XORed with bits 1-2 of the row: measured with the LDS
// bank-conflict counter on MI355X, that read is conflict-free, while rows
// at a 64-byte stride unpermuted, or XORed with bits 0-1, 2-3, or
// (bit 3 ^ bit 1, bit 2), stall on about a sixth of their LDS cycles; the
// staging writes (lane l writes part l % 4 of row l / 4) are conflict-free
// under any of these.  The int8 rows' four 8-byte units are XORed with bits
// 2-3 of the row: both the operand read (lane (i, j): unit j of row i) and the
// staging writes (two 8-byte units a lane) conflict-free, where the earlier
// permutation stalled the writes on half their cycles.
template <int ACT>
__device__ __forceinline__ int a_part(int r, int unit) {
  if constexpr (ACT == kActBf16) {
    return (unit ^ ((r >> 1) & 3)) * 16;
  } else {
    return (unit ^ ((r >> 2) & 3)) * 8;
  }
}

// The bf16 weight's 16-byte part swizzle for column c (see gemm_store): bit 2
// of the column.  Measured with the LDS bank-conflict counter on MI355X, it
// leaves both the staging writes (lane c writes column c's parts) and the
// operand reads (lane (i, j) reads part j % 2 of column 16g + i) conflict-free;
// unpermuted, the writes stall on half their cycles, and with bits 2 ^ 3 the
// reads stall on about a sixth of theirs.
__device__ __forceinline__ int w_part_swizzle(int c) { return (c >> 2) & 1; }

// One thread's share of a stage: which 16-byte pieces it copies, from where
// (an offset from the stage's wave-uniform region base) and to where in LDS.
// Computed once per workgroup; a stage only moves the region bases:
//   activation: row0's row at the stage's first block;
//   weight values / scales: tile t0's chunk / scale row of that block.
// Thread tid copies activation pieces tid + 256k (k < kNA), weight pieces
// tid + 256k (k < kNW) and, when tid < kNS, scale piece tid.  Rows past m and
// tiles past T are clamped to valid ones: their LDS rows and columns feed
// only outputs that are never stored.
template <int ACT, int BM>
struct GemmPlan {
  using S = GemmShape<ACT, BM>;
  static constexpr int kNA = S::kA / 16 / kGemmThreads;
  static constexpr int kNW = S::kW / 16 / kGemmThreads;
  static constexpr int kNS = S::kS / 16;   // pieces; threads below it copy one
  static_assert(S::kA % (16 * kGemmThreads) == 0 && S::kW % (16 * kGemmThreads) == 0 &&
                kNS <= kGemmThreads && kNS % 64 == 0, "whole pieces per thread, whole waves");
  unsigned asrc[kNA], wsrc[kNW], ssrc;   // byte offsets from the region bases
  int adst[kNA], adst2[kNA], wdst[kNW], sdst;
  int acb[kNA], wcb[kNW], scb;           // the piece's block within the stage
  unsigned dxsrc[S::kDxPer];
  int dxcb[S::kDxPer];
};

template <int ACT, int BM>
__device__ __forceinline__ void gemm_plan(GemmPlan<ACT, BM> &pl, int m, int K, int NB, int T,
                                          int row0, int t0) {
  using S = GemmShape<ACT, BM>;
  using P = GemmPlan<ACT, BM>;
  constexpr int kPPB = S::kRowB / 16;
  constexpr int kElt = ACT == kActBf16 ? 2 : 1;
  const int tid = (int)threadIdx.x;
  // activation pieces: consecutive threads take the parts of consecutive
  // rows of one block (so a store's 16 lanes write 4 rows: distinct banks)
  constexpr int RA = S::kRowsA;
#pragma unroll
  for (int k = 0; k < P::kNA; ++k) {
    const int p = k * kGemmThreads + tid;
    const int q = p % kPPB, r = (p / kPPB) % RA, cb = p / (kPPB * RA);
    // staged row r: row row0 + r, or (two words, r >= BM) the second words
    // of row row0 + r - BM, m rows further on
    const int rr = r < BM ? r : r - BM;
    const int rc = min(row0 + rr, m - 1) - row0 + (r < BM ? 0 : m);
    pl.asrc[k] = (unsigned)rc * (unsigned)K * kElt + cb * kBlock * kElt + q * 16;
    pl.acb[k] = cb;
    if constexpr (ACT == kActBf16) {
      pl.adst[k] = (cb * RA + r) * S::kRowB + a_part<ACT>(r, q);
      pl.adst2[k] = 0;
    } else {
      pl.adst[k] = (cb * RA + r) * S::kRowB + a_part<ACT>(r, 2 * q);
      pl.adst2[k] = (cb * RA + r) * S::kRowB + a_part<ACT>(r, 2 * q + 1);
    }
  }
#pragma unroll
  for (int k = 0; k < P::kNW; ++k) {
    const int p = k * kGemmThreads + tid;
    const int q = p % 128, cb = (p / 128) % kGemmCB, wn = p / (128 * kGemmCB);
    const int tc = min(t0 + wn, T - 1) - t0;
    pl.wsrc[k] = ((unsigned)tc * NB + cb) * kChunkBytes + q * 16;
    pl.wcb[k] = cb;
    // int8 form: the chunk as it is.  bf16 form: column c's 16 values of half h
    // at h * 2048 + c * 32, in two 16-byte parts (swizzled at the store)
    pl.wdst[k] = S::kA + S::kDx + (wn * kGemmCB + cb) * kChunkBytes * S::kWElt + q * 16 * S::kWElt;
  }
  {
    const int p = min(tid, P::kNS - 1);
    const int q = p % 16, cb = (p / 16) % kGemmCB, wn = p / (16 * kGemmCB);
    const int tc = min(t0 + wn, T - 1) - t0;
    pl.ssrc = ((unsigned)tc * NB + cb) * (kTile * 4) + q * 16;
    pl.scb = cb;
    pl.sdst = S::kA + S::kDx + S::kWL + (wn * kGemmCB + cb) * kTile * 4 + q * 16;
  }
  if constexpr (ACT != kActBf16) {
#pragma unroll
    for (int k = 0; k < S::kDxPer; ++k) {
      const int p = min(k * kGemmThreads + tid, kGemmCB * BM - 1);
      const int cb = p / BM, r = p % BM;   // LDS order [cb][r]
      pl.dxsrc[k] = (unsigned)(min(row0 + r, m - 1) - row0) * NB + cb;
      pl.dxcb[k] = cb;
    }
  }
}

// Registers holding one stage between its global loads and its LDS write.
template <int ACT, int BM>
struct GemmStaging {
  using P = GemmPlan<ACT, BM>;
  u32x4_t va[P::kNA], vw[P::kNW], vs;   // native vectors (a uint4 struct copy becomes a
                                        // memcpy that keeps the array in scratch memory)
  float dx[GemmShape<ACT, BM>::kDxPer];
};

// Issue the global loads of a stage.  nvalid: the stage's blocks inside K.
// Pieces of later blocks (the last stage only) reload the stage's last block
// in K instead -- in bounds, and those LDS blocks are never computed.  Loads
// and stores are unconditional (a staging array written under divergent
// conditions would be kept in scratch memory).
template <int ACT, int BM, bool DOTS>
__device__ __forceinline__ void gemm_load(GemmStaging<ACT, BM> &st, const GemmPlan<ACT, BM> &pl,
                                          const char *abase, const char *wbase,
                                          const char *sbase, const float *dxbase, int nvalid) {
  using P = GemmPlan<ACT, BM>;
  constexpr unsigned kAStride = kBlock * (ACT == kActBf16 ? 2 : 1);   // one block of a row
  if (nvalid >= kGemmCB) {
#pragma unroll
    for (int k = 0; k < P::kNA; ++k) st.va[k] = *reinterpret_cast<const u32x4_t *>(abase + pl.asrc[k]);
#pragma unroll
    for (int k = 0; k < P::kNW; ++k) st.vw[k] = *reinterpret_cast<const u32x4_t *>(wbase + pl.wsrc[k]);
    if (!DOTS && (int)threadIdx.x < P::kNS)
      st.vs = *reinterpret_cast<const u32x4_t *>(sbase + pl.ssrc);
    if constexpr (ACT != kActBf16 && !DOTS) {
#pragma unroll
      for (int k = 0; k < GemmShape<ACT, BM>::kDxPer; ++k) st.dx[k] = dxbase[pl.dxsrc[k]];
    }
  } else {
    // back off by the blocks past K
#pragma unroll
    for (int k = 0; k < P::kNA; ++k) {
      const unsigned back = (unsigned)max(pl.acb[k] - nvalid + 1, 0);
      st.va[k] = *reinterpret_cast<const u32x4_t *>(abase + pl.asrc[k] - back * kAStride);
    }
#pragma unroll
    for (int k = 0; k < P::kNW; ++k) {
      const unsigned back = (unsigned)max(pl.wcb[k] - nvalid + 1, 0);
      st.vw[k] = *reinterpret_cast<const u32x4_t *>(wbase + pl.wsrc[k] - back * kChunkBytes);
    }
    if (!DOTS && (int)threadIdx.x < P::kNS) {
      const unsigned back = (unsigned)max(pl.scb - nvalid + 1, 0);
      st.vs = *reinterpret_cast<const u32x4_t *>(sbase + pl.ssrc - back * (kTile * 4));
    }
    if constexpr (ACT != kActBf16 && !DOTS) {
#pragma unroll
      for (int k = 0; k < GemmShape<ACT, BM>::kDxPer; ++k)
        st.dx[k] = dxbase[pl.dxsrc[k] - (unsigned)max(pl.dxcb[k] - nvalid + 1, 0)];
    }
  }
}

// Write a loaded stage into LDS buffer `buf`.
template <int ACT, int BM, bool DOTS>
__device__ __forceinline__ void gemm_store(const GemmStaging<ACT, BM> &st,
                                           const GemmPlan<ACT, BM> &pl, char *buf) {
  using S = GemmShape<ACT, BM>;
  using P = GemmPlan<ACT, BM>;
#pragma unroll
  for (int k = 0; k < P::kNA; ++k) {
    if constexpr (ACT != kActBf16) {
      *reinterpret_cast<u32x2_t *>(buf + pl.adst[k]) = u32x2_t{st.va[k].x, st.va[k].y};
      *reinterpret_cast<u32x2_t *>(buf + pl.adst2[k]) = u32x2_t{st.va[k].z, st.va[k].w};
    } else {
      *reinterpret_cast<u32x4_t *>(buf + pl.adst[k]) = st.va[k];
    }
  }
#pragma unroll
  for (int k = 0; k < P::kNW; ++k) {
    if constexpr (ACT == kActBf16) {
      // 16 int8 values of column c (piece q = h * 64 + c) -> two 8-value bf16
      // parts; part p sits at (p ^ w_part_swizzle(c)) * 16 so that neither
      // these writes nor the operand reads stall on LDS banks
      const int c = (k * kGemmThreads + (int)threadIdx.x) & 63;
      const int sw = w_part_swizzle(c);
      const bf16x8_t lo = i8x8_to_bf16(make_uint2(st.vw[k].x, st.vw[k].y));
      const bf16x8_t hi = i8x8_to_bf16(make_uint2(st.vw[k].z, st.vw[k].w));
      *reinterpret_cast<bf16x8_t *>(buf + pl.wdst[k] + sw * 16) = lo;
      *reinterpret_cast<bf16x8_t *>(buf + pl.wdst[k] + (sw ^ 1) * 16) = hi;
    } else {
      *reinterpret_cast<u32x4_t *>(buf + pl.wdst[k]) = st.vw[k];
    }
  }
  if (!DOTS && (int)threadIdx.x < P::kNS) *reinterpret_cast<u32x4_t *>(buf + pl.sdst) = st.vs;
  if constexpr (ACT != kActBf16 && !DOTS) {
    float *dxs = reinterpret_cast<float *>(buf + S::kA);
#pragma unroll
    for (int k = 0; k < S::kDxPer; ++k) {
      const int p = k * kGemmThreads + (int)threadIdx.x;
      if (p < kGemmCB * BM) dxs[p] = st.dx[k];
    }
  }
}

// Two workgroups per CU (8 waves): the register budget is then 256 per lane,
// which the accumulators, the in-flight stage and its descriptors need.
// PARTS: several weights of one activation (the pages' GemmParts above the
// GEMV's rows, plan.rs merged_projections): the column blocks of part p are
// blocks cum[p] .. cum[p+1]-1 of the grid, and a workgroup takes its part's
// weight, output, width and bias; y = x.W_p + bias_p, pad columns 0.
template <int ACT, int BM, bool DOTS, bool PARTS>
__global__ void __launch_bounds__(kGemmThreads) __attribute__((amdgpu_waves_per_eu(1, 2)))
gemm_kernel(const void *__restrict__ xv, const int8_t *__restrict__ wq,
            const float *__restrict__ wsc, float *__restrict__ y, int32_t *__restrict__ dots,
            int m, int K, int NB, int Npad, int T, int MB, int NBN, unsigned act_scale_off,
            Parts parts) {
  using S = GemmShape<ACT, BM>;
  extern __shared__ __attribute__((aligned(16))) char lds[];

  // XCD-aware numbering: workgroups are dealt round-robin over the 8 XCDs,
  // so (when the grid divides) give XCD x the logical range x*G/8 ...
  const int G = MB * NBN;
  const int bid = (int)blockIdx.x;
  const int logical = (G % 8 == 0) ? (bid % 8) * (G / 8) + bid / 8 : bid;
  const int mb = logical % MB;
  int nb = logical / MB;
  const float *bias = nullptr;
  int N = Npad;
  if constexpr (PARTS) {
    int p = 0;
#pragma unroll
    for (int i = 1; i < kMaxParts; ++i)
      if (i < parts.n && nb >= parts.cum[i]) p = i;
    nb -= parts.cum[p];
    wq = parts.wq[p];
    wsc = parts.wsc[p];
    y = parts.y[p];
    bias = parts.bias[p];
    N = parts.N[p];
    Npad = (N + kTile - 1) / kTile * kTile;
    T = Npad / kTile;
  }
  const int row0 = mb * BM, t0 = nb * S::WN;

  const int lane = threadIdx.x & 63;
  const int li = lane & 15, lj = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int wm = wave / S::WN, wn = wave % S::WN;
  const int t = t0 + wn;   // this wave's 64-column tile

  f32x4_t acc[4][4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int g = 0; g < 4; ++g) acc[rt][g] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  const int NC = (NB + kGemmCB - 1) / kGemmCB;
  constexpr int kElt = ACT == kActBf16 ? 2 : 1;
  GemmPlan<ACT, BM> pl;
  gemm_plan<ACT, BM>(pl, m, K, NB, T, row0, t0);
  // the regions' bases at stage 0; each stage advances them by kGemmCB blocks
  const char *abase = static_cast<const char *>(xv) + (size_t)row0 * K * kElt;
  const char *wbase = reinterpret_cast<const char *>(wq) + (size_t)t0 * NB * kChunkBytes;
  const char *sbase = reinterpret_cast<const char *>(wsc) + (size_t)t0 * NB * kTile * 4;
  const float *dxbase = reinterpret_cast<const float *>(static_cast<const char *>(xv) +
                                                        act_scale_off) + (size_t)row0 * NB;
  // lane's bytes of a chunk: half j/2, column 16g + i, k offset 8 * (j % 2)
  const int w_lane = (lj >> 1) * kHalfBytes + li * 16 + (lj & 1) * 8;
  // bf16 form: half j/2 at 2048 * (j/2), column 16g + i at 32 * (16g + i), the
  // lane's 8 values (part j % 2) at the swizzled 16-byte offset
  const int wb_lane = (lj >> 1) * 2 * kHalfBytes + li * 32 + (((lj & 1) ^ w_part_swizzle(li)) * 16);
  // lane's activation bytes within a row (rows 16rt + i: the swizzle depends on i)
  const int a_lane = a_part<ACT>(li, lj);

  // One stage (blocks b0 .. b0 + kGemmCB - 1) from LDS buffer `buf`.
  auto compute = [&](const char *buf, int b0) {
#pragma unroll
    for (int cb = 0; cb < kGemmCB; ++cb) {
      const int b = b0 + cb;
      if (b >= NB) break;
      const char *As = buf + cb * S::kRowsA * S::kRowB;
      const char *Ws = buf + S::kA + S::kDx + (wn * kGemmCB + cb) * kChunkBytes * S::kWElt;
      float4 sc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      if constexpr (!DOTS)
        sc = *reinterpret_cast<const float4 *>(buf + S::kA + S::kDx + S::kWL +
                                               ((wn * kGemmCB + cb) * kTile + 4 * li) * 4);
      const float scs[4] = {sc.x, sc.y, sc.z, sc.w};
      if constexpr (ACT == kActBf16) {
        bf16x8_t bb[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) bb[g] = *reinterpret_cast<const bf16x8_t *>(Ws + wb_lane + g * 512);
        // Per row group: the four MFMAs first (independent, so the matrix
        // core pipelines them), then their sixteen scale FMAs.
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          const bf16x8_t a = *reinterpret_cast<const bf16x8_t *>(
              As + (wm * 64 + rt * 16 + li) * S::kRowB + a_lane);
          f32x4_t d[4];
#pragma unroll
          for (int g = 0; g < 4; ++g)
            d[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bb[g],
                                                           f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
#pragma unroll
          for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[rt][g][e] = fmaf(scs[g], d[g][e], acc[rt][g][e]);
        }
      } else if constexpr (ACT == kActQ8x2) {
        // Two words: the first words' and the second words' int8 MFMAs meet
        // exactly in int32 (|128 D_hi + D_lo| < 2^27), then one FMA with the
        // block's dx * s / 128.
        uint2 bw[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) bw[g] = *reinterpret_cast<const uint2 *>(Ws + w_lane + g * 256);
        const float *dxs = reinterpret_cast<const float *>(buf + S::kA) + cb * BM;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          const long ahi = *reinterpret_cast<const long *>(
              As + (wm * 64 + rt * 16 + li) * S::kRowB + a_lane);
          const long alo = *reinterpret_cast<const long *>(
              As + (BM + wm * 64 + rt * 16 + li) * S::kRowB + a_lane);
          const float4 d4 = *reinterpret_cast<const float4 *>(dxs + wm * 64 + rt * 16 + lj * 4);
          const float dxv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const long b8 = __builtin_bit_cast(long, bw[g]);
            const i32x4_t dh =
                __builtin_amdgcn_mfma_i32_16x16x32_i8(ahi, b8, i32x4_t{0, 0, 0, 0}, 0, 0, 0);
            const i32x4_t dl =
                __builtin_amdgcn_mfma_i32_16x16x32_i8(alo, b8, i32x4_t{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              acc[rt][g][e] = fmaf(dxv[e] * scs[g], (float)(dh[e] * 128 + dl[e]) * 0.0078125f,
                                   acc[rt][g][e]);
          }
        }
      } else {
        uint2 bw[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) bw[g] = *reinterpret_cast<const uint2 *>(Ws + w_lane + g * 256);
        const float *dxs = reinterpret_cast<const float *>(buf + S::kA) + cb * BM;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          const long a = *reinterpret_cast<const long *>(
              As + (wm * 64 + rt * 16 + li) * S::kRowB + a_lane);
          float dxv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
          if constexpr (!DOTS) {
            const float4 d4 = *reinterpret_cast<const float4 *>(dxs + wm * 64 + rt * 16 + lj * 4);
            dxv[0] = d4.x; dxv[1] = d4.y; dxv[2] = d4.z; dxv[3] = d4.w;
          }
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const i32x4_t d = __builtin_amdgcn_mfma_i32_16x16x32_i8(
                a, __builtin_bit_cast(long, bw[g]), i32x4_t{0, 0, 0, 0}, 0, 0, 0);
            if constexpr (DOTS) {
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int r = row0 + wm * 64 + rt * 16 + lj * 4 + e;
                if (r < m && t < T)
                  dots[((size_t)r * NB + b) * Npad + (size_t)t * kTile + g * 16 + li] = d[e];
              }
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                acc[rt][g][e] = fmaf(dxv[e] * scs[g], (float)d[e], acc[rt][g][e]);
            }
          }
        }
      }
    }
  };
  // The global loads of stage c (its region bases moved by c stages).
  auto load = [&](GemmStaging<ACT, BM> &st, int c) {
    const int b0 = c * kGemmCB;
    gemm_load<ACT, BM, DOTS>(st, pl, abase + (size_t)b0 * kBlock * kElt,
                             wbase + (size_t)b0 * kChunkBytes,
                             sbase + (size_t)b0 * kTile * 4, dxbase + b0,
                             min(NB - b0, kGemmCB));
  };

  // Pipeline: LDS double-buffered, and the global loads of each stage issued
  // two stages ahead of its compute (into the register set freed when the
  // stage before it went to LDS), so a load has two stages' compute to land.
  GemmStaging<ACT, BM> r0, r1;
  char *buf0 = lds, *buf1 = lds + S::kStage;
  load(r0, 0);
  gemm_store<ACT, BM, DOTS>(r0, pl, buf0);
  if (NC > 1) load(r1, 1);
  __syncthreads();
  for (int c = 0;;) {
    // buf0 holds stage c, r1 stage c + 1 (in flight)
    if (c + 2 < NC) load(r0, c + 2);
    compute(buf0, c * kGemmCB);
    if (c + 1 < NC) gemm_store<ACT, BM, DOTS>(r1, pl, buf1);
    __syncthreads();
    if (++c >= NC) break;
    // buf1 holds stage c, r0 stage c + 1
    if (c + 2 < NC) load(r1, c + 2);
    compute(buf1, c * kGemmCB);
    if (c + 1 < NC) gemm_store<ACT, BM, DOTS>(r0, pl, buf0);
    __syncthreads();
    if (++c >= NC) break;
  }
  if constexpr (DOTS) return;

  if (t >= T) return;
  // the part's bias on its real columns (pad columns stay the exact zero of
  // zero values and scales)
  float bv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if constexpr (PARTS) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int c = t * kTile + g * 16 + li;
      if (bias && c < N) bv[g] = bias[c];
    }
  }
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = row0 + wm * 64 + rt * 16 + lj * 4 + e;
      if (r < m) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float v = acc[rt][g][e];
          if constexpr (PARTS) {
            if (t * kTile + g * 16 + li < N) v += bv[g];
          }
          y[(size_t)r * Npad + (size_t)t * kTile + g * 16 + li] = v;
        }
      }
    }
}

template <int ACT, int BM, bool DOTS, bool PARTS>
hipError_t launch_gemm_kp(const GemmArgs &a, hipStream_t stream) {
  using S = GemmShape<ACT, BM>;
  const int MB = (a.m + BM - 1) / BM;
  // parts: each part's tiles start a new column block
  Parts parts = a.parts;
  int NBN = (a.T + S::WN - 1) / S::WN;
  if constexpr (PARTS) {
    NBN = 0;
    for (int i = 0; i < parts.n; ++i) {
      const int tiles = a.parts.cum[i + 1] - a.parts.cum[i];
      parts.cum[i] = NBN;
      NBN += (tiles + S::WN - 1) / S::WN;
    }
    parts.cum[parts.n] = NBN;
  }
  const size_t lds = 2 * (size_t)S::kStage;
  auto kern = gemm_kernel<ACT, BM, DOTS, PARTS>;
  static bool granted = false;
  if (!granted && lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    granted = true;
  }
  (void)hipGetLastError();
  kern<<<dim3((unsigned)(MB * NBN)), dim3(kGemmThreads), lds, stream>>>(
      a.x, a.wq, a.wsc, a.y, a.dots, a.m, a.K, a.NB, a.Npad, a.T, MB, NBN, a.act_scale_off,
      parts);
  return hipGetLastError();
}

// One weight, or (a.parts.n > 0, no dots) the parts.
template <int ACT, int BM, bool DOTS>
hipError_t launch_gemm_k(const GemmArgs &a, hipStream_t stream) {
  if constexpr (!DOTS) {
    if (a.parts.n > 0) return launch_gemm_kp<ACT, BM, false, true>(a, stream);
  }
  return launch_gemm_kp<ACT, BM, DOTS, false>(a, stream);
}

}  // namespace

int gemm_rows_per_block(int64_t m) { return m > 64 ? 128 : 64; }

hipError_t launch_gemm(int act, bool write_dots, int bm, const GemmArgs &a, hipStream_t stream) {
  if (act == kActBf16 && !write_dots) {
    if (bm == 64) return launch_gemm_k<kActBf16, 64, false>(a, stream);
    if (bm == 128) return launch_gemm_k<kActBf16, 128, false>(a, stream);
  }
  if (act == kActQ8) {
    if (bm == 64)
      return write_dots ? launch_gemm_k<kActQ8, 64, true>(a, stream)
                        : launch_gemm_k<kActQ8, 64, false>(a, stream);
    if (bm == 128)
      return write_dots ? launch_gemm_k<kActQ8, 128, true>(a, stream)
                        : launch_gemm_k<kActQ8, 128, false>(a, stream);
  }
  if (act == kActQ8x2 && !write_dots) {
    if (bm == 64) return launch_gemm_k<kActQ8x2, 64, false>(a, stream);
    if (bm == 128) return launch_gemm_k<kActQ8x2, 128, false>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace q8
