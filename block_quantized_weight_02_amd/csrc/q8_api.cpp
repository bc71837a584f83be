// q8_api.cpp -- host side of the C ABI declared in include/q8gemv.h:
// argument validation (before any launch), the launch plan, the split-K
// workspace cache, and error reporting.
//
// Shape rules follow docs.logicaffeine.com, logicaffeine_compile/spatial/
// passes/from_q8.rs, fn q8_gemv_applies (1 <= m <= 32 rows, K > 0 and whole
// 32-row blocks, N > 0, the last column tile zero-padded) and the whole-block
// check of codegen_cuda/lane/plan.rs, fn whole_blocks, whose error names the
// declared length and the next whole bound.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <map>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "../../include/q8gemv.h"
#include "q8_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return Q8_OK;
}

}  // namespace

namespace q8 {
int report_error(int status, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}
}  // namespace q8

namespace {

int64_t round_up(int64_t v, int64_t to) { return (v + to - 1) / to * to; }

// Largest sizes the 32-bit launch arithmetic admits (checked, not assumed).
constexpr int64_t kMaxK = int64_t(1) << 24;
constexpr int64_t kMaxN = int64_t(1) << 24;

int check_kn(int64_t K, int64_t N) {
  if (K <= 0 || K > kMaxK)
    return fail(Q8_ERR_SHAPE, "K = %lld out of range: need 0 < K <= %lld",
                (long long)K, (long long)kMaxK);
  if (K % Q8_BLOCK != 0)
    return fail(Q8_ERR_SHAPE,
                "K = %lld is not whole %d-row blocks: declared %lld, bound %lld",
                (long long)K, Q8_BLOCK, (long long)K,
                (long long)round_up(K, Q8_BLOCK));
  if (N < 1 || N > kMaxN)
    return fail(Q8_ERR_SHAPE, "N = %lld out of range: need 1 <= N <= %lld",
                (long long)N, (long long)kMaxN);
  if (K * round_up(N, Q8_TILE_COLS) >= (int64_t(1) << 40))
    return fail(Q8_ERR_SHAPE, "K*N_pad = %lld exceeds 2^40",
                (long long)(K * round_up(N, Q8_TILE_COLS)));
  return Q8_OK;
}

int check_m(int64_t m, int64_t max_rows = Q8_MAX_ROWS) {
  if (m < 1 || m > max_rows)
    return fail(Q8_ERR_SHAPE, "m = %lld out of range: need 1 <= m <= %lld",
                (long long)m, (long long)max_rows);
  return Q8_OK;
}

int check_act(int act_fmt) {
  if (act_fmt != Q8_ACT_BF16 && act_fmt != Q8_ACT_Q8_0 && act_fmt != Q8_ACT_Q8_0_TWO_WORDS)
    return fail(Q8_ERR_ACT_FMT,
                "act_fmt = %d: no kernel for it (0 bf16, 1 Q8_0, 2 Q8_0 two words)", act_fmt);
  return Q8_OK;
}

// Rows of a product for its activation format (two words: at most 16).
int check_m_act(int64_t m, int act_fmt) {
  int st = check_m(m);
  if (st) return st;
  if (act_fmt == Q8_ACT_Q8_0_TWO_WORDS) return check_m(m, Q8_MAX_TWO_WORD_ROWS);
  return Q8_OK;
}

// The products that take no two-word activation.
// The format, and the row limit of two-word activations.
int check_act_rows(int act_fmt, int64_t m) {
  int st = check_act(act_fmt);
  if (st) return st;
  if (act_fmt == Q8_ACT_Q8_0_TWO_WORDS) return check_m(m, Q8_MAX_TWO_WORD_ROWS);
  return Q8_OK;
}

int check_ptr(const void *p, const char *name) {
  if (!p) return fail(Q8_ERR_NULL, "%s is NULL", name);
  if (reinterpret_cast<uintptr_t>(p) % 16 != 0)
    return fail(Q8_ERR_ALIGN, "%s = %p is not 16-byte aligned", name, p);
  return Q8_OK;
}

int hip_fail(hipError_t e, const char *what) {
  return fail(Q8_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t act_scales_offset(int64_t m, int64_t K) {
  return (size_t)round_up(m * K, 256);
}

// Offset of the one-word buffer's block-interleaved view of the codes.
size_t act_view_offset(int64_t m, int64_t K) {
  return (size_t)round_up((int64_t)act_scales_offset(m, K) + m * (K / Q8_BLOCK) * 4, 256);
}

// Offset of the scales in the activation buffer of a format: the two-word
// form holds 2m rows of words before its scales.
size_t act_scales_offset_of(int act_fmt, int64_t m, int64_t K) {
  return act_scales_offset(act_fmt == Q8_ACT_Q8_0_TWO_WORDS ? 2 * m : m, K);
}

// Most K splits of a plan (the splits are the launch grid's second
// dimension).
constexpr int kMaxSplits = 65535;

// LDS per workgroup kept free for the kernels' static shared variables.
constexpr size_t kStaticLdsReserve = 1024;

// ---- device facts -----------------------------------------------------------

struct DeviceFacts {
  int cus = 256;
  int lds_per_block = 64 * 1024;
};

DeviceFacts device_facts() {
  DeviceFacts f;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return f;
  static std::mutex mu;
  static std::map<int, DeviceFacts> cache;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(dev);
  if (it != cache.end()) return it->second;
  int v = 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
    f.cus = v;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) == hipSuccess &&
      v > 0)
    f.lds_per_block = v;
  cache[dev] = f;
  return f;
}

// ---- plans --------------------------------------------------------------------

int rows_for(int64_t m) {
  int r = 1;
  while (r < m) r *= 2;
  return r;
}

// The default launch (settled by measurement on MI355X):
//  * VALU kernel (lane per column) up to 2 rows, the rows whose activation
//    it prefetches into scalar registers with each weight stage; MFMA kernel
//    above (the reasons and figures are at the VALU branch below).
//  * VALU: 8 waves per workgroup for 1 row, 16 for 2; K split across
//    workgroups only when the column tiles alone leave CUs idle (splits =
//    CUs / tiles, each split at least 40 blocks: the split-K combine costs
//    more than the extra workgroups gain below that; measured on MI355X,
//    m = 1, K = 1024, N = 1024: 1 split 3.9-4.0 us against 4 splits 5.1;
//    K = 4096, N = 4096: 3 splits 7.1-7.2 against 2 splits 7.3-7.5 and
//    4 splits 7.6-7.7).
//  * MFMA (see below): 16 waves; the fewest K splits whose staged activation
//    fits the LDS, more (each at least 32 blocks) while the splits still fit
//    one workgroup per CU.  Block-interleaved, except for 17-32 rows whose
//    LDS splits alone give more workgroups than CUs: there the column-group
//    form.
// Rows up to which two-word activations take the VALU kernel (the rows whose
// activation it prefetches; from 3 rows the MFMA kernel, whose 32-row tile
// holds both words of up to 16 rows).
constexpr int64_t kValuTwoWordRows = 2;

// One-word Q8_0 activations of 17-32 rows take the tile-per-workgroup
// 32x32x32 kernel (MFMA32_TILE; a product of one weight only).  Measured on MI355X against the
// block-interleaved and column-group kernels (us, rows 17 / 24 / 32):
// K=5120, N=32000: 36.6 / 37.5 / 39.2 against 45.7 / 47.2 / 48.8 (column-
// group, 2 splits); K=4096, N=14336: 16.9 / 17.4 / 18.0 against 18.1 / 19.4 /
// 20.1; N=4096: 11.1 / 11.3 / 11.6 against 12.9 / 13.1 / 13.3; N=1024: 10.3 /
// 10.6 / 10.9 against 11.7 / 11.9 / 12.0; K=5120, N=40: 10.4 / 10.3 / 10.6
// against 11.2 / 11.4 / 11.6.  8 waves from 384 tiles (N=32000: 39.2 against
// 44.2 us with 16), else 16 (N=14336: 18.0 against 21.1); K split only below
// 128 tiles: 3 ways from 8 tiles (N=4096: 11.5 against 11.8 with 4 and 12.4
// with 2; N=1024: 10.9 against 11.0 with 4), 4 ways below (N=40: 10.6 against
// 11.4 with 5).  Up to 16 rows the 16-row kernels stay ahead (the
// block-interleaved one at m=16, N=32000: 34.4 against 36.3 us; N=14336: 16.0
// against 16.9), and the 16-row tile kernel below is faster still.

// Raises a tile plan's K split until its LDS (the split's activation scales
// and the carries) fits a workgroup.
void fit_tile_lds(q8_plan &p, int64_t NB, int act_fmt) {
  const size_t budget = (size_t)device_facts().lds_per_block - kStaticLdsReserve;
  int64_t S = p.split_k;
  while (S < NB && q8::gemv_lds_bytes(p.kernel, p.rows, act_fmt, p.waves, p.kslices, (int)NB,
                                      (int)S) > budget)
    ++S;
  p.split_k = (int32_t)S;
}

q8_plan tile32_plan(int64_t K, int64_t N) {
  const int64_t NB = K / Q8_BLOCK;
  const int64_t T = round_up(N, Q8_TILE_COLS) / Q8_TILE_COLS;
  q8_plan p;
  p.kernel = Q8_KERNEL_MFMA32_TILE;
  p.rows = 32;
  // From 384 tiles each wave covers two column tiles (one activation load
  // serves four MFMAs; half the workgroups still cover the CUs).  Measured on
  // MI355X (loop us, two tiles against one, 8 waves): K=5120, N=32000: m=17
  // 35.6 against 37.3, m=24 36.4 against 38.3-38.8, m=32 39.6 against 39.4;
  // K=8192, N=32000, m=32: 57.7 against 61.3.  Below 384 tiles one (m=32,
  // K=4096, N=14336: 24.2 against 17.6-17.7 with 16 waves).
  p.kslices = T >= 384 ? 2 : 1;
  p.waves = T >= 384 ? 8 : 16;
  int64_t S = T >= 128 ? 1 : (T >= 8 ? 3 : 4);
  const int64_t smax = NB / 8 > 0 ? NB / 8 : 1;
  if (S > smax) S = smax;
  p.split_k = (int32_t)S;
  fit_tile_lds(p, NB, Q8_ACT_Q8_0);
  return p;
}

// 3-16 rows (bf16 or one-word Q8_0) take the tile-per-workgroup 16x16x32
// kernel (MFMA16_TILE) (Q8_0: 16 waves; bf16: below), K split only below 128 tiles (256 / tiles
// ways, at most 8).  Measured on MI355X against the block-interleaved MFMA
// kernel (us, rows 3 / 8 / 16): bf16, K=4096, N=14336: 13.2 / 13.5 / 15.5
// against 14.8 / 14.9 / 15.7; K=5120, N=32000: 30.9 / 30.7 / 35.1 against
// 37.1 / 38.9 / 40.7; K=4096, N=4096 (4 splits): 8.2 / 8.2 / 8.4 against 9.3 /
// 9.3 / 9.5; N=1024 (8 splits): 6.7 / 6.9 / 7.1 against 8.4 / 8.5 / 8.6.
// Q8_0, K=4096, N=14336: 13.6 / 13.9 / 14.1 against 15.2 / 15.6 / 16.1;
// K=5120, N=32000: 31.5 / 31.8 / 32.1 against 31.9 / 33.2 / 34.4.
//
// 17-32 bf16 rows take the same kernel with two row groups of 16 (rows 32), 8
// waves, one-block stages; measured on MI355X against the column-group and
// block-interleaved kernels the single-product plan took before (loop us):
// K=4096, N=14336: m=24 18.2 against 23.0, m=32 19.9 against 23.0 (16 waves
// 20.0); K=5120, N=32000, m=32: 46.8 against 58.0 (4 waves 48.4); K=4096,
// N=4096 (4 splits), m=32: 11.5 against 12.2.
q8_plan tile16_plan(int64_t m, int64_t K, int64_t N, int act_fmt) {
  const int64_t NB = K / Q8_BLOCK;
  const int64_t T = round_up(N, Q8_TILE_COLS) / Q8_TILE_COLS;
  q8_plan p;
  p.kernel = Q8_KERNEL_MFMA16_TILE;
  p.rows = m <= 16 ? 16 : 32;
  p.kslices = 1;
  p.waves = 16;
  // bf16, swept on MI355X (loop us, best plan against the next form):
  //   K = 4096, N = 14336: m <= 12 one-block stages of 8 waves (m = 3, 6, 12:
  //     12.8, 13.0, 13.5); m = 16 two-block stages of 16 waves (14.1, one-block
  //     14.4);
  //   K = 5120, N = 32000: m <= 9 one-block stages of 8 waves (30.9, 31.1, 31.6
  //     at m = 3, 6, 9); m = 12, 16 two-block stages of 4 waves (32.0, 33.3
  //     against 32.8, 34.3);
  //   K = 4096, N = 4096 (4 splits): one-block stages, 8 waves up to 8 rows
  //     (m = 3: 8.0 against 8.2), 16 above (m = 16: 8.4 against 8.8).
  if (act_fmt == Q8_ACT_BF16 && m > 16) {
    p.waves = 8;
  } else if (act_fmt == Q8_ACT_BF16) {
    if (T >= 384) {
      p.kslices = m >= 12 ? 2 : 1;
      p.waves = m >= 12 ? 4 : 8;
    } else if (T >= 128) {
      p.kslices = m >= 13 ? 2 : 1;
      p.waves = m >= 13 ? 16 : 8;
    } else {
      p.waves = m <= 8 ? 8 : 16;
    }
  }
  int64_t S = T >= 128 ? 1 : 256 / T;
  if (S > 8) S = 8;
  const int64_t smax = NB / 8 > 0 ? NB / 8 : 1;
  if (S > smax) S = smax;
  if (S < 1) S = 1;
  p.split_k = (int32_t)S;
  fit_tile_lds(p, NB, act_fmt);
  // two-block stages only where the last K split has an even block count
  if (p.kslices == 2 && (NB / p.split_k) % 2 != 0) {
    p.kslices = 1;
    p.waves = 8;
  }
  return p;
}

// The many-row product at few rows of bf16 or one-word Q8_0: the GEMM gives
// each workgroup 64 or 128 rows by four or two column tiles, so at these rows
// it runs one workgroup per several tiles, too few to cover the CUs.  Instead
// each column tile streams through the tile-per-workgroup kernel (MFMA16_TILE,
// 16, 32 or 64 rows a wave; above 64 rows one workgroup per tile and chunk of
// 64 rows), without a K split, so that it needs no workspace.  Up to 64 rows
// always; up to 1024 while the workgroups (tiles x chunks) stay within 512
// (bf16) or 1024 (int8, whose GEMM is slower).  Measured on MI355X (loop us,
// tile kernel against the GEMM), K = 4096: bf16 N = 14336: m = 65 45.8
// against 69.9, m = 128 54.8 against 70.8, m = 160 72.8 against 72.9, m = 192
// 80.9 against 73.4; bf16 m = 128: N = 4096 26.5 against 68.2, N = 8192 27.8
// against 69.2, N = 20480 80.1 against 72.4; bf16 m = 96, N = 24576 77.9
// against 73.0; m = 256, N = 4096 27.3 against 68.3 (int8 28.3 against
// 125.6); int8 N = 14336: m = 128 54.0 against 129.0, m = 192 79.5 against
// 129.2, m = 256 106.8 against 130.5; K = 5120, N = 32000: bf16 m = 64 70.9
// against 98.9, m = 96 124.3 against 93.4, m = 128 140.3 against 96.1; int8
// m = 128 133.3 against 168.2, m = 160 190.8 against 191.6; bf16 m = 384 and
// 512, N = 4096: 51.8 and 53.8 against 69.2 and 70.0; m = 512, N = 2048 and
// 1024: 27.5 and 25.8 against 68.2 and 67.5; m = 1024, N = 1024: 27.4
// against 66.5; K = 14336, m = 512, N = 4096: 164.5 against 228.8; int8
// m = 512, N = 4096 and 8192: 55.2 and 109.2 against 126.2 and 129.6;
// m = 1024, N = 2048: 57.3 against 126.0.  The choice depends on m, K, the
// format and the width; q8_gemm_parts takes it for all its parts' columns
// (q/k/v at m = 512, N = 4096 + 1024 + 1024, 768 workgroups: each part on
// the tile kernel in one launch 80.7 us, the GEMM 73.4).
struct GemmTileRoute {
  bool on;
  int rows, waves, kslices;
};
constexpr int64_t kTileRouteRows = 1024;
GemmTileRoute gemm_tile_route(int64_t m, int64_t K, int64_t N, int act_fmt) {
  GemmTileRoute r{false, 0, 0, 1};
  if (m > kTileRouteRows || (act_fmt != Q8_ACT_BF16 && act_fmt != Q8_ACT_Q8_0)) return r;
  if (act_fmt == Q8_ACT_Q8_0 && act_view_offset(m, K) > 0xffffffffull) return r;
  const int64_t chunks = (m + 63) / 64;
  const int64_t T = round_up(N, Q8_TILE_COLS) / Q8_TILE_COLS;
  if (chunks > 1 && T * chunks > (act_fmt == Q8_ACT_BF16 ? 512 : 1024)) return r;
  r.rows = m <= 16 ? 16 : (m <= 32 ? 32 : 64);
  const size_t budget = (size_t)device_facts().lds_per_block - kStaticLdsReserve;
  for (int w : {8, 4}) {
    if (q8::tile16_lds_bytes(r.rows, act_fmt, w, (int)(K / Q8_BLOCK), 1) <= budget) {
      r.waves = w;
      r.on = true;
      return r;
    }
  }
  return r;
}

// tiles: the tile-per-workgroup kernels may be chosen (they run one weight:
// the gated pair and the parts pass false).
q8_plan default_plan(int64_t m, int64_t K, int64_t N, int act_fmt, bool tiles = true) {
  const int64_t NB = K / Q8_BLOCK;
  const int64_t T = round_up(N, Q8_TILE_COLS) / Q8_TILE_COLS;
  const DeviceFacts dev = device_facts();
  const int64_t smax = NB / 40 > 0 ? NB / 40 : 1;
  if (tiles && act_fmt == Q8_ACT_Q8_0 && m > 16) return tile32_plan(K, N);
  if (tiles && act_fmt != Q8_ACT_Q8_0_TWO_WORDS && m > 2 && (m <= 16 || act_fmt == Q8_ACT_BF16))
    return tile16_plan(m, K, N, act_fmt);
  q8_plan p;
  p.kslices = 1;
  if (act_fmt == Q8_ACT_Q8_0_TWO_WORDS && m <= kValuTwoWordRows) {
    // Few rows: the VALU kernel, two sdot4 passes per block and row
    // (m = 1, K = 4096, N = 14336: 12.7 us against 16.0 on the MFMA kernel).
    p.kernel = Q8_KERNEL_VALU;
    p.rows = rows_for(m);
    p.waves = p.rows >= 2 ? 16 : 8;
    int64_t S = dev.cus / T;
    if (S > smax) S = smax;
    if (S < 1) S = 1;
    p.split_k = (int32_t)S;
    return p;
  }
  if (act_fmt == Q8_ACT_Q8_0_TWO_WORDS) {
    // The block-interleaved MFMA kernel, its 32 rows the two words' 16 each;
    // K split for the LDS, then further (each split at least 32 blocks)
    // while the splits still fill one workgroup per CU.
    p.kernel = Q8_KERNEL_MFMA;
    p.rows = 32;
    p.waves = 16;
    const size_t budget = (size_t)dev.lds_per_block - kStaticLdsReserve;
    int64_t S = 1;
    while (S < NB && q8::gemv_lds_bytes(p.kernel, p.rows, act_fmt, p.waves, p.kslices, (int)NB,
                                        (int)S) > budget)
      ++S;
    while (S < NB / 32 && T * (S + 1) <= dev.cus) ++S;
    p.split_k = (int32_t)S;
    return p;
  }
  // The VALU kernel up to 2 rows: there the activation of each stage is
  // prefetched into scalar registers with the weight; from 3 rows it is read
  // when used, and when the activation has just been written (by its
  // producer, as in a decode step) those reads miss the caches.  Measured on
  // MI355X, K = 4096, N = 14336, activation rewritten before every product
  // (rewrite included): bf16 m = 3: 17.6 us VALU against 16.3 MFMA; int8
  // m = 3: 20.8 against 17.3, m = 4: 23.9 against 17.4; 16 waves for 2 rows
  // (bf16 m = 2: 13.9 against 14.8 us with 8).
  if (m <= 2) {
    p.kernel = Q8_KERNEL_VALU;
    p.rows = rows_for(m);
    p.waves = p.rows >= 2 ? 16 : 8;
    int64_t S = dev.cus / T;
    if (S > smax) S = smax;
    if (S < 1) S = 1;
    p.split_k = (int32_t)S;
    return p;
  }
  // Matrix cores.  The block-interleaved kernel: waves split K and each
  // covers the whole tile, so one LDS fragment read serves four MFMAs.  For
  // 17-32 rows whose 32-row stage needs K splits that already give more
  // workgroups than CUs, the column-group kernel instead: each wave owns a
  // 16-column group and the workgroup walks tiles with the activation staged
  // once, so no split beyond the LDS's is paid for.  Measured on MI355X
  // (int8, m = 32, K = 5120, where the stage needs 2 splits): N = 40
  // block-interleaved 11.4 us against column-group 16.6; N = 4096 13.4
  // against 22.2; N = 8192 16.4 against 22.2 (its best); N = 14336 (448
  // workgroups) 28.2 against 26.7, N = 32000 52.0 against 49.9.  m = 24,
  // K = 4096, N = 14336 (one split): 17.8 against 24.7.  bf16, m = 32,
  // K = 4096 (2 splits): N = 4096 block-interleaved 12.0 against 13.0;
  // N = 14336 25.1 against 23.2.  int8, m = 16, K = 4096, N = 14336: 16.2 us
  // block-interleaved against 24-52 us column-group over its splits and
  // widths.
  p.kernel = Q8_KERNEL_MFMA;
  p.rows = m <= 16 ? 16 : 32;
  p.waves = 16;
  p.kslices = 1;
  const size_t budget = (size_t)dev.lds_per_block;
  const auto lds_splits = [&](const q8_plan &pl) {
    int64_t s = 1;
    while (s < NB && q8::gemv_lds_bytes(pl.kernel, pl.rows, act_fmt, pl.waves, pl.kslices,
                                        (int)NB, (int)s) > budget - kStaticLdsReserve)
      ++s;
    return s;
  };
  int64_t S = lds_splits(p);
  if (m > 16 && T * S > dev.cus) {
    p.kernel = Q8_KERNEL_MFMA_COLS;
    S = lds_splits(p);
  }
  // Then more splits while they still fit one workgroup per CU, each split
  // at least 32 blocks: a narrow product's few tiles alone leave CUs idle.
  // Measured on MI355X: bf16, m = 4, K = 4096, N = 640: 1 split 12.2 us,
  // 4 splits 8.9, 16 splits 11.1; m = 16, N = 4096: 1 split 13.6, 4 splits
  // 10.2, 8 splits 15.0; int8, m = 32, K = 5120, N = 40: 3 splits 12.3,
  // 4 splits 11.4, 5 splits 11.7, 8 splits 12.1.
  const int64_t tiles_per_wg = p.kernel == Q8_KERNEL_MFMA_COLS ? p.waves / (4 * p.kslices) : 1;
  const int64_t wgs = (T + tiles_per_wg - 1) / tiles_per_wg;
  const int64_t smax_mfma = NB / 32 > 1 ? NB / 32 : 1;
  while (S < smax_mfma && wgs * (S + 1) <= dev.cus) ++S;
  p.split_k = (int32_t)S;
  return p;
}

int check_plan(const q8_plan *p, int64_t m, int64_t K, int act, bool dots) {
  if (!p) return fail(Q8_ERR_NULL, "plan is NULL");
  const int64_t NB = K / Q8_BLOCK;
  if (p->rows < m || p->rows > Q8_MAX_ROWS || (p->rows & (p->rows - 1)) != 0)
    return fail(Q8_ERR_PLAN, "plan rows = %d: need a power of two in [m = %lld, %d]",
                p->rows, (long long)m, Q8_MAX_ROWS);
  if (p->split_k < 1 || p->split_k > NB || p->split_k > kMaxSplits)
    return fail(Q8_ERR_PLAN, "plan split_k = %d: need 1 <= split_k <= min(K/32 = %lld, %d)",
                p->split_k, (long long)NB, kMaxSplits);
  if (!q8::gemv_instantiated(p->kernel, p->rows, act, dots, p->waves, p->kslices))
    return fail(Q8_ERR_PLAN,
                "no kernel built for kernel=%d rows=%d act=%d dots=%d waves=%d kslices=%d",
                p->kernel, p->rows, act, (int)dots, p->waves, p->kslices);
  // Two-block stages of the 16x16x32 tile kernel read a pair's two blocks of
  // every row as whole lines: a pair that started at the rows' last block
  // would read past the last row.  Its waves' pairs start at the split's
  // first block plus even offsets, so the last split (K/32 / split_k blocks)
  // must have an even count.
  if (p->kernel == Q8_KERNEL_MFMA16_TILE && p->kslices == 2 && (NB / p->split_k) % 2 != 0)
    return fail(Q8_ERR_PLAN, "two-block stages need an even block count in the last K split "
                "(K/32 / split_k = %lld): use kslices 1 or another split_k",
                (long long)(NB / p->split_k));
  if (p->kernel != Q8_KERNEL_VALU) {
    const size_t need =
        q8::gemv_lds_bytes(p->kernel, p->rows, act, p->waves, p->kslices, (int)NB, p->split_k);
    // keep room for the kernels' own static LDS (a few bytes of flags)
    const size_t have = (size_t)device_facts().lds_per_block - kStaticLdsReserve;
    if (need > have)
      return fail(Q8_ERR_PLAN, "plan needs %zu bytes of LDS per workgroup, the device has %zu: "
                  "raise split_k", need, have);
  }
  return Q8_OK;
}

// Workspace layout: arrival counters first, at fixed places for every shape
// (the VALU kernel uses one per 64-column tile, the MFMA kernel one per
// 16-column group: 4 per tile), then the partial carries.  Every call leaves
// its counters at zero and nothing else writes that region, so a workspace
// zeroed once stays valid for calls of any shape.
constexpr size_t kCounterBytes = (size_t)(kMaxN / Q8_TILE_COLS) * 4 * 4;

// nw: weights whose carries meet in the workspace (2 for the gated pair,
// whose two weights' carries always meet there).
size_t plan_ws_bytes(const q8_plan &p, int64_t m, int64_t N, int nw = 1) {
  if (p.split_k * nw <= 1) return 0;
  const int64_t Npad = round_up(N, Q8_TILE_COLS);
  // the column-group and 32x32 kernels keep whole records of their tile rows
  const int64_t rows =
      (p.kernel == Q8_KERNEL_MFMA_COLS || p.kernel >= Q8_KERNEL_MFMA32) ? p.rows : m;
  return kCounterBytes + (size_t)round_up((int64_t)nw * p.split_k * rows * Npad * 4, 256);
}

// ---- library-owned workspaces, per (device, stream) ---------------------------

struct Workspace {
  void *ptr = nullptr;
  size_t bytes = 0;
};
std::mutex g_ws_mu;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;
std::vector<std::pair<int, void *>> g_ws_retired;  // freed by q8_release_workspaces

int library_workspace(hipStream_t stream, size_t need, void **out) {
  *out = nullptr;
  if (need == 0) return Q8_OK;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lock(g_ws_mu);
  Workspace &w = g_ws[{dev, stream}];
  if (w.bytes < need) {
    // Allocating (and clearing) a workspace is not a graph-capturable step:
    // refuse under capture rather than record a memset node and bake a
    // buffer the library may later retire into the graph.
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cap) == hipSuccess && cap != hipStreamCaptureStatusNone)
      return fail(Q8_ERR_WORKSPACE,
                  "this call needs a %zu-byte split-K workspace and the stream is being "
                  "captured: the library does not allocate under capture; pass a workspace "
                  "(q8_gemv_ws / the _planned calls) or make one uncaptured call first",
                  need);
    // Work already queued on the stream may still use the old buffer: retire
    // it rather than free it.
    if (w.ptr) g_ws_retired.push_back({dev, w.ptr});
    w.ptr = nullptr;
    w.bytes = 0;
    const size_t bytes = (size_t)round_up((int64_t)need, 1 << 20);
    void *p = nullptr;
    e = hipMalloc(&p, bytes);
    if (e != hipSuccess) return hip_fail(e, "hipMalloc(workspace)");
    // Zero once: the arrival counters start at zero and every call leaves
    // them at zero.
    e = hipMemsetAsync(p, 0, bytes, stream);
    if (e != hipSuccess) {
      (void)hipFree(p);
      return hip_fail(e, "hipMemsetAsync(workspace)");
    }
    w.ptr = p;
    w.bytes = bytes;
  }
  *out = w.ptr;
  return Q8_OK;
}

// The epilogue check: pointers present and aligned, something written.
int check_epilogue(const q8_epilogue *ep, const float *y) {
  int st;
  if (!ep) return check_ptr(y, "y");
  if (ep->write_y && (st = check_ptr(y, "y"))) return st;
  if (!ep->write_y && !ep->y_q8)
    return fail(Q8_ERR_NULL, "epilogue writes neither y nor y_q8");
  if (ep->bias && (st = check_ptr(ep->bias, "epilogue bias"))) return st;
  if (ep->residual && (st = check_ptr(ep->residual, "epilogue residual"))) return st;
  if (ep->y_q8 && (st = check_ptr(ep->y_q8, "epilogue y_q8"))) return st;
  return Q8_OK;
}

// The gated pair's second weight and its bias.
struct PairArgs {
  const int8_t *wq_u;
  const float *wsc_u;
  const float *bias_u;
};

int run_gemv(const void *x, const int8_t *W_q8, const float *W_q8_scale,
             float *y, int32_t *dots, int64_t m, int64_t K, int64_t N,
             int act_fmt, const q8_plan &plan, hipStream_t stream,
             void *workspace, size_t ws_bytes, const q8_epilogue *ep = nullptr,
             const PairArgs *pair = nullptr) {
  const bool write_dots = dots != nullptr;
  const int nw = pair ? 2 : 1;
  if (pair && plan.kernel >= Q8_KERNEL_MFMA32)
    return fail(Q8_ERR_PLAN, "the MFMA32 kernels do not run the gated pair: "
                "use the VALU, MFMA or MFMA_COLS kernel");
  if (ep && ep->y_q8 && plan.kernel == Q8_KERNEL_MFMA_COLS && plan.split_k * nw < 2)
    return fail(Q8_ERR_PLAN, "the MFMA_COLS kernel quantizes its output in the split-K "
                "finish: y_q8 needs split_k >= 2 (or the MFMA or VALU kernel)");
  int st = check_plan(&plan, m, K, act_fmt, write_dots);
  if (st) return st;
  const int64_t Npad = round_up(N, Q8_TILE_COLS);
  q8::GemvArgs a{};
  a.x = x;
  a.wq = W_q8;
  a.wsc = W_q8_scale;
  a.y = y;
  a.dots = dots;
  a.m = (int)m;
  a.K = (int)K;
  a.NB = (int)(K / Q8_BLOCK);
  a.Npad = (int)Npad;
  a.T = (int)(Npad / Q8_TILE_COLS);
  a.split_k = plan.split_k;
  a.act_scale_off = (unsigned)act_scales_offset_of(act_fmt, m, K);
  if (act_fmt != Q8_ACT_BF16 && act_view_offset(m, K) > 0xffffffffull)
    return fail(Q8_ERR_SHAPE, "activation too large");
  a.act_view_off = act_fmt == Q8_ACT_Q8_0 ? (unsigned)act_view_offset(m, K) : 0u;
  a.ep.N = (int)N;
  a.ep.write_y = 1;
  a.ep.nw = nw;
  if (pair) {
    a.ep.wq_u = pair->wq_u;
    a.ep.wsc_u = pair->wsc_u;
    a.ep.bias_u = pair->bias_u;
  }
  if (ep) {
    a.ep.bias = ep->bias;
    a.ep.residual = ep->residual;
    a.ep.write_y = ep->write_y != 0;
    if (ep->y_q8) {
      a.ep.yq = static_cast<int8_t *>(ep->y_q8);
      a.ep.yq_scale = reinterpret_cast<float *>(static_cast<char *>(ep->y_q8) +
                                                act_scales_offset(m, Npad));
      a.ep.yq_view = static_cast<int8_t *>(ep->y_q8) + act_view_offset(m, Npad);
    }
  }
  if (!write_dots && plan.split_k * nw > 1) {
    const size_t need = plan_ws_bytes(plan, m, N, nw);
    if (!workspace || ws_bytes < need)
      return fail(Q8_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed",
                  workspace ? ws_bytes : (size_t)0, need);
    a.counters = static_cast<unsigned *>(workspace);
    a.partial = reinterpret_cast<float *>(static_cast<char *>(workspace) + kCounterBytes);
  }
  (void)hipGetLastError();  // clear a stale error so the launch's own is seen
  hipError_t e = q8::launch_gemv(plan.kernel, plan.rows, act_fmt, write_dots,
                                 plan.waves, plan.kslices, a, stream);
  if (e != hipSuccess) {
    (void)hipGetLastError();   // do not leave the failure for the caller's next HIP call
    return hip_fail(e, "gemv launch");
  }
  return ok();
}

int check_gemv_args(const void *x, const int8_t *W_q8, const float *W_q8_scale,
                    const void *out, const char *out_name, int64_t m, int64_t K,
                    int64_t N, int act_fmt, bool need_scales, bool need_out = true) {
  int st;
  if ((st = check_m(m))) return st;
  if ((st = check_kn(K, N))) return st;
  if ((st = check_act(act_fmt))) return st;
  if (act_fmt == Q8_ACT_Q8_0_TWO_WORDS && (st = check_m(m, Q8_MAX_TWO_WORD_ROWS))) return st;
  if ((st = check_ptr(x, "x"))) return st;
  if ((st = check_ptr(W_q8, "W_q8"))) return st;
  if (need_scales && (st = check_ptr(W_q8_scale, "W_q8_scale"))) return st;
  if (need_out && (st = check_ptr(out, out_name))) return st;
  return Q8_OK;
}

// q8_gemv's plan, except that an output quantizer needs MFMA_COLS to split K
// (its quantizer runs in the split-K finish); with one block only, MFMA.
q8_plan fused_default_plan(int64_t m, int64_t K, int64_t N, int act_fmt,
                           const q8_epilogue *ep) {
  q8_plan p = default_plan(m, K, N, act_fmt);
  if (ep && ep->y_q8 && p.kernel == Q8_KERNEL_MFMA_COLS && p.split_k < 2 &&
      K / Q8_BLOCK >= 2) {
    p.split_k = 2;
  } else if (ep && ep->y_q8 && p.kernel == Q8_KERNEL_MFMA_COLS && p.split_k < 2) {
    p.kernel = Q8_KERNEL_MFMA;
    p.waves = 16;
    p.kslices = 1;
    const int64_t NB = K / Q8_BLOCK;
    const size_t budget = (size_t)device_facts().lds_per_block - kStaticLdsReserve;
    int64_t S = 1;
    while (S < NB && q8::gemv_lds_bytes(p.kernel, p.rows, act_fmt, p.waves, p.kslices, (int)NB,
                                        (int)S) > budget)
      ++S;
    p.split_k = (int32_t)S;
  }
  return p;
}

// The gated pair's plan: q8_gemv's for the pair's 2*N_pad columns of work
// (the VALU split count counts both weights' tiles); its two weights always
// meet in the workspace, so the column-group kernel's quantizer needs no
// K split.
// With the VALU kernel, the pair's twice as many workgroups take half the
// single product's waves each once they outnumber the CUs, which keeps the
// waves streaming at once (and the bytes each wave streams) those of the
// single product (measured on MI355X, m = 1, K = 4096, N = 14336: 4 waves
// 23.0 us, 8 waves 24.2 us).
q8_plan glu_default_plan(int64_t m, int64_t K, int64_t N, int act_fmt) {
  q8_plan p = default_plan(m, K, 2 * round_up(N, Q8_TILE_COLS), act_fmt, false);
  const int64_t units = 2 * round_up(N, Q8_TILE_COLS) / Q8_TILE_COLS;
  if (p.kernel == Q8_KERNEL_VALU && units * p.split_k > device_facts().cus) p.waves /= 2;
  return p;
}

int check_glu_epilogue(const q8_glu_epilogue *ep, const float *y) {
  int st;
  if (!ep) return check_ptr(y, "y");
  if (ep->write_y && (st = check_ptr(y, "y"))) return st;
  if (!ep->write_y && !ep->y_q8)
    return fail(Q8_ERR_NULL, "epilogue writes neither y nor y_q8");
  if (ep->bias_g && (st = check_ptr(ep->bias_g, "epilogue bias_g"))) return st;
  if (ep->bias_u && (st = check_ptr(ep->bias_u, "epilogue bias_u"))) return st;
  if (ep->y_q8 && (st = check_ptr(ep->y_q8, "epilogue y_q8"))) return st;
  return Q8_OK;
}

int run_glu(const void *x, const int8_t *Wg, const float *Wg_s, const int8_t *Wu,
            const float *Wu_s, float *y, int64_t m, int64_t K, int64_t N, int act_fmt,
            const q8_glu_epilogue *gep, const q8_plan &plan, hipStream_t stream,
            void *workspace, size_t ws_bytes) {
  q8_epilogue ep{};
  ep.write_y = 1;
  if (gep) {
    ep.bias = gep->bias_g;
    ep.y_q8 = gep->y_q8;
    ep.write_y = gep->write_y;
  }
  const PairArgs pair{Wu, Wu_s, gep ? gep->bias_u : nullptr};
  return run_gemv(x, Wg, Wg_s, y, nullptr, m, K, N, act_fmt, plan, stream, workspace, ws_bytes,
                  &ep, &pair);
}

int check_glu_args(const void *x, const int8_t *Wg, const float *Wg_s, const int8_t *Wu,
                   const float *Wu_s, const float *y, int64_t m, int64_t K, int64_t N,
                   int act_fmt, const q8_glu_epilogue *ep) {
  int st = check_gemv_args(x, Wg, Wg_s, y, "y", m, K, N, act_fmt, true, false);
  if (st) return st;
  if ((st = check_ptr(Wu, "Wu_q8")) || (st = check_ptr(Wu_s, "Wu_q8_scale"))) return st;
  return check_glu_epilogue(ep, y);
}

// ---- projections in parts -------------------------------------------------------

static_assert(Q8_MAX_PARTS == q8::kMaxParts, "parts limit of the ABI and the kernels");

// Checks the parts and returns their padded widths summed: the launch's
// output columns side by side.
int check_parts(const q8_part *parts, int n_parts, int64_t *cols_out) {
  if (!parts) return fail(Q8_ERR_NULL, "parts is NULL");
  if (n_parts < 1 || n_parts > Q8_MAX_PARTS)
    return fail(Q8_ERR_SHAPE, "n_parts = %d out of range: need 1 <= n_parts <= %d", n_parts,
                Q8_MAX_PARTS);
  int64_t cols = 0;
  for (int i = 0; i < n_parts; ++i) {
    const int64_t N = parts[i].N;
    if (N < 1 || N > kMaxN)
      return fail(Q8_ERR_SHAPE, "part %d: N = %lld out of range: need 1 <= N <= %lld", i,
                  (long long)N, (long long)kMaxN);
    cols += round_up(N, Q8_TILE_COLS);
  }
  if (cols > kMaxN)
    return fail(Q8_ERR_SHAPE, "the parts' padded widths sum to %lld, more than %lld",
                (long long)cols, (long long)kMaxN);
  *cols_out = cols;
  return Q8_OK;
}

int check_parts_args(const void *x, const q8_part *parts, int n_parts, int64_t m, int64_t K,
                     int act_fmt, int64_t *cols) {
  int st;
  if ((st = check_parts(parts, n_parts, cols))) return st;
  if ((st = check_m(m)) || (st = check_kn(K, *cols)) || (st = check_act_rows(act_fmt, m)))
    return st;
  if ((st = check_ptr(x, "x"))) return st;
  for (int i = 0; i < n_parts; ++i) {
    const q8_part &pt = parts[i];
    if ((st = check_ptr(pt.W_q8, "W_q8")) || (st = check_ptr(pt.W_q8_scale, "W_q8_scale")) ||
        (st = check_ptr(pt.y, "y")) || (pt.bias && (st = check_ptr(pt.bias, "bias")))) {
      const std::string what = g_last_error;
      return fail(st, "part %d: %s", i, what.c_str());
    }
  }
  return Q8_OK;
}

// The product's plan over the parts' columns side by side, on a kernel that
// walks units of any part (VALU or block-interleaved MFMA); the VALU kernel
// takes half its waves once the workgroups outnumber the CUs, as the gated
// pair does.  The MFMA kernel splits K further while the splits still
// fit one workgroup per CU: the parts of one attention block are narrower
// than the products the single-product plan was settled on; each split
// keeps at least 32 blocks (measured on
// MI355X, m = 16, K = 4096, N = 4096 + 1024 + 1024: one split 14.7 us, two
// 12.1 us, three 16.0 us).
//
// From 3 rows of bf16 or one-word Q8_0 activations the parts take the
// 16x16x32 tile kernel (its workgroups walk the parts' tiles), with the
// single product's rows and K split; below 128 tiles 16 waves and one-block
// stages.  Measured on MI355X, K = 4096, N = 4096 + 1024 + 1024 (2 splits,
// loop us, against the block-interleaved MFMA kernel): bf16 m = 3, 8, 16:
// 9.9, 10.1, 10.8 against 11.5, 11.6, 11.8 (8 waves 10.1-11.4; two-block
// stages 10.2-10.9); m = 24: 13.2 against 14.1; Q8_0 m = 16: 10.8 against
// 12.5; m = 32: 14.1 against 15.6 (8 waves 14.5; 3 splits 16.3).
q8_plan parts_default_plan(int64_t m, int64_t K, int64_t cols, int act_fmt) {
  const int64_t NB = K / Q8_BLOCK;
  const int64_t units = cols / Q8_TILE_COLS;
  if (act_fmt != Q8_ACT_Q8_0_TWO_WORDS && m > 2) {
    q8_plan t = tile16_plan(m, K, cols, act_fmt);
    if (units < 128) {
      t.waves = 16;
      t.kslices = 1;
      fit_tile_lds(t, NB, act_fmt);
    }
    return t;
  }
  q8_plan p = default_plan(m, K, cols, act_fmt, false);
  const DeviceFacts dev = device_facts();
  if (p.kernel == Q8_KERNEL_MFMA_COLS) {
    p.kernel = Q8_KERNEL_MFMA;
    p.waves = 16;
    p.kslices = 1;
    const size_t budget = (size_t)dev.lds_per_block - kStaticLdsReserve;
    int64_t S = 1;
    while (S < NB && q8::gemv_lds_bytes(p.kernel, p.rows, act_fmt, p.waves, p.kslices, (int)NB,
                                        (int)S) > budget)
      ++S;
    p.split_k = (int32_t)S;
  }
  if (p.kernel == Q8_KERNEL_MFMA) {
    int64_t S = p.split_k;
    while (S < NB / 32 && units * (S + 1) <= dev.cus) ++S;
    p.split_k = (int32_t)S;
  }
  if (p.kernel == Q8_KERNEL_VALU && units * p.split_k > dev.cus) p.waves /= 2;
  return p;
}

int run_parts(const void *x, const q8_part *parts, int n_parts, int64_t m, int64_t K,
              int64_t cols, int act_fmt, const q8_plan &plan, hipStream_t stream,
              void *workspace, size_t ws_bytes) {
  if (plan.kernel == Q8_KERNEL_MFMA_COLS ||
      (plan.kernel >= Q8_KERNEL_MFMA32 && plan.kernel != Q8_KERNEL_MFMA16_TILE))
    return fail(Q8_ERR_PLAN, "the MFMA_COLS and MFMA32 kernels do not run parts: "
                "use the VALU, MFMA or MFMA16_TILE kernel");
  int st = check_plan(&plan, m, K, act_fmt, false);
  if (st) return st;
  if (act_fmt != Q8_ACT_BF16 && (act_scales_offset_of(act_fmt, m, K) > 0xffffffffull ||
                                 act_view_offset(m, K) > 0xffffffffull))
    return fail(Q8_ERR_SHAPE, "activation too large");
  q8::GemvArgs a{};
  a.x = x;
  a.wq = parts[0].W_q8;
  a.wsc = parts[0].W_q8_scale;
  a.y = parts[0].y;
  a.m = (int)m;
  a.K = (int)K;
  a.NB = (int)(K / Q8_BLOCK);
  a.Npad = (int)cols;
  a.T = (int)(cols / Q8_TILE_COLS);
  a.split_k = plan.split_k;
  a.act_scale_off = (unsigned)act_scales_offset_of(act_fmt, m, K);
  a.act_view_off = act_fmt == Q8_ACT_Q8_0 ? (unsigned)act_view_offset(m, K) : 0u;
  a.ep.N = (int)parts[0].N;
  a.ep.write_y = 1;
  a.ep.nw = 1;
  q8::Parts &pp = a.ep.parts;
  pp.n = n_parts;
  pp.cum[0] = 0;
  for (int i = 0; i < q8::kMaxParts; ++i) {
    const bool on = i < n_parts;
    pp.wq[i] = on ? parts[i].W_q8 : nullptr;
    pp.wsc[i] = on ? parts[i].W_q8_scale : nullptr;
    pp.y[i] = on ? parts[i].y : nullptr;
    pp.bias[i] = on ? parts[i].bias : nullptr;
    pp.N[i] = on ? (int)parts[i].N : 0;
    pp.cum[i + 1] =
        pp.cum[i] + (on ? (int)(round_up(parts[i].N, Q8_TILE_COLS) / Q8_TILE_COLS) : 0);
  }
  if (plan.split_k > 1) {
    const size_t need = plan_ws_bytes(plan, m, cols);
    if (!workspace || ws_bytes < need)
      return fail(Q8_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed",
                  workspace ? ws_bytes : (size_t)0, need);
    a.counters = static_cast<unsigned *>(workspace);
    a.partial = reinterpret_cast<float *>(static_cast<char *>(workspace) + kCounterBytes);
  }
  (void)hipGetLastError();
  hipError_t e = q8::launch_gemv(plan.kernel, plan.rows, act_fmt, false, plan.waves,
                                 plan.kslices, a, stream);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return hip_fail(e, "gemv parts launch");
  }
  return ok();
}

}  // namespace

extern "C" {

int64_t q8_padded_cols(int64_t N) {
  if (N < 1) return -1;
  return round_up(N, Q8_TILE_COLS);
}

size_t q8_packed_values_bytes(int64_t K, int64_t N) {
  if (K <= 0 || K % Q8_BLOCK || N < 1) return 0;
  return (size_t)K * (size_t)round_up(N, Q8_TILE_COLS);
}

size_t q8_packed_scales_bytes(int64_t K, int64_t N) {
  if (K <= 0 || K % Q8_BLOCK || N < 1) return 0;
  return (size_t)(K / Q8_BLOCK) * (size_t)round_up(N, Q8_TILE_COLS) * 4;
}

size_t q8_act_scales_offset(int64_t m, int64_t K) {
  if (m < 1 || K <= 0 || K % Q8_BLOCK) return 0;
  return act_scales_offset(m, K);
}

size_t q8_act_view_offset(int64_t m, int64_t K) {
  if (m < 1 || K <= 0 || K % Q8_BLOCK) return 0;
  return act_view_offset(m, K);
}

size_t q8_act_bytes(int64_t m, int64_t K) {
  if (m < 1 || K <= 0 || K % Q8_BLOCK) return 0;
  return act_view_offset(m, K) + (size_t)(m * K);
}

size_t q8_gemv_workspace_bytes(int64_t m, int64_t K, int64_t N, int act_fmt) {
  if (check_act(act_fmt) || check_m_act(m, act_fmt) || check_kn(K, N)) return 0;
  return plan_ws_bytes(default_plan(m, K, N, act_fmt), m, N);
}

int q8_repack(const int8_t *q_kn, const float *s_kn, int64_t K, int64_t N,
              int8_t *W_q8, float *W_q8_scale, hipStream_t stream) {
  int st;
  if ((st = check_kn(K, N))) return st;
  if ((st = check_ptr(q_kn, "q_kn")) || (st = check_ptr(s_kn, "s_kn")) ||
      (st = check_ptr(W_q8, "W_q8")) || (st = check_ptr(W_q8_scale, "W_q8_scale")))
    return st;
  (void)hipGetLastError();
  hipError_t e = q8::launch_repack(q_kn, s_kn, (int)K, (int)N, W_q8, W_q8_scale, stream);
  if (e != hipSuccess) return hip_fail(e, "repack launch");
  return ok();
}

int q8_unpack(const int8_t *W_q8, const float *W_q8_scale, int64_t K, int64_t N,
              int8_t *q_kn, float *s_kn, hipStream_t stream) {
  int st;
  if ((st = check_kn(K, N))) return st;
  if ((st = check_ptr(W_q8, "W_q8")) || (st = check_ptr(W_q8_scale, "W_q8_scale")) ||
      (st = check_ptr(q_kn, "q_kn")) || (st = check_ptr(s_kn, "s_kn")))
    return st;
  (void)hipGetLastError();
  hipError_t e = q8::launch_unpack(W_q8, W_q8_scale, (int)K, (int)N, q_kn, s_kn, stream);
  if (e != hipSuccess) return hip_fail(e, "unpack launch");
  return ok();
}

int q8_quantize_act(const uint16_t *x_bf16, void *x_q8, int64_t m, int64_t K,
                    hipStream_t stream) {
  int st;
  if ((st = check_m(m, Q8_MAX_GEMM_ROWS))) return st;
  if ((st = check_kn(K, 1))) return st;
  if (act_view_offset(m, K) > 0xffffffffull)
    return fail(Q8_ERR_SHAPE, "m*K = %lld too large for the quantized layout",
                (long long)(m * K));
  if ((st = check_ptr(x_bf16, "x_bf16")) || (st = check_ptr(x_q8, "x_q8"))) return st;
  (void)hipGetLastError();
  hipError_t e = q8::launch_quantize_act(x_bf16, x_q8, (int)m, (int)K, act_scales_offset(m, K),
                                         act_view_offset(m, K), stream);
  if (e != hipSuccess) return hip_fail(e, "quantize_act launch");
  return ok();
}

size_t q8_act_two_words_scales_offset(int64_t m, int64_t K) {
  if (m < 1 || K <= 0 || K % Q8_BLOCK) return 0;
  return act_scales_offset(2 * m, K);
}

size_t q8_act_two_words_bytes(int64_t m, int64_t K) {
  if (m < 1 || K <= 0 || K % Q8_BLOCK) return 0;
  return act_scales_offset(2 * m, K) + (size_t)(m * (K / Q8_BLOCK)) * 4;
}

int q8_quantize_act_two_words(const uint16_t *x_bf16, void *x_q8x2, int64_t m, int64_t K,
                              hipStream_t stream) {
  int st;
  if ((st = check_m(m, Q8_MAX_GEMM_ROWS))) return st;
  if ((st = check_kn(K, 1))) return st;
  if (act_scales_offset(2 * m, K) > 0xffffffffull)
    return fail(Q8_ERR_SHAPE, "m*K = %lld too large for the two-word layout",
                (long long)(m * K));
  if ((st = check_ptr(x_bf16, "x_bf16")) || (st = check_ptr(x_q8x2, "x_q8x2"))) return st;
  (void)hipGetLastError();
  hipError_t e = q8::launch_quantize_act_two_words(x_bf16, x_q8x2, (int)m, (int)K,
                                                   (unsigned)act_scales_offset(2 * m, K), stream);
  if (e != hipSuccess) return hip_fail(e, "quantize_act_two_words launch");
  return ok();
}

int q8_gemv_default_plan(int64_t m, int64_t K, int64_t N, int act_fmt, q8_plan *plan) {
  int st;
  if ((st = check_act(act_fmt)) || (st = check_m_act(m, act_fmt)) || (st = check_kn(K, N)))
    return st;
  if (!plan) return fail(Q8_ERR_NULL, "plan is NULL");
  *plan = default_plan(m, K, N, act_fmt);
  return ok();
}

size_t q8_plan_workspace_bytes(const q8_plan *plan, int64_t m, int64_t K, int64_t N) {
  if (!plan || check_m(m) || check_kn(K, N)) return 0;
  return plan_ws_bytes(*plan, m, N);
}

int q8_gemv_planned(const void *x, const int8_t *W_q8, const float *W_q8_scale,
                    float *y, int64_t m, int64_t K, int64_t N, int act_fmt,
                    const q8_plan *plan, hipStream_t stream, void *workspace,
                    size_t ws_bytes) {
  int st = check_gemv_args(x, W_q8, W_q8_scale, y, "y", m, K, N, act_fmt, true);
  if (st) return st;
  if (!plan) return fail(Q8_ERR_NULL, "plan is NULL");
  if (workspace && (st = check_ptr(workspace, "workspace"))) return st;
  return run_gemv(x, W_q8, W_q8_scale, y, nullptr, m, K, N, act_fmt, *plan,
                  stream, workspace, ws_bytes);
}

int q8_gemv_ws(const void *x, const int8_t *W_q8, const float *W_q8_scale,
               float *y, int64_t m, int64_t K, int64_t N, int act_fmt,
               hipStream_t stream, void *workspace, size_t ws_bytes) {
  int st = check_gemv_args(x, W_q8, W_q8_scale, y, "y", m, K, N, act_fmt, true);
  if (st) return st;
  if (workspace && (st = check_ptr(workspace, "workspace"))) return st;
  const q8_plan plan = default_plan(m, K, N, act_fmt);
  return run_gemv(x, W_q8, W_q8_scale, y, nullptr, m, K, N, act_fmt, plan,
                  stream, workspace, ws_bytes);
}

int q8_gemv(const void *x, const int8_t *W_q8, const float *W_q8_scale,
            float *y, int64_t m, int64_t K, int64_t N, int act_fmt,
            hipStream_t stream) {
  int st = check_gemv_args(x, W_q8, W_q8_scale, y, "y", m, K, N, act_fmt, true);
  if (st) return st;
  const q8_plan plan = default_plan(m, K, N, act_fmt);
  const size_t need = plan_ws_bytes(plan, m, N);
  void *ws = nullptr;
  if ((st = library_workspace(stream, need, &ws))) return st;
  return run_gemv(x, W_q8, W_q8_scale, y, nullptr, m, K, N, act_fmt, plan,
                  stream, ws, need);
}

int q8_gemv_fused_default_plan(int64_t m, int64_t K, int64_t N, int act_fmt,
                               const q8_epilogue *epilogue, q8_plan *plan) {
  int st;
  if ((st = check_act(act_fmt)) || (st = check_m_act(m, act_fmt)) || (st = check_kn(K, N)))
    return st;
  if (!plan) return fail(Q8_ERR_NULL, "plan is NULL");
  *plan = fused_default_plan(m, K, N, act_fmt, epilogue);
  return ok();
}

int q8_gemv_planned_fused(const void *x, const int8_t *W_q8, const float *W_q8_scale,
                          float *y, int64_t m, int64_t K, int64_t N, int act_fmt,
                          const q8_epilogue *epilogue, const q8_plan *plan,
                          hipStream_t stream, void *workspace, size_t ws_bytes) {
  int st = check_gemv_args(x, W_q8, W_q8_scale, y, "y", m, K, N, act_fmt, true, false);
  if (st) return st;
  if ((st = check_epilogue(epilogue, y))) return st;
  if (!plan) return fail(Q8_ERR_NULL, "plan is NULL");
  if (workspace && (st = check_ptr(workspace, "workspace"))) return st;
  return run_gemv(x, W_q8, W_q8_scale, y, nullptr, m, K, N, act_fmt, *plan,
                  stream, workspace, ws_bytes, epilogue);
}

int q8_gemv_fused(const void *x, const int8_t *W_q8, const float *W_q8_scale,
                  float *y, int64_t m, int64_t K, int64_t N, int act_fmt,
                  const q8_epilogue *epilogue, hipStream_t stream) {
  int st = check_gemv_args(x, W_q8, W_q8_scale, y, "y", m, K, N, act_fmt, true, false);
  if (st) return st;
  if ((st = check_epilogue(epilogue, y))) return st;
  const q8_plan plan = fused_default_plan(m, K, N, act_fmt, epilogue);
  const size_t need = plan_ws_bytes(plan, m, N);
  void *ws = nullptr;
  if ((st = library_workspace(stream, need, &ws))) return st;
  return run_gemv(x, W_q8, W_q8_scale, y, nullptr, m, K, N, act_fmt, plan,
                  stream, ws, need, epilogue);
}

int q8_gemv_block_dots_planned(const void *x_q8, const int8_t *W_q8,
                               int32_t *dots, int64_t m, int64_t K, int64_t N,
                               const q8_plan *plan, hipStream_t stream) {
  int st = check_gemv_args(x_q8, W_q8, nullptr, dots, "dots", m, K, N,
                           Q8_ACT_Q8_0, false);
  if (st) return st;
  if (!plan) return fail(Q8_ERR_NULL, "plan is NULL");
  return run_gemv(x_q8, W_q8, nullptr, nullptr, dots, m, K, N, Q8_ACT_Q8_0,
                  *plan, stream, nullptr, 0);
}

int q8_gemv_block_dots(const void *x_q8, const int8_t *W_q8, int32_t *dots,
                       int64_t m, int64_t K, int64_t N, hipStream_t stream) {
  int st = check_gemv_args(x_q8, W_q8, nullptr, dots, "dots", m, K, N,
                           Q8_ACT_Q8_0, false);
  if (st) return st;
  const q8_plan plan = default_plan(m, K, N, Q8_ACT_Q8_0);
  return run_gemv(x_q8, W_q8, nullptr, nullptr, dots, m, K, N, Q8_ACT_Q8_0,
                  plan, stream, nullptr, 0);
}

size_t q8_glu_workspace_bytes(const q8_plan *plan, int64_t m, int64_t K, int64_t N) {
  if (!plan || check_m(m) || check_kn(K, N)) return 0;
  return plan_ws_bytes(*plan, m, N, 2);
}

int q8_gemv_glu_default_plan(int64_t m, int64_t K, int64_t N, int act_fmt, q8_plan *plan) {
  int st;
  if ((st = check_m(m)) || (st = check_kn(K, N)) ||
      (st = check_act_rows(act_fmt, m)))
    return st;
  if (!plan) return fail(Q8_ERR_NULL, "plan is NULL");
  *plan = glu_default_plan(m, K, N, act_fmt);
  return ok();
}

int q8_gemv_glu_planned(const void *x, const int8_t *Wg_q8, const float *Wg_q8_scale,
                        const int8_t *Wu_q8, const float *Wu_q8_scale, float *y, int64_t m,
                        int64_t K, int64_t N, int act_fmt, const q8_glu_epilogue *epilogue,
                        const q8_plan *plan, hipStream_t stream, void *workspace,
                        size_t ws_bytes) {
  int st = check_glu_args(x, Wg_q8, Wg_q8_scale, Wu_q8, Wu_q8_scale, y, m, K, N, act_fmt,
                          epilogue);
  if (st) return st;
  if (!plan) return fail(Q8_ERR_NULL, "plan is NULL");
  if (workspace && (st = check_ptr(workspace, "workspace"))) return st;
  return run_glu(x, Wg_q8, Wg_q8_scale, Wu_q8, Wu_q8_scale, y, m, K, N, act_fmt, epilogue,
                 *plan, stream, workspace, ws_bytes);
}

int q8_gemv_glu(const void *x, const int8_t *Wg_q8, const float *Wg_q8_scale,
                const int8_t *Wu_q8, const float *Wu_q8_scale, float *y, int64_t m, int64_t K,
                int64_t N, int act_fmt, const q8_glu_epilogue *epilogue, hipStream_t stream) {
  int st = check_glu_args(x, Wg_q8, Wg_q8_scale, Wu_q8, Wu_q8_scale, y, m, K, N, act_fmt,
                          epilogue);
  if (st) return st;
  const q8_plan plan = glu_default_plan(m, K, N, act_fmt);
  const size_t need = plan_ws_bytes(plan, m, N, 2);
  void *ws = nullptr;
  if ((st = library_workspace(stream, need, &ws))) return st;
  return run_glu(x, Wg_q8, Wg_q8_scale, Wu_q8, Wu_q8_scale, y, m, K, N, act_fmt, epilogue, plan,
                 stream, ws, need);
}

namespace {

int run_gemm(const void *x, const int8_t *W_q8, const float *W_q8_scale, float *y,
             int32_t *dots, int64_t m, int64_t K, int64_t N, int act_fmt, hipStream_t stream) {
  int st;
  if ((st = check_m(m, Q8_MAX_GEMM_ROWS)) || (st = check_kn(K, N)) || (st = check_act(act_fmt)))
    return st;
  if ((st = check_ptr(x, "x")) || (st = check_ptr(W_q8, "W_q8"))) return st;
  if (!dots && (st = check_ptr(W_q8_scale, "W_q8_scale"))) return st;
  if (dots ? (st = check_ptr(dots, "dots")) : (st = check_ptr(y, "y"))) return st;
  if (act_fmt != Q8_ACT_BF16 && act_scales_offset_of(act_fmt, m, K) > 0xffffffffull)
    return fail(Q8_ERR_SHAPE, "m*K = %lld too large for the quantized layout",
                (long long)(m * K));
  const int64_t Npad = round_up(N, Q8_TILE_COLS);
  const GemmTileRoute route = gemm_tile_route(m, K, N, act_fmt);
  if (route.on) {
    q8::GemvArgs g{};
    g.x = x;
    g.wq = W_q8;
    g.wsc = W_q8_scale;
    g.y = y;
    g.dots = dots;
    g.m = (int)m;
    g.K = (int)K;
    g.NB = (int)(K / Q8_BLOCK);
    g.Npad = (int)Npad;
    g.T = (int)(Npad / Q8_TILE_COLS);
    g.split_k = 1;
    g.act_scale_off = (unsigned)act_scales_offset_of(act_fmt, m, K);
    g.act_view_off = act_fmt == Q8_ACT_Q8_0 ? (unsigned)act_view_offset(m, K) : 0u;
    g.ep.N = (int)N;
    g.ep.write_y = 1;
    g.ep.nw = 1;
    (void)hipGetLastError();
    hipError_t e = q8::launch_gemv_tile16(route.rows, act_fmt, route.waves, route.kslices,
                                          dots != nullptr, g, stream);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return hip_fail(e, "gemm launch");
    }
    return ok();
  }
  q8::GemmArgs a{};
  a.x = x;
  a.wq = W_q8;
  a.wsc = W_q8_scale;
  a.y = y;
  a.dots = dots;
  a.m = (int)m;
  a.K = (int)K;
  a.NB = (int)(K / Q8_BLOCK);
  a.Npad = (int)Npad;
  a.T = (int)(Npad / Q8_TILE_COLS);
  a.act_scale_off = (unsigned)act_scales_offset_of(act_fmt, m, K);
  (void)hipGetLastError();
  hipError_t e = q8::launch_gemm(act_fmt, dots != nullptr, q8::gemm_rows_per_block(m), a, stream);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return hip_fail(e, "gemm launch");
  }
  return ok();
}

// The GEMM in parts: the parts' column tiles side by side in one launch.
int run_gemm_parts(const void *x, const q8_part *parts, int n_parts, int64_t m, int64_t K,
                   int act_fmt, hipStream_t stream) {
  int st;
  int64_t cols = 0;
  if ((st = check_parts(parts, n_parts, &cols))) return st;
  if ((st = check_m(m, Q8_MAX_GEMM_ROWS)) || (st = check_kn(K, cols)) ||
      (st = check_act(act_fmt)))
    return st;
  if ((st = check_ptr(x, "x"))) return st;
  for (int i = 0; i < n_parts; ++i) {
    const q8_part &pt = parts[i];
    if ((st = check_ptr(pt.W_q8, "W_q8")) || (st = check_ptr(pt.W_q8_scale, "W_q8_scale")) ||
        (st = check_ptr(pt.y, "y")) || (pt.bias && (st = check_ptr(pt.bias, "bias")))) {
      const std::string what = g_last_error;
      return fail(st, "part %d: %s", i, what.c_str());
    }
  }
  if (act_fmt != Q8_ACT_BF16 && act_scales_offset_of(act_fmt, m, K) > 0xffffffffull)
    return fail(Q8_ERR_SHAPE, "m*K = %lld too large for the quantized layout",
                (long long)(m * K));
  // One launch over the parts' tiles side by side, on the kernel q8_gemm
  // would take for one product of all their columns.
  q8::Parts pp{};
  pp.n = n_parts;
  pp.cum[0] = 0;
  for (int i = 0; i < q8::kMaxParts; ++i) {
    const bool on = i < n_parts;
    pp.wq[i] = on ? parts[i].W_q8 : nullptr;
    pp.wsc[i] = on ? parts[i].W_q8_scale : nullptr;
    pp.y[i] = on ? parts[i].y : nullptr;
    pp.bias[i] = on ? parts[i].bias : nullptr;
    pp.N[i] = on ? (int)parts[i].N : 0;
    pp.cum[i + 1] =
        pp.cum[i] + (on ? (int)(round_up(parts[i].N, Q8_TILE_COLS) / Q8_TILE_COLS) : 0);
  }
  const GemmTileRoute route = gemm_tile_route(m, K, cols, act_fmt);
  hipError_t e;
  (void)hipGetLastError();
  if (route.on) {
    q8::GemvArgs g{};
    g.x = x;
    g.m = (int)m;
    g.K = (int)K;
    g.NB = (int)(K / Q8_BLOCK);
    g.T = pp.cum[n_parts];
    g.Npad = g.T * Q8_TILE_COLS;
    g.split_k = 1;
    g.act_scale_off = (unsigned)act_scales_offset_of(act_fmt, m, K);
    g.act_view_off = act_fmt == Q8_ACT_Q8_0 ? (unsigned)act_view_offset(m, K) : 0u;
    g.ep.write_y = 1;
    g.ep.nw = 1;
    g.ep.parts = pp;
    e = q8::launch_gemv_tile16(route.rows, act_fmt, route.waves, route.kslices, false, g,
                               stream);
  } else {
    q8::GemmArgs a{};
    a.x = x;
    a.m = (int)m;
    a.K = (int)K;
    a.NB = (int)(K / Q8_BLOCK);
    a.act_scale_off = (unsigned)act_scales_offset_of(act_fmt, m, K);
    a.parts = pp;
    e = q8::launch_gemm(act_fmt, false, q8::gemm_rows_per_block(m), a, stream);
  }
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return hip_fail(e, "gemm launch");
  }
  return ok();
}

}  // namespace

int q8_gemm_parts(const void *x, const q8_part *parts, int n_parts, int64_t m, int64_t K,
                  int act_fmt, hipStream_t stream) {
  return run_gemm_parts(x, parts, n_parts, m, K, act_fmt, stream);
}

int q8_gemm(const void *x, const int8_t *W_q8, const float *W_q8_scale, float *y, int64_t m,
            int64_t K, int64_t N, int act_fmt, hipStream_t stream) {
  return run_gemm(x, W_q8, W_q8_scale, y, nullptr, m, K, N, act_fmt, stream);
}

int q8_gemm_block_dots(const void *x_q8, const int8_t *W_q8, int32_t *dots, int64_t m, int64_t K,
                       int64_t N, hipStream_t stream) {
  return run_gemm(x_q8, W_q8, nullptr, nullptr, dots, m, K, N, Q8_ACT_Q8_0, stream);
}

const char *q8_status_string(int status) {
  switch (status) {
    case Q8_OK: return "Q8_OK";
    case Q8_ERR_SHAPE: return "Q8_ERR_SHAPE";
    case Q8_ERR_ACT_FMT: return "Q8_ERR_ACT_FMT";
    case Q8_ERR_NULL: return "Q8_ERR_NULL";
    case Q8_ERR_ALIGN: return "Q8_ERR_ALIGN";
    case Q8_ERR_WORKSPACE: return "Q8_ERR_WORKSPACE";
    case Q8_ERR_HIP: return "Q8_ERR_HIP";
    case Q8_ERR_PLAN: return "Q8_ERR_PLAN";
    default: return "Q8_ERR_UNKNOWN";
  }
}

const char *q8_last_error(void) { return g_last_error.c_str(); }

int q8_release_workspaces(void) {
  std::lock_guard<std::mutex> lock(g_ws_mu);
  if (g_ws.empty() && g_ws_retired.empty()) return ok();
  hipError_t e = hipDeviceSynchronize();
  if (e != hipSuccess) return hip_fail(e, "hipDeviceSynchronize");
  int cur = 0;
  (void)hipGetDevice(&cur);
  auto release = [&](int dev, void *p) {
    (void)hipSetDevice(dev);
    (void)hipDeviceSynchronize();
    (void)hipFree(p);
  };
  for (auto &kv : g_ws)
    if (kv.second.ptr) release(kv.first.first, kv.second.ptr);
  for (auto &r : g_ws_retired) release(r.first, r.second);
  g_ws.clear();
  g_ws_retired.clear();
  (void)hipSetDevice(cur);
  return ok();
}

int q8_layout_version(void) { return q8::kLayoutVersion; }

int q8_stream_read(const void *src, size_t bytes, int workgroups, int waves, int depth,
                   void *sink, hipStream_t stream) {
  int st;
  if ((st = check_ptr(src, "src")) || (st = check_ptr(sink, "sink"))) return st;
  if (bytes < 16 || bytes % 16 != 0)
    return fail(Q8_ERR_SHAPE, "bytes = %zu: need a positive multiple of 16", bytes);
  if (workgroups < 1 || workgroups > 65536)
    return fail(Q8_ERR_SHAPE, "workgroups = %d out of range: need 1 <= workgroups <= 65536",
                workgroups);
  if (waves < 1 || waves > 16)
    return fail(Q8_ERR_SHAPE, "waves = %d out of range: need 1 <= waves <= 16", waves);
  if (depth != 1 && depth != 2 && depth != 4)
    return fail(Q8_ERR_SHAPE, "depth = %d: need 1, 2 or 4", depth);
  const size_t slice = ((bytes + 1023) / 1024 + workgroups - 1) / workgroups * 1024;
  if (slice > ((size_t)1 << 31))
    return fail(Q8_ERR_SHAPE, "a workgroup's slice of %zu bytes exceeds 2^31: more workgroups",
                slice);
  (void)hipGetLastError();
  hipError_t e = q8::launch_stream_read(src, bytes, workgroups, waves, depth,
                                        static_cast<unsigned *>(sink), stream);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return hip_fail(e, "stream read launch");
  }
  return ok();
}


int q8_gemv_parts_default_plan(const q8_part *parts, int n_parts, int64_t m, int64_t K,
                               int act_fmt, q8_plan *plan) {
  int st;
  int64_t cols = 0;
  if ((st = check_parts(parts, n_parts, &cols))) return st;
  if ((st = check_m(m)) || (st = check_kn(K, cols)) ||
      (st = check_act_rows(act_fmt, m)))
    return st;
  if (!plan) return fail(Q8_ERR_NULL, "plan is NULL");
  *plan = parts_default_plan(m, K, cols, act_fmt);
  return ok();
}

size_t q8_parts_workspace_bytes(const q8_plan *plan, const q8_part *parts, int n_parts,
                                int64_t m, int64_t K) {
  int64_t cols = 0;
  if (!plan || check_parts(parts, n_parts, &cols) || check_m(m) || check_kn(K, cols)) return 0;
  return plan_ws_bytes(*plan, m, cols);
}

int q8_gemv_parts_planned(const void *x, const q8_part *parts, int n_parts, int64_t m,
                          int64_t K, int act_fmt, const q8_plan *plan, hipStream_t stream,
                          void *workspace, size_t ws_bytes) {
  int64_t cols = 0;
  int st = check_parts_args(x, parts, n_parts, m, K, act_fmt, &cols);
  if (st) return st;
  if (!plan) return fail(Q8_ERR_NULL, "plan is NULL");
  if (workspace && (st = check_ptr(workspace, "workspace"))) return st;
  return run_parts(x, parts, n_parts, m, K, cols, act_fmt, *plan, stream, workspace, ws_bytes);
}

int q8_gemv_parts(const void *x, const q8_part *parts, int n_parts, int64_t m, int64_t K,
                  int act_fmt, hipStream_t stream) {
  int64_t cols = 0;
  int st = check_parts_args(x, parts, n_parts, m, K, act_fmt, &cols);
  if (st) return st;
  const q8_plan plan = parts_default_plan(m, K, cols, act_fmt);
  const size_t need = plan_ws_bytes(plan, m, cols);
  void *ws = nullptr;
  if ((st = library_workspace(stream, need, &ws))) return st;
  return run_parts(x, parts, n_parts, m, K, cols, act_fmt, plan, stream, ws, need);
}

}  // extern "C"
