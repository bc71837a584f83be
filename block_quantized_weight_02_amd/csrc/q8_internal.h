// q8_internal.h -- declarations shared by the host API (q8_api.cpp) and the
// gfx950 kernels (q8_kernels.hip).  Not installed; the public ABI is
// include/q8gemv.h.
//
// Packed weight layout (version 2), private to this library:
//   N is padded to N_pad = 64*T columns; the weight is T column tiles of 64.
//   K is NB = K/32 Q8_0 blocks.  Tile t, block b is one contiguous 2048-byte
//   chunk at byte (t*NB + b)*2048, itself two 1024-byte halves h (k 0..15 and
//   k 16..31 of the block); half h holds, for each of the 64 columns c, the
//   column's 16 values at byte h*1024 + c*16 + (k mod 16).  A tile's chunks are
//   consecutive, so one tile over all K is one contiguous run of K*64 bytes.
//   Scales: one 64-float (256-byte) row per chunk at (t*NB + b)*64; column
//   c = i + 16g (i < 16, g < 4) sits at position 4i + g of the row, so the
//   four columns a 16-column MFMA lane group touches are one 16-byte load.
//   Pad columns carry zero values and zero scales.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace q8 {

constexpr int kBlock = 32;          // K rows of a Q8_0 block
constexpr int kTile = 64;           // columns of a packed tile
constexpr int kChunkBytes = 2048;   // one tile x one block of values
constexpr int kHalfBytes = 1024;    // 16 k-values of each of the 64 columns
constexpr int kLayoutVersion = 2;

// The one-word quantized activation buffer: int8 m x K row-major at 0, fp32
// scales m x K/32 row-major at the scale offset, and the same int8 values in
// the block-interleaved view at the view offset: block b of row r at
// ((b * m + r) * 32), so one block's m rows are m*32 consecutive bytes.
//
// Activation forms: bf16; int8 with one scale per 32 (one word); and two
// int8 words per value with one scale per 32, the second word the first's
// rounding residual in steps of 1/128 of the scale (a buffer laid out as
// 2m one-word rows: the first words, then the second, then m rows of scales).
enum Act { kActBf16 = 0, kActQ8 = 1, kActQ8x2 = 2 };

// Several products of one activation in one launch (the GEMV in parts): part
// p multiplies by its own packed weight (wq[p], wsc[p], N[p] columns) into
// its own output y[p] (m x N_pad(p)), plus its optional bias.  Units (the
// launch's 64-column tiles) cum[p] .. cum[p+1]-1 are part p's tiles.
constexpr int kMaxParts = 4;
struct Parts {
  int n;                          // parts; 0: not a parts launch
  int cum[kMaxParts + 1];
  const int8_t *wq[kMaxParts];
  const float *wsc[kMaxParts];
  float *y[kMaxParts];
  const float *bias[kMaxParts];
  int N[kMaxParts];
};

// Fused epilogue of a product (all pointers optional, device memory).
// nw == 1: z = x.W + bias + residual.
// nw == 2 (gated pair): z = silu(x.W + bias) * (x.W_u + bias_u), W_u the
//   second packed weight (wq_u, wsc_u) of the same shape.
// Then y = z when write_y; yq/yq_scale = the quantized form of z per 32
// columns (int8 m x Npad, fp32 m x Npad/32).  Pad columns of z are exactly 0.
struct Epi {
  const float *bias;
  const float *residual;
  int8_t *yq;
  float *yq_scale;
  int8_t *yq_view;       // the quantized output's block-interleaved view (with yq)
  int N;
  int write_y;
  int nw;                // weights: 1, or 2 for the gated pair
  const int8_t *wq_u;    // the pair's second weight
  const float *wsc_u;
  const float *bias_u;
  Parts parts;           // the GEMV in parts (parts.n > 0): units are its parts' tiles
};

// Everything a product launch needs; pointers are device pointers.
struct GemvArgs {
  const void *x;          // bf16 m x K, or the quantized activation buffer
  const int8_t *wq;       // packed values
  const float *wsc;       // packed scales (unused when writing dots)
  float *y;               // m x Npad
  float *partial;         // split_k x m x Npad (split_k > 1)
  unsigned *counters;     // arrival counters (split_k > 1), zero between calls:
                          // VALU one per tile, MFMA one per 16-column group
  int32_t *dots;          // m x NB x Npad (dot mode)
  int m, K, NB, Npad, T;
  int split_k;
  unsigned act_scale_off; // byte offset of the activation scales (Q8 mode)
  unsigned act_view_off;  // byte offset of the block-interleaved view (one-word Q8)
  Epi ep;                 // epilogue (plain product: N set, write_y 1, nw 1, rest null)
  // Output tiles times weights: the launch's units of work.
  int tiles() const { return T * ep.nw; }
};

// Launchers (q8_kernels.hip).  Return the launch's hipError_t.
hipError_t launch_repack(const int8_t *q_kn, const float *s_kn, int K, int N,
                         int8_t *wq, float *wsc, hipStream_t stream);
hipError_t launch_unpack(const int8_t *wq, const float *wsc, int K, int N,
                         int8_t *q_kn, float *s_kn, hipStream_t stream);
hipError_t launch_quantize_act(const uint16_t *x, void *x_q8, int m, int K,
                               size_t scale_off, size_t view_off, hipStream_t stream);
hipError_t launch_quantize_act_two_words(const uint16_t *x, void *x_q8x2, int m, int K,
                                         unsigned scale_off, hipStream_t stream);
// kernel: 0 VALU, 1 MFMA (waves split K, each over all 64 columns), 2 MFMA
// (waves own 16-column groups), 3 MFMA 32x32x32 int8 (waves split K, each
// over all 64 columns); rows: 1,2,4,8,16,32; act: Act; waves: 4, 8 or 16;
// kslices: waves sharing one column group's K range (kernel 2 only).
// Returns hipErrorInvalidValue for a combination that is not instantiated.
hipError_t launch_gemv(int kernel, int rows, int act, bool write_dots, int waves, int kslices,
                       const GemvArgs &a, hipStream_t stream);
bool gemv_instantiated(int kernel, int rows, int act, bool write_dots, int waves, int kslices);
// Dynamic LDS bytes a launch needs (activation stage plus carries; 0 for VALU).
size_t gemv_lds_bytes(int kernel, int rows, int act, int waves, int kslices, int NB,
                      int split_k);

// The 32x32x32 int8 matrix-core product (q8_mfma32.hip, kernel 3): 32 rows of
// a one-word Q8_0 activation; waves = kslices (waves splitting one tile's K
// range) x tiles side by side; one weight (no pair, no parts).
// kernel 4 is its direct form: the activation fragments loaded from memory
// with each weight stage, only the activation scales staged; kernel 5 the
// tile-per-workgroup form (the VALU kernel's weight stream, operands moved
// into place with lane swaps).
bool mfma32_instantiated(int kernel, int rows, int act, bool write_dots, int waves,
                         int kslices);
size_t mfma32_lds_bytes(int kernel, int waves, int kslices, int NB, int split_k);
hipError_t launch_gemv_mfma32(int kernel, int waves, int kslices, bool write_dots,
                              const GemvArgs &a, hipStream_t stream);

// The tile-per-workgroup 16x16x32 product (q8_tile16.hip, kernel 6): rows 16
// (4, 8 or 16 waves), 32 (4, 8 or 16) or 64 (4 or 8) of bf16 or one-word
// Q8_0 activations; one weight, or the parts (ep.parts, no dots).
bool tile16_instantiated(int rows, int act, bool write_dots, int waves, int kslices);
size_t tile16_lds_bytes(int rows, int act, int waves, int NB, int split_k);
hipError_t launch_gemv_tile16(int rows, int act, int waves, int kslices, bool write_dots,
                              const GemvArgs &a, hipStream_t stream);

// The many-row product (q8_gemm.hip): no split, no workspace.
struct GemmArgs {
  const void *x;
  const int8_t *wq;
  const float *wsc;
  float *y;
  int32_t *dots;           // non-null: write the int32 block dots instead of y
  int m, K, NB, Npad, T;
  unsigned act_scale_off;
  // n > 0: several weights of one activation side by side (the GEMM in
  // parts); cum[] counts 64-column tiles, each part's tiles starting a new
  // column block; wq, wsc, y, Npad, T above are then unused
  Parts parts;
};
// Output rows per workgroup the GEMM takes for m rows (64 or 128).
int gemm_rows_per_block(int64_t m);
hipError_t launch_gemm(int act, bool write_dots, int bm, const GemmArgs &a, hipStream_t stream);

// The read ceiling (q8_measure.hip): reads `bytes` once, `workgroups`
// contiguous slices of whole KiB, `waves` waves each with `depth` (1, 2, 4)
// pieces of 1 KiB in flight.
hipError_t launch_stream_read(const void *src, unsigned long long bytes, int workgroups,
                              int waves, int depth, unsigned *sink, hipStream_t stream);

// Sets the calling thread's q8_last_error() message and returns status.
int report_error(int status, const char *fmt, ...);

}  // namespace q8
