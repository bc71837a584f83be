/*
 * q8gemv.h -- C ABI of the MI355X (gfx950) Q8_0 weight product.
 *
 * The operation (docs.logicaffeine.com, logicaffeine_compile/spatial/passes/
 * from_q8.rs, module doc): a Q8_0 weight keeps each column's rows in blocks
 * of 32 with one fp32 scale d and 32 int8 values q per block, w = q*d; it is
 * two tensors, the values (K x N int8) and the scales (K/32 x N fp32).  For an
 * m-row activation x (1 <= m <= 32, fn q8_gemv_applies)
 *
 *     y[r,n] = sum_b s[b,n] * sum_i x[r,32b+i] * q[32b+i,n]
 *
 * carried in fp32, the weight streamed once for all m rows.  The activation
 * is bf16, or its quantized form (int8 values and one fp32 scale per 32
 * values: codegen_cuda/lane/plan.rs, const QBLOCK and struct Buffer).
 *
 * Conventions for every call below:
 *   - Pointers are DEVICE pointers (memory of the current HIP device) unless
 *     stated otherwise.  The caller allocates and owns every buffer; the
 *     library keeps no pointer past the call's stream work.
 *   - Work is enqueued on `stream` (0 = the null stream) and is asynchronous:
 *     a return of Q8_OK means "validated and launched"; device faults surface
 *     at the caller's synchronize.
 *   - Every precondition is checked on the host before any launch.  Failures
 *     return a q8_status; q8_last_error() then gives a thread-local message
 *     naming the argument, its value and the bound.  No exception crosses the
 *     ABI.
 *   - Inputs are read-only.  Outputs must not overlap inputs.
 *   - Device pointers must be 16-byte aligned (Q8_ERR_ALIGN otherwise).
 *
 * Layouts:
 *   canonical values  q_kn : K x N int8, row-major (row k, stride N)
 *   canonical scales  s_kn : K/32 x N fp32, row-major
 *   packed values     W_q8 : library-private layout written by q8_repack,
 *                            q8_packed_values_bytes(K, N) bytes
 *   packed scales     W_q8_scale : q8_packed_scales_bytes(K, N) bytes
 *   bf16 activation   x    : m x K bf16 (uint16 bit patterns), row-major
 *   quantized act.    x_q8 : one buffer of q8_act_bytes(m, K) bytes: int8
 *                            values m x K row-major at offset 0, fp32 scales
 *                            m x K/32 row-major at q8_act_scales_offset(m, K),
 *                            and the same int8 values again in the pages'
 *                            block-interleaved view of the rows (from_q8.rs,
 *                            fn relayout_rows_to_q8_view: each 32-value block
 *                            of every row side by side) at
 *                            q8_act_view_offset(m, K): value (r, k) at byte
 *                            ((k/32) * m + r) * 32 + k % 32
 *   output            y    : m x N_pad fp32 row-major, N_pad = q8_padded_cols(N);
 *                            columns N..N_pad-1 are written and are exactly +0
 *                            (pad values and scales are zero: from_q8.rs,
 *                            fn q8_gemv_applies)
 */
#ifndef Q8GEMV_H
#define Q8GEMV_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Activation formats. */
typedef enum {
  Q8_ACT_BF16 = 0,           /* x is m x K bf16                              */
  Q8_ACT_Q8_0 = 1,           /* x is the q8_quantize_act buffer              */
  Q8_ACT_Q8_0_TWO_WORDS = 2  /* x is the q8_quantize_act_two_words buffer    */
} q8_act_fmt;

/* Status codes (errors are values, as the pages' lowering returns its
 * rejections: from_q8.rs SpatialReject, plan.rs LaneError). */
typedef enum {
  Q8_OK = 0,
  Q8_ERR_SHAPE = 1,     /* m, K or N out of range; K not whole 32-blocks      */
  Q8_ERR_ACT_FMT = 2,   /* unknown act_fmt                                    */
  Q8_ERR_NULL = 3,      /* a required pointer is NULL                         */
  Q8_ERR_ALIGN = 4,     /* a device pointer is not 16-byte aligned            */
  Q8_ERR_WORKSPACE = 5, /* workspace missing or smaller than required         */
  Q8_ERR_HIP = 6,       /* a HIP call failed (message from hipGetErrorString) */
  Q8_ERR_PLAN = 7       /* an explicit plan is not valid for the shape        */
} q8_status;

#define Q8_BLOCK 32     /* K rows per Q8_0 block                              */
#define Q8_MAX_ROWS 32  /* most activation rows per call (fn q8_gemv_applies) */
#define Q8_TILE_COLS 64 /* column tile: N is padded to a multiple of this     */
#define Q8_MAX_TWO_WORD_ROWS 16 /* most rows of a two-word activation product */

/* ---- sizes (host functions, no device work) ---------------------------- */

/* ceil(N/64)*64, or -1 when N < 1. */
int64_t q8_padded_cols(int64_t N);
/* K * N_pad: bytes of the packed values. 0 on a bad shape. */
size_t q8_packed_values_bytes(int64_t K, int64_t N);
/* 4 * (K/32) * N_pad: bytes of the packed scales. 0 on a bad shape. */
size_t q8_packed_scales_bytes(int64_t K, int64_t N);
/* Byte offset of the fp32 scales inside a quantized activation buffer:
 * m*K rounded up to 256. */
size_t q8_act_scales_offset(int64_t m, int64_t K);
/* Byte offset of the block-interleaved view inside a quantized activation
 * buffer: the scales' end rounded up to 256. */
size_t q8_act_view_offset(int64_t m, int64_t K);
/* Total bytes of a quantized activation buffer (values, scales and view).
 * 0 on a bad shape. */
size_t q8_act_bytes(int64_t m, int64_t K);
/* The same two for the two-word form: its 2*m*K bytes of words, then the
 * scales at 2*m*K rounded up to 256 (m rows of K/32 fp32). */
size_t q8_act_two_words_scales_offset(int64_t m, int64_t K);
size_t q8_act_two_words_bytes(int64_t m, int64_t K);
/* Bytes of the split-K workspace q8_gemv_ws needs for this shape (may be 0). */
size_t q8_gemv_workspace_bytes(int64_t m, int64_t K, int64_t N, int act_fmt);

/* ---- weight layout ------------------------------------------------------ */

/*
 * q8_repack: canonical -> packed (from_q8.rs, enum Q8Part: what the host
 * repacks from the checkpoint's blocks into the two stored tensors).
 * Reads q_kn (K x N int8) and s_kn (K/32 x N fp32); writes W_q8 and
 * W_q8_scale in the packed layout over N_pad columns, the pad columns' values
 * and scales zero.  Requires K > 0, K % 32 == 0, N >= 1.
 */
int q8_repack(const int8_t *q_kn, const float *s_kn, int64_t K, int64_t N,
              int8_t *W_q8, float *W_q8_scale, hipStream_t stream);

/*
 * q8_unpack: packed -> canonical, the inverse of q8_repack on the N real
 * columns.  Writes q_kn (K x N) and s_kn (K/32 x N).
 */
int q8_unpack(const int8_t *W_q8, const float *W_q8_scale, int64_t K,
              int64_t N, int8_t *q_kn, float *s_kn, hipStream_t stream);

/* ---- activation --------------------------------------------------------- */

/*
 * q8_quantize_act: bf16 activation -> its quantized form, per row and per
 * 32-value block (plan.rs, const QBLOCK and struct Buffer field `quantized`:
 * int8 values with one scale for each 32 of them).
 * The pages do not give the formula; this library computes
 *     amax = max|x|,  d = fp32(amax / 127)  (amax == 0: d = 0, xq = 0),
 *     xq   = clamp(round_half_away_from_zero(fp32(x / d)), -127, 127)
 * with correctly rounded divisions.  Requires 1 <= m <= Q8_MAX_GEMM_ROWS,
 * K > 0, K % 32 == 0.  x_q8 receives q8_act_bytes(m, K) bytes: the codes
 * row-major, the scales, and the codes' block-interleaved view (the
 * MFMA32_TILE kernel reads one block's rows from it as one run).
 */
int q8_quantize_act(const uint16_t *x_bf16, void *x_q8, int64_t m, int64_t K,
                    hipStream_t stream);

/*
 * q8_quantize_act_two_words: bf16 activation -> its two-word form, the
 * quantized form of the two-pass numerics (plan.rs, enum Q8MatKind, variant
 * TwoPassInt8, and struct Buffer field `quantized`: two int8 words a value,
 * still one scale per 32).  The pages do not give the split; this library
 * takes d and the first word hi as q8_quantize_act does and puts the first
 * word's rounding residual, in steps of d/128, in the second:
 *     quot = fp32(x / d),  hi = clamp(round_half_away(quot), -127, 127),
 *     lo   = round_half_away(128 * (quot - hi))        (|lo| <= 64)
 * so the words stand for d * (hi + lo/128).  Layout: hi as m x K int8 at 0,
 * lo as m x K int8 at m*K (the two are the rows of a 2m-row one-word
 * buffer), the m x K/32 fp32 scales at q8_act_two_words_scales_offset(m, K);
 * q8_act_two_words_bytes(m, K) bytes in all.  Requires 1 <= m <=
 * Q8_MAX_GEMM_ROWS, K > 0, K % 32 == 0.
 */
int q8_quantize_act_two_words(const uint16_t *x_bf16, void *x_q8x2, int64_t m,
                              int64_t K, hipStream_t stream);

/* ---- the product ---------------------------------------------------------- */

/*
 * q8_gemv: y = x . W over the packed Q8_0 weight (from_q8.rs, module doc and
 * fn q8_fold).  x per act_fmt; y is m x N_pad fp32.  Requires 1 <= m <= 32
 * (two-word activations: m <= Q8_MAX_TWO_WORD_ROWS), K > 0, K % 32 == 0,
 * N >= 1.  Two-word activations run each block's two int8 passes (v_dot4
 * or the matrix cores) and join them exactly in int32 before the block's
 * scale (128 * D_hi + D_lo, then times dx * s / 128); the VALU kernel (up to
 * 4 rows) and the block-interleaved MFMA kernel take them (plans naming
 * another kernel are Q8_ERR_PLAN), also for the gated pair and the parts.
 * When the chosen plan splits K across
 * workgroups it uses a workspace the library allocates on first need and
 * keeps per (device, stream) until q8_release_workspaces(); a call that would
 * allocate while its stream is being captured returns Q8_ERR_WORKSPACE
 * instead (make one uncaptured call first, or pass a workspace through
 * q8_gemv_ws).  Calls on one stream are ordered; calls on different streams
 * use different workspaces.
 */
int q8_gemv(const void *x, const int8_t *W_q8, const float *W_q8_scale,
            float *y, int64_t m, int64_t K, int64_t N, int act_fmt,
            hipStream_t stream);

/*
 * q8_gemv_ws: q8_gemv with the caller's workspace (device memory of at least
 * q8_gemv_workspace_bytes(m, K, N, act_fmt) bytes, 16-byte aligned, or NULL
 * when that size is 0).  Its first 4 MiB hold split-K arrival counters at
 * fixed places (per 16-column group); they must be zero at the first use,
 * and every call leaves them at zero again, so a workspace zeroed once serves
 * calls of any shape.  Calls that share a workspace must be ordered (one
 * stream).  Q8_ERR_WORKSPACE when too small.
 */
int q8_gemv_ws(const void *x, const int8_t *W_q8, const float *W_q8_scale,
               float *y, int64_t m, int64_t K, int64_t N, int act_fmt,
               hipStream_t stream, void *workspace, size_t ws_bytes);

/*
 * q8_gemv_block_dots: test hook of the int8 path.  Runs the same device code
 * as q8_gemv with Q8_ACT_Q8_0 but writes the exact per-block int32 dots
 *     dots[r, b, n] = sum_i xq[r,32b+i] * q[32b+i,n]
 * as an m x K/32 x N_pad int32 array (pad columns 0) instead of scaling them.
 */
int q8_gemv_block_dots(const void *x_q8, const int8_t *W_q8, int32_t *dots,
                       int64_t m, int64_t K, int64_t N, hipStream_t stream);

/* ---- plans: what q8_gemv launches, and an explicit choice for tuning ----- */

typedef enum {
  Q8_KERNEL_VALU = 0,     /* lane per column, activation broadcast from SGPRs     */
  Q8_KERNEL_MFMA = 1,     /* 16x16x32 matrix-core block dots, activation in LDS;
                             waves split K, each over all 64 columns of a tile    */
  Q8_KERNEL_MFMA_COLS = 2, /* as MFMA, but each wave owns one 16-column group     */
  Q8_KERNEL_MFMA32 = 3,    /* 32x32x32 int8 matrix-core block dots, 32 rows of a
                              one-word Q8_0 activation in LDS; each wave covers all
                              64 columns of a tile, kslices waves split a tile's K
                              range, waves / kslices tiles side by side; one weight
                              (no gated pair, no parts)                             */
  Q8_KERNEL_MFMA32_DIRECT = 4, /* as MFMA32, but the activation fragments are loaded
                              from memory with each weight stage and only the
                              activation scales are staged in LDS, so a workgroup's
                              K range is not bounded by the LDS                    */
  Q8_KERNEL_MFMA32_TILE = 5, /* the 32x32x32 block dots with the VALU kernel's weight
                              stream: one workgroup per (kslices tiles, K split),
                              waves (4, 8 or 16; with kslices 2: 4 or 8) split K,
                              the activation fragments loaded with the weights and
                              shared by the kslices (1 or 2) tiles of a wave       */
  Q8_KERNEL_MFMA16_TILE = 6 /* 16x16x32 block dots of 16 or 32 rows (bf16 or
                              one-word Q8_0; rows 32 as two groups of 16) with the
                              VALU kernel's weight stream: one workgroup per (tile,
                              K split), waves (4, 8 or 16) split K, kslices =
                              blocks a wave's stage holds (bf16: 1, or 2 with the
                              activation read as whole lines and moved into place
                              through the LDS, 32 rows with 4 or 8 waves only, and
                              only where the last K split, K/32 / split_k blocks,
                              is even, else Q8_ERR_PLAN; Q8_0: 1); one weight, or
                              the parts                                             */
} q8_kernel;

typedef struct q8_plan {
  int32_t kernel;  /* q8_kernel                                                */
  int32_t rows;    /* row count the kernel is built for: VALU 1,2,4,8,16,32
                      (two-word activations: 1, 2, 4); MFMA 16 or 32 (two-word
                      activations: 32); MFMA32* 32; MFMA16_TILE 16 or 32; >= m  */
  int32_t split_k; /* K splits across workgroups, 1..K/32                      */
  int32_t waves;   /* waves (64 lanes) per workgroup: 4, 8 or 16               */
  int32_t kslices; /* MFMA_COLS: waves that split one 16-column group's K range
                      (1, 2 or 4; waves = 4 * kslices * tiles side by side);
                      MFMA32(_DIRECT): waves that split one tile's K range (waves 4:
                      1, 2, 4; waves 8: 1, 2, 4, 8; waves = kslices * tiles
                      side by side); MFMA16_TILE: blocks per stage (above);
                      MFMA32_TILE: column tiles a wave covers (above); VALU,
                      MFMA: ignored (all their waves split K)                   */
} q8_plan;

/* The plan q8_gemv would launch for this shape on the current device. */
int q8_gemv_default_plan(int64_t m, int64_t K, int64_t N, int act_fmt,
                         q8_plan *plan /* host pointer */);
/* Workspace bytes an explicit plan needs. */
size_t q8_plan_workspace_bytes(const q8_plan *plan, int64_t m, int64_t K,
                               int64_t N);
/* q8_gemv_ws with an explicit plan (Q8_ERR_PLAN when it does not fit). */
int q8_gemv_planned(const void *x, const int8_t *W_q8,
                    const float *W_q8_scale, float *y, int64_t m, int64_t K,
                    int64_t N, int act_fmt, const q8_plan *plan,
                    hipStream_t stream, void *workspace, size_t ws_bytes);
/* q8_gemv_block_dots with an explicit plan. */
int q8_gemv_block_dots_planned(const void *x_q8, const int8_t *W_q8,
                               int32_t *dots, int64_t m, int64_t K, int64_t N,
                               const q8_plan *plan, hipStream_t stream);

/* ---- fused epilogues ------------------------------------------------------- */

/*
 * What a product does with its fp32 carry before it leaves the kernel: the
 * bias and output-quantize options of codegen_cuda/lane/plan.rs, enum Launch,
 * variant Gemv (fields `bias`, `quant`), and the residual add that the same
 * enum folds into a projection's epilogue (its `gemv_norm_epilogue` note).
 * Per output element (r, n), n < N:
 *     z[r, n] = (x . W)[r, n] + bias[n] + residual[r, n]
 * (each term only when its pointer is given, added in that order in fp32);
 * pad columns N <= n < N_pad get z = 0.  Then
 *   - y[r, n] = z[r, n] when write_y (else y is not touched and may be NULL);
 *   - when y_q8 is given, z's quantized form per row and per 32 columns, by
 *     exactly the q8_quantize_act arithmetic applied to fp32 z, in the
 *     activation layout of q8_act_bytes(m, N_pad): int8 m x N_pad at y_q8,
 *     fp32 scales m x N_pad/32 at y_q8 + q8_act_scales_offset(m, N_pad), the
 *     view at y_q8 + q8_act_view_offset(m, N_pad) -- the input of the next
 *     product with act_fmt Q8_ACT_Q8_0 and K = N_pad.
 * All pointers are device pointers, 16-byte aligned.  bias holds N fp32;
 * residual is m x N_pad fp32 like y and may be y itself (each element is read
 * before it is written, by the same thread).  The MFMA_COLS kernel quantizes
 * its output in the split-K finish (a 32-column block spans two of its
 * waves): a plan naming it with y_q8 set and split_k < 2 is Q8_ERR_PLAN (the
 * fused default plan then splits K in two, or with K = 32 takes the MFMA
 * kernel).
 */
typedef struct q8_epilogue {
  const float *bias;     /* N fp32, or NULL                                   */
  const float *residual; /* m x N_pad fp32, or NULL; may equal y             */
  void *y_q8;            /* q8_act_bytes(m, N_pad) bytes, or NULL             */
  int32_t write_y;       /* nonzero: write y                                  */
} q8_epilogue;

/* q8_gemv with an epilogue (NULL epilogue: plain q8_gemv).  Library workspace
 * as q8_gemv.  Q8_ERR_NULL when nothing would be written. */
int q8_gemv_fused(const void *x, const int8_t *W_q8, const float *W_q8_scale,
                  float *y, int64_t m, int64_t K, int64_t N, int act_fmt,
                  const q8_epilogue *epilogue /* host pointer */, hipStream_t stream);

/* q8_gemv_planned with an epilogue. */
int q8_gemv_planned_fused(const void *x, const int8_t *W_q8,
                          const float *W_q8_scale, float *y, int64_t m,
                          int64_t K, int64_t N, int act_fmt,
                          const q8_epilogue *epilogue, const q8_plan *plan,
                          hipStream_t stream, void *workspace, size_t ws_bytes);

/* The plan q8_gemv_fused launches (differs from q8_gemv_default_plan only
 * when the epilogue quantizes the output). */
int q8_gemv_fused_default_plan(int64_t m, int64_t K, int64_t N, int act_fmt,
                               const q8_epilogue *epilogue, q8_plan *plan);

/* ---- the gated pair --------------------------------------------------------- */

/*
 * Two products of one activation through a gate, in one launch: the pages'
 * codegen_cuda/lane/plan.rs, enum Launch, variant GemvGlu, whose output is
 * act(x.Wg + bg) * (x.Wu + bu), SwiGLU when no activation is named.  This
 * library computes the SwiGLU form, per output element (r, n), n < N:
 *     g = (x . Wg)[r, n] + bias_g[n],  u = (x . Wu)[r, n] + bias_u[n]
 *     z = silu(g) * u,  silu(g) = g / (1 + exp(-g))
 * in fp32 (each bias only when given); pad columns get z = 0.  y and y_q8 as
 * in q8_epilogue.  Wg and Wu are packed weights of the same K x N shape (one
 * q8_repack each); x and act_fmt as in q8_gemv.  The two weights' carries
 * always meet through the workspace (q8_glu_workspace_bytes).
 */
typedef struct q8_glu_epilogue {
  const float *bias_g;   /* N fp32, or NULL                                   */
  const float *bias_u;   /* N fp32, or NULL                                   */
  void *y_q8;            /* q8_act_bytes(m, N_pad) bytes, or NULL             */
  int32_t write_y;       /* nonzero: write y                                  */
} q8_glu_epilogue;

/* The pair with the library's workspace (as q8_gemv).  NULL epilogue: y
 * only, no biases. */
int q8_gemv_glu(const void *x, const int8_t *Wg_q8, const float *Wg_q8_scale,
                const int8_t *Wu_q8, const float *Wu_q8_scale, float *y, int64_t m,
                int64_t K, int64_t N, int act_fmt,
                const q8_glu_epilogue *epilogue /* host pointer */, hipStream_t stream);

/* The pair with an explicit plan and the caller's workspace (zeroed once,
 * as in q8_gemv_ws). */
int q8_gemv_glu_planned(const void *x, const int8_t *Wg_q8,
                        const float *Wg_q8_scale, const int8_t *Wu_q8,
                        const float *Wu_q8_scale, float *y, int64_t m, int64_t K,
                        int64_t N, int act_fmt, const q8_glu_epilogue *epilogue,
                        const q8_plan *plan, hipStream_t stream, void *workspace,
                        size_t ws_bytes);

/* The plan q8_gemv_glu launches, and the workspace a plan needs for it. */
int q8_gemv_glu_default_plan(int64_t m, int64_t K, int64_t N, int act_fmt,
                             q8_plan *plan);
size_t q8_glu_workspace_bytes(const q8_plan *plan, int64_t m, int64_t K,
                              int64_t N);

/* ---- projections in parts ----------------------------------------------------- */

/* Most parts one launch takes. */
#define Q8_MAX_PARTS 4

/*
 * Several products of one activation in one launch: the pages'
 * codegen_cuda/lane/plan.rs, enum Launch, variant GemmParts, and its part,
 * struct GemmPart (a matrix, an optional bias, a destination and its output
 * width), which run as the GEMV in parts at the GEMV's rows.  Part i computes
 *     y_i[r, n] = (x . W_i)[r, n] + bias_i[n]        n < N_i (pad columns 0)
 * with q8_gemv's arithmetic and layouts: every W_i is a packed K x N_i weight
 * (its own q8_repack) over the same K, y_i is m x q8_padded_cols(N_i) fp32.
 * The parts' column tiles are the launch's units side by side, so the
 * workgroups stream all the weights at once.
 */
typedef struct q8_part {
  const int8_t *W_q8;        /* q8_packed_values_bytes(K, N) bytes            */
  const float *W_q8_scale;   /* q8_packed_scales_bytes(K, N) bytes            */
  const float *bias;         /* N fp32, or NULL                               */
  float *y;                  /* m x N_pad fp32, written whole                 */
  int64_t N;                 /* output columns, 1 <= N                        */
} q8_part;

/* 1 <= n_parts <= Q8_MAX_PARTS parts (a host array of them), the padded
 * widths summing to at most 2^24; m, K, x, act_fmt as in q8_gemv.  Uses the
 * library's workspace (as q8_gemv).  Q8_ERR_SHAPE for a bad count or width,
 * Q8_ERR_NULL / Q8_ERR_ALIGN naming the part whose pointer is wrong. */
int q8_gemv_parts(const void *x, const q8_part *parts, int n_parts, int64_t m,
                  int64_t K, int act_fmt, hipStream_t stream);

/* With an explicit plan (the VALU or MFMA kernel; MFMA_COLS is Q8_ERR_PLAN)
 * and the caller's workspace (zeroed once, as in q8_gemv_ws). */
int q8_gemv_parts_planned(const void *x, const q8_part *parts, int n_parts,
                          int64_t m, int64_t K, int act_fmt, const q8_plan *plan,
                          hipStream_t stream, void *workspace, size_t ws_bytes);

/* The plan q8_gemv_parts launches, and the workspace a plan needs for it
 * (0 on invalid arguments). */
int q8_gemv_parts_default_plan(const q8_part *parts, int n_parts, int64_t m,
                               int64_t K, int act_fmt, q8_plan *plan);
size_t q8_parts_workspace_bytes(const q8_plan *plan, const q8_part *parts,
                                int n_parts, int64_t m, int64_t K);

/* ---- many rows: the prefill product ----------------------------------------- */

/* Rows the many-row product accepts. */
#define Q8_MAX_GEMM_ROWS 8192

/*
 * q8_gemm: y = x . W for 1 <= m <= Q8_MAX_GEMM_ROWS activation rows (a prefill
 * chunk), over the same packed weight as q8_gemv, with the same arithmetic
 * (per-block dots scaled once per block, fp32 carry) and the same layouts: x
 * m x K bf16 or the q8_quantize_act buffer of m rows, y m x N_pad fp32 (pad
 * columns 0).  The pages' CUDA planner runs the product as a tensor-core GEMM
 * above its GEMV's rows (codegen_cuda/lane/plan.rs, Launch::on_tensor_cores,
 * gemm_blk_rows); this is its matrix-core form on gfx950.  At few rows of
 * bf16 or one-word Q8_0 activations each 64-column tile of the weight is
 * streamed by one workgroup per chunk of up to 64 rows (the GEMV's 16x16x32
 * tile kernel, 16, 32 or 64 rows a wave): up to 64 rows always, up to 1024
 * while tiles x chunks stay within 512 (bf16) or 1024 (int8), unless K is so
 * long that its int8 activation scales do not fit a workgroup's LDS (with
 * 160 KiB: K above 16256, 36608 or 77312 at 64, 32 or 16 rows a chunk);
 * otherwise, and for two-word activations, a GEMM of 64- or 128-row blocks.
 * No workspace; the call allocates nothing.  Requires K > 0, K % 32 == 0, N >= 1.  Two-word
 * activations (act_fmt 2, the pages' two-pass numerics, whose GEMM plan.rs
 * runs with fewer rows per block): each block's first and second words run
 * as two int8 matrix-core passes joined exactly in int32 before the scale,
 * as in q8_gemv.
 */
int q8_gemm(const void *x, const int8_t *W_q8, const float *W_q8_scale,
            float *y, int64_t m, int64_t K, int64_t N, int act_fmt,
            hipStream_t stream);

/*
 * q8_gemm_block_dots: test hook of q8_gemm's int8 path: the exact per-block
 * int32 dots, m x K/32 x N_pad, as q8_gemv_block_dots writes them.
 */
int q8_gemm_block_dots(const void *x_q8, const int8_t *W_q8, int32_t *dots,
                       int64_t m, int64_t K, int64_t N, hipStream_t stream);

/*
 * q8_gemm_parts: the product in parts above the GEMV's rows, as one launch:
 * the pages' codegen_cuda/lane/plan.rs, enum Launch, variant GemmParts, whose
 * parts run at more rows as one tensor-core GEMM over the parts' tiles side
 * by side (merged_projections).  Part i computes
 *     y_i[r, n] = (x . W_i)[r, n] + bias_i[n]        n < N_i (pad columns 0)
 * with q8_gemm's arithmetic; the parts (a host array, 1 <= n_parts <=
 * Q8_MAX_PARTS, padded widths summing to at most 2^24), x and act_fmt as in
 * q8_gemv_parts, for 1 <= m <= Q8_MAX_GEMM_ROWS.  The launch takes the kernel
 * q8_gemm would take for one product of all the parts' columns, and each
 * part's columns start a new column block of the GEMM (on the tile kernel
 * every tile is its own workgroup), so a part's outputs are bit-identical to
 * q8_gemm on that part alone (before the bias) whenever q8_gemm takes the
 * same kernel for it -- always up to 64 rows, and whenever the parts take
 * the tile kernel -- and within the product's tolerance otherwise.  No
 * workspace; allocates nothing.  Errors as q8_gemv_parts.
 */
int q8_gemm_parts(const void *x, const q8_part *parts, int n_parts, int64_t m,
                  int64_t K, int act_fmt, hipStream_t stream);

/* ---- errors and resources ------------------------------------------------ */

/* Static name of a status code. */
const char *q8_status_string(int status);
/* Thread-local message of this thread's last failing call ("" if none). */
const char *q8_last_error(void);
/* Frees the workspaces q8_gemv allocated (synchronizes the device first).  A
 * graph captured over a library workspace keeps that buffer's address: after
 * this call such a graph must not be replayed. */
int q8_release_workspaces(void);
/* Version of the packed layout: weights packed by another version are
 * rejected by no check -- repack them. */
int q8_layout_version(void);

/* ---- measurement ------------------------------------------------------------ */

/*
 * q8_stream_read: the read ceiling of the product.  A decode step is bound by
 * the weight's bytes (from_q8.rs, module doc), so the rate at which this chip
 * reads a given number of bytes once bounds the product's.  This call reads
 * `bytes` at `src` once with the product's weight-stream loads (16-byte
 * non-temporal loads; `workgroups` contiguous slices of whole KiB, each read
 * by `waves` waves with `depth` KiB in flight per wave) and computes nothing
 * from them; `sink` (4 bytes, 16-byte aligned) is written only for an input
 * no caller supplies.  Requires bytes a positive multiple of 16, 1 <=
 * workgroups <= 65536, 1 <= waves <= 16, depth 1, 2 or 4, and a slice of at
 * most 2^31 bytes (Q8_ERR_SHAPE otherwise).  Allocates nothing.
 */
int q8_stream_read(const void *src, size_t bytes, int workgroups, int waves, int depth,
                   void *sink, hipStream_t stream);

/* ---- the product without allocation ------------------------------------------ */

/* Bytes of the device scratch array q8_gemv_noalloc takes its split-K
 * workspace from (one array per GPU, held until the process ends). */
#define Q8_NOALLOC_SCRATCH_BYTES (16 * 1024 * 1024)

/*
 * q8_gemv_noalloc: for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Computes exactly what q8_gemv computes (same default plan, same kernels,
 * bit-identical y), but its split-K workspace is a fixed device array of
 * Q8_NOALLOC_SCRATCH_BYTES per GPU inside the library instead of an
 * allocation: the call allocates nothing and frees nothing.  Arguments,
 * layouts and errors as q8_gemv; in addition Q8_ERR_WORKSPACE when the shape's
 * plan needs more workspace than the array holds
 * (q8_gemv_workspace_bytes(m, K, N, act_fmt) > Q8_NOALLOC_SCRATCH_BYTES).
 * The first call on each GPU looks up that GPU's copy of the array and clears
 * it with a kernel on `stream`.  Every call on one GPU shares its array and
 * leaves its counters zero for the next: calls that overlap on one GPU
 * (unordered streams or threads) race.
 */
int q8_gemv_noalloc(const void *x, const int8_t *W_q8, const float *W_q8_scale,
                    float *y, int64_t m, int64_t K, int64_t N, int act_fmt,
                    hipStream_t stream);
/* Q8_NOALLOC_SCRATCH_BYTES, as the library was built. */
size_t q8_noalloc_scratch_bytes(void);

#ifdef __cplusplus
}
#endif

#endif /* Q8GEMV_H */
