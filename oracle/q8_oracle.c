/*
 * q8_oracle.c -- plain, slow, CPU reference of the Q8_0 weight product.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file: only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no source with the HIP
 * library (no headers, helpers, tables or constants) and reads the weight in
 * the canonical layout the pages define, never the library's packed layout.
 *
 * Sources (docs.logicaffeine.com pages):
 *   [Q8]   logicaffeine_compile/spatial/passes/from_q8.rs
 *          - module doc: Q8_0 keeps each column's rows in blocks of 32, one
 *            fp32 scale d and 32 int8 values q per block, w = q*d; the values
 *            tensor is K x N, the scales tensor K/32 x N; the product is
 *            y[n] = sum_b s[b,n] * sum_i x[32b+i] * q[32b+i,n] carried in fp32;
 *            an int8 times a bf16 activation is exact in fp32.
 *          - fn quantize: the exact Q8_0 encoder of a declared weight.
 *          - fn q8_gemv_applies: 1 <= m <= 32 rows, whole blocks of K.
 *          - fn q8_gemv: a weight declared and never set is all zeros.
 *   [LANE] logicaffeine_compile/codegen_cuda/lane/plan.rs
 *          - const QBLOCK / struct Buffer field `quantized`: an activation's
 *            quantized form is int8 values and one scale per 32 values.
 *          - enum Q8MatKind, variant TwoPassInt8, and struct Buffer field
 *            `quantized`: the two-pass numerics keeps two int8 words a value
 *            and one scale per 32.
 *          - enum Launch, variant GemvGlu: two projections of one activation
 *            through a gate, act(x.wg + bg) * (x.wu + bu), SwiGLU (the SiLU
 *            gate) when no activation is named.
 *
 * Precision: every product below is formed in fp64 (bf16 x int8 x fp32 has
 * 8 + 8 + 24 significant bits <= 53, so each term is exact), integer block
 * dots in int64 (exact).  Sums run in the order the definition writes them:
 * i ascending inside a block, b ascending over blocks.
 *
 * Where the pages leave a step open (the activation quantizer's exact
 * formula, its rounding of ties) the reading taken is stated at the function.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define Q8O_BLOCK 32 /* rows of a Q8_0 block [Q8] const Q8_BLOCK */

/* ------------------------------------------------------------------------ */
/* threads                                                                   */
/* ------------------------------------------------------------------------ */

static int g_threads = 0; /* 0 = OpenMP default */

void q8o_set_threads(int n) { g_threads = n; }

int q8o_threads(void) {
#ifdef _OPENMP
  return g_threads > 0 ? g_threads : omp_get_max_threads();
#else
  return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* scalar helpers                                                            */
/* ------------------------------------------------------------------------ */

/* A bf16 value is the top 16 bits of an IEEE binary32. */
static double bf16_value(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* Round to nearest, ties away from zero (C99 round(), the same rule as the
 * pages' `f64::round`). */
static double round_half_away(double v) { return round(v); }

/* ------------------------------------------------------------------------ */
/* [Q8] fn quantize -- the exact Q8_0 encoder                                 */
/* ------------------------------------------------------------------------ */

/*
 * Encodes the K x N weight w (row-major, k outer) as int8 values q (K x N)
 * and fp32 scales s (K/32 x N).  Per block b and column n: amax = max|w|;
 * an all-zero block keeps q = 0 and s = 0; otherwise d = amax/127 must be an
 * fp32 value, and every w/d must be within 1e-9 of an integer r with
 * |r| <= 127 and r*d == w exactly.
 *
 * Returns 1 when w is exactly Q8_0, 0 when some block is not (the pages'
 * NotQ8_0 rejection), -1 on a bad shape.
 */
int q8o_quantize_exact(const double *w, int64_t K, int64_t N, int8_t *q,
                       float *s) {
  if (K <= 0 || N <= 0 || K % Q8O_BLOCK != 0) return -1;
  const int64_t NB = K / Q8O_BLOCK;
  memset(q, 0, (size_t)(K * N));
  for (int64_t i = 0; i < NB * N; ++i) s[i] = 0.0f;
  for (int64_t b = 0; b < NB; ++b) {
    for (int64_t n = 0; n < N; ++n) {
      double amax = 0.0;
      for (int64_t i = 0; i < Q8O_BLOCK; ++i) {
        double a = fabs(w[(Q8O_BLOCK * b + i) * N + n]);
        if (a > amax) amax = a;
      }
      if (amax == 0.0) continue;
      double d = amax / 127.0;
      if ((double)(float)d != d) return 0;
      for (int64_t i = 0; i < Q8O_BLOCK; ++i) {
        double wv = w[(Q8O_BLOCK * b + i) * N + n];
        double v = wv / d;
        double r = round_half_away(v);
        if (fabs(v - r) > 1e-9 || fabs(r) > 127.0 || r * d != wv) return 0;
        q[(Q8O_BLOCK * b + i) * N + n] = (int8_t)r;
      }
      s[b * N + n] = (float)d;
    }
  }
  return 1;
}

/* w = q * d, elementwise, in fp64 (exact: 8 + 24 bits). */
void q8o_dequant(const int8_t *q, const float *s, int64_t K, int64_t N,
                 double *w) {
  for (int64_t k = 0; k < K; ++k)
    for (int64_t n = 0; n < N; ++n)
      w[k * N + n] = (double)q[k * N + n] * (double)s[(k / Q8O_BLOCK) * N + n];
}

/* ------------------------------------------------------------------------ */
/* [LANE] the activation's quantized form                                     */
/* ------------------------------------------------------------------------ */

/*
 * Quantizes each row of the m x K bf16 activation per 32-value block into
 * int8 values xq (m x K) and one fp32 scale dx per block (m x K/32).
 *
 * The pages give only the form (int8 values and a scale per 32).  Reading
 * taken, borrowed from the weight encoder's rule (amax/127, round half away
 * from zero):
 *   amax = max |x| over the block;
 *   d    = fp32(amax / 127);                 amax == 0 gives d = 0, xq = 0;
 *   xq   = clamp(round_half_away(fp32(x / d)), -127, 127).
 * Each division is done in fp64 and rounded once to fp32; for one division of
 * fp32 operands this equals the correctly rounded fp32 quotient.
 */
void q8o_quantize_act(const uint16_t *x, int64_t m, int64_t K, int8_t *xq,
                      float *dx) {
  const int64_t NB = K / Q8O_BLOCK;
  for (int64_t r = 0; r < m; ++r) {
    for (int64_t b = 0; b < NB; ++b) {
      const uint16_t *xb = x + r * K + b * Q8O_BLOCK;
      double amax = 0.0;
      for (int i = 0; i < Q8O_BLOCK; ++i) {
        double a = fabs(bf16_value(xb[i]));
        if (a > amax) amax = a;
      }
      float d = (float)(amax / 127.0);
      dx[r * NB + b] = d;
      for (int i = 0; i < Q8O_BLOCK; ++i) {
        int v = 0;
        if (d != 0.0f) {
          float quot = (float)(bf16_value(xb[i]) / (double)d);
          double rv = round_half_away((double)quot);
          if (rv > 127.0) rv = 127.0;
          if (rv < -127.0) rv = -127.0;
          v = (int)rv;
        }
        xq[r * K + b * Q8O_BLOCK + i] = (int8_t)v;
      }
    }
  }
}

/*
 * The same quantizer on fp32 input: the quantized form of a product's own
 * output, as the next projection reads it (codegen_cuda/lane/plan.rs, enum
 * Launch, field `quant` of a projection: its epilogue quantizes the output;
 * const QBLOCK).  z is m x K fp32, row-major; the reading is the one above:
 *   amax = max |z| over the block, d = fp32(amax / 127),
 *   zq = clamp(round_half_away(fp32(z / d)), -127, 127); amax == 0: zeros.
 */
void q8o_quantize_rows_f32(const float *z, int64_t m, int64_t K, int8_t *zq,
                           float *dz) {
  const int64_t NB = K / Q8O_BLOCK;
  for (int64_t r = 0; r < m; ++r) {
    for (int64_t b = 0; b < NB; ++b) {
      const float *zb = z + r * K + b * Q8O_BLOCK;
      double amax = 0.0;
      for (int i = 0; i < Q8O_BLOCK; ++i) {
        double a = fabs((double)zb[i]);
        if (a > amax) amax = a;
      }
      float d = (float)(amax / 127.0);
      dz[r * NB + b] = d;
      for (int i = 0; i < Q8O_BLOCK; ++i) {
        int v = 0;
        if (d != 0.0f) {
          float quot = (float)((double)zb[i] / (double)d);
          double rv = round_half_away((double)quot);
          if (rv > 127.0) rv = 127.0;
          if (rv < -127.0) rv = -127.0;
          v = (int)rv;
        }
        zq[r * K + b * Q8O_BLOCK + i] = (int8_t)v;
      }
    }
  }
}

/*
 * The two-word form ([LANE] struct Buffer field `quantized`, enum Q8MatKind,
 * variant TwoPassInt8: under the two-pass numerics the quantized form holds
 * two int8 words per value and still one scale per 32).  The pages do not
 * give the split.  Reading taken: the first word and the scale are the
 * one-word quantizer's above; the second word carries the first word's
 * rounding residual in steps of d/128:
 *   quot = fp32(x / d),  hi = clamp(round_half_away(quot), -127, 127),
 *   lo   = round_half_away(128 * (quot - hi)),      so |lo| <= 64,
 * and the value the words stand for is d * (hi + lo / 128).  amax == 0 gives
 * d = 0 and both words 0.  hi, lo are m x K; dx is m x K/32.
 * Parity against the pages is unpinned here: they define no split, so the
 * pins fix this reading (worked values, invariants, its reduction to the
 * one-word quantizer), not a formula the pages give.
 */
void q8o_quantize_act_two_words(const uint16_t *x, int64_t m, int64_t K, int8_t *hi,
                                int8_t *lo, float *dx) {
  const int64_t NB = K / Q8O_BLOCK;
  for (int64_t r = 0; r < m; ++r) {
    for (int64_t b = 0; b < NB; ++b) {
      const uint16_t *xb = x + r * K + b * Q8O_BLOCK;
      double amax = 0.0;
      for (int i = 0; i < Q8O_BLOCK; ++i) {
        double a = fabs(bf16_value(xb[i]));
        if (a > amax) amax = a;
      }
      float d = (float)(amax / 127.0);
      dx[r * NB + b] = d;
      for (int i = 0; i < Q8O_BLOCK; ++i) {
        int vh = 0, vl = 0;
        if (d != 0.0f) {
          float quot = (float)(bf16_value(xb[i]) / (double)d);
          double rh = round_half_away((double)quot);
          if (rh > 127.0) rh = 127.0;
          if (rh < -127.0) rh = -127.0;
          vh = (int)rh;
          vl = (int)round_half_away(128.0 * ((double)quot - rh));
        }
        hi[r * K + b * Q8O_BLOCK + i] = (int8_t)vh;
        lo[r * K + b * Q8O_BLOCK + i] = (int8_t)vl;
      }
    }
  }
}

/* ------------------------------------------------------------------------ */
/* [Q8] module doc -- the product                                            */
/* ------------------------------------------------------------------------ */

/* Column list: `cols` (ncols entries, each in [0, N)), or all N when NULL. */
static int64_t col_at(const int64_t *cols, int64_t j) { return cols ? cols[j] : j; }

/*
 * bf16 activations.  For each row r and listed column n:
 *   y[r,n]     = sum_b s[b,n] * sum_i x[r,32b+i] * q[32b+i,n]
 *   bound[r,n] = sum_b |s[b,n]| * sum_i |x[r,32b+i] * q[32b+i,n]|
 *              = sum_k |x_k * w_kn|
 * y and bound are m x ncols, row-major.  Returns 0, or -1 on a bad shape.
 */
int q8o_gemv_bf16(const uint16_t *x, const int8_t *q, const float *s,
                  int64_t m, int64_t K, int64_t N, const int64_t *cols,
                  int64_t ncols, double *y, double *bound) {
  if (m <= 0 || K <= 0 || N <= 0 || K % Q8O_BLOCK != 0) return -1;
  if (!cols) ncols = N;
  const int64_t NB = K / Q8O_BLOCK;
  int nt = q8o_threads();
#pragma omp parallel for schedule(static) num_threads(nt)
  for (int64_t j = 0; j < ncols; ++j) {
    const int64_t n = col_at(cols, j);
    for (int64_t r = 0; r < m; ++r) {
      double acc = 0.0, bnd = 0.0;
      for (int64_t b = 0; b < NB; ++b) {
        double blk = 0.0, blk_abs = 0.0;
        for (int64_t i = 0; i < Q8O_BLOCK; ++i) {
          const int64_t k = Q8O_BLOCK * b + i;
          double t = bf16_value(x[r * K + k]) * (double)q[k * N + n];
          blk += t;
          blk_abs += fabs(t);
        }
        double sv = (double)s[b * N + n];
        acc += sv * blk;
        bnd += fabs(sv) * blk_abs;
      }
      y[r * ncols + j] = acc;
      bound[r * ncols + j] = bnd;
    }
  }
  return 0;
}

/*
 * int8 activations: the integer block dots
 *   D[r,b,n] = sum_i xq[r,32b+i] * q[32b+i,n]      (int64, exact)
 * written m x NB x ncols, row-major.  Returns 0, or -1 on a bad shape.
 */
int q8o_block_dots(const int8_t *xq, const int8_t *q, int64_t m, int64_t K,
                   int64_t N, const int64_t *cols, int64_t ncols, int64_t *D) {
  if (m <= 0 || K <= 0 || N <= 0 || K % Q8O_BLOCK != 0) return -1;
  if (!cols) ncols = N;
  const int64_t NB = K / Q8O_BLOCK;
  int nt = q8o_threads();
#pragma omp parallel for schedule(static) num_threads(nt)
  for (int64_t j = 0; j < ncols; ++j) {
    const int64_t n = col_at(cols, j);
    for (int64_t r = 0; r < m; ++r)
      for (int64_t b = 0; b < NB; ++b) {
        int64_t acc = 0;
        for (int64_t i = 0; i < Q8O_BLOCK; ++i) {
          const int64_t k = Q8O_BLOCK * b + i;
          acc += (int64_t)xq[r * K + k] * (int64_t)q[k * N + n];
        }
        D[(r * NB + b) * ncols + j] = acc;
      }
  }
  return 0;
}

/*
 * int8 activations: the product over the activation's quantized form,
 * x_k = dx[r, k/32] * xq[r,k]:
 *   y[r,n]     = sum_b dx[r,b] * s[b,n] * D[r,b,n]
 *   bound[r,n] = sum_b |dx[r,b] * s[b,n]| * sum_i |xq * q|
 * Returns 0, or -1 on a bad shape.
 */
int q8o_gemv_q8(const int8_t *xq, const float *dx, const int8_t *q,
                const float *s, int64_t m, int64_t K, int64_t N,
                const int64_t *cols, int64_t ncols, double *y, double *bound) {
  if (m <= 0 || K <= 0 || N <= 0 || K % Q8O_BLOCK != 0) return -1;
  if (!cols) ncols = N;
  const int64_t NB = K / Q8O_BLOCK;
  int nt = q8o_threads();
#pragma omp parallel for schedule(static) num_threads(nt)
  for (int64_t j = 0; j < ncols; ++j) {
    const int64_t n = col_at(cols, j);
    for (int64_t r = 0; r < m; ++r) {
      double acc = 0.0, bnd = 0.0;
      for (int64_t b = 0; b < NB; ++b) {
        int64_t dot = 0, dot_abs = 0;
        for (int64_t i = 0; i < Q8O_BLOCK; ++i) {
          const int64_t k = Q8O_BLOCK * b + i;
          int64_t t = (int64_t)xq[r * K + k] * (int64_t)q[k * N + n];
          dot += t;
          dot_abs += t < 0 ? -t : t;
        }
        double scale = (double)dx[r * NB + b] * (double)s[b * N + n];
        acc += scale * (double)dot;
        bnd += fabs(scale) * (double)dot_abs;
      }
      y[r * ncols + j] = acc;
      bound[r * ncols + j] = bnd;
    }
  }
  return 0;
}

/*
 * Two-word int8 activations, x_k = dx[r, k/32] * (hi[r,k] + lo[r,k] / 128):
 *   y[r,n]     = sum_b dx[r,b] * s[b,n] * (D_hi[r,b,n] + D_lo[r,b,n] / 128)
 *   bound[r,n] = sum_k |x_k * w_kn|
 * with D_hi, D_lo the int64 block dots of each word (hi + lo/128 is exact in
 * fp64).  Returns 0, or -1 on a bad shape.
 */
int q8o_gemv_q8_two_words(const int8_t *hi, const int8_t *lo, const float *dx,
                          const int8_t *q, const float *s, int64_t m, int64_t K,
                          int64_t N, const int64_t *cols, int64_t ncols, double *y,
                          double *bound) {
  if (m <= 0 || K <= 0 || N <= 0 || K % Q8O_BLOCK != 0) return -1;
  if (!cols) ncols = N;
  const int64_t NB = K / Q8O_BLOCK;
  int nt = q8o_threads();
#pragma omp parallel for schedule(static) num_threads(nt)
  for (int64_t j = 0; j < ncols; ++j) {
    const int64_t n = col_at(cols, j);
    for (int64_t r = 0; r < m; ++r) {
      double acc = 0.0, bnd = 0.0;
      for (int64_t b = 0; b < NB; ++b) {
        int64_t dot_hi = 0, dot_lo = 0;
        double dot_abs = 0.0;
        for (int64_t i = 0; i < Q8O_BLOCK; ++i) {
          const int64_t k = Q8O_BLOCK * b + i;
          const int64_t w = q[k * N + n];
          dot_hi += (int64_t)hi[r * K + k] * w;
          dot_lo += (int64_t)lo[r * K + k] * w;
          dot_abs += fabs(((double)hi[r * K + k] + (double)lo[r * K + k] / 128.0) * (double)w);
        }
        double scale = (double)dx[r * NB + b] * (double)s[b * N + n];
        acc += scale * ((double)dot_hi + (double)dot_lo / 128.0);
        bnd += fabs(scale) * dot_abs;
      }
      y[r * ncols + j] = acc;
      bound[r * ncols + j] = bnd;
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* [Q8] fn q8_view_rows and the byte gate of fn q8_gemv                       */
/* ------------------------------------------------------------------------ */

/* Rows of the K/32 x 32 view of an m-row activation: K/32 for one row; for a
 * batch, each row's K chunks of 1024 a whole 32-row tile apiece (the tail's
 * unused rows included). */
/*
 * [LANE] GemvGlu, SwiGLU form, elementwise over m x n values in fp64:
 *   out = silu(g + bg) * (u + bu),  silu(v) = v / (1 + exp(-v)) = v * sigmoid(v)
 * g, u: the two products (fp64, m x n); bg, bu: fp32 biases of n, or NULL.
 */
void q8o_swiglu(const double *g, const double *u, const float *bg,
                const float *bu, int64_t m, int64_t n, double *out) {
  for (int64_t r = 0; r < m; ++r) {
    for (int64_t j = 0; j < n; ++j) {
      double gv = g[r * n + j] + (bg ? (double)bg[j] : 0.0);
      double uv = u[r * n + j] + (bu ? (double)bu[j] : 0.0);
      double sig = 1.0 / (1.0 + exp(-gv));
      out[r * n + j] = gv * sig * uv;
    }
  }
}

int64_t q8o_view_rows(int64_t m, int64_t K) {
  if (m == 1) return K / Q8O_BLOCK;
  const int64_t chunk = Q8O_BLOCK * Q8O_BLOCK;
  return m * ((K + chunk - 1) / chunk) * Q8O_BLOCK;
}

/* Bytes the fold moves, by the pages' model: the weight as stored (values
 * plus fp32 scales over the padded columns) and the view, read once per
 * group of wb 32-wide column tiles for every 1024-row chunk of K. */
void q8o_fold_bytes(int64_t m, int64_t K, int64_t N, int64_t wb,
                    int64_t x_bytes, int64_t *weight, int64_t *view_reads) {
  const int64_t tw = 32, tile = 32 * 32;
  const int64_t n_t = (N + tw - 1) / tw, padded = n_t * tw;
  *weight = K * padded + 4 * (K / Q8O_BLOCK) * padded;
  *view_reads = (n_t / wb) * ((K + tile - 1) / tile) * m * tile * x_bytes;
}

/* ------------------------------------------------------------------------ */
/* [LANE] enum Launch, variant Gemv: the projection's epilogue               */
/* ------------------------------------------------------------------------ */

/*
 * The fused epilogue of one product, over the listed columns: the pages'
 * projection adds its bias to x.w (field `bias`), and the note on
 * gemv_norm_epilogue folds the residual add into the projection's epilogue.
 * Reading taken: bias first, then the residual, each added to the product in
 * fp64 (exact here up to the one rounding of each sum):
 *   z[r,j]     = y[r,j] + bias[n] + residual[r, n]
 *   zbound[r,j] = bound[r,j] + |bias[n]| + |residual[r, n]|
 * with n = cols[j] (or j when cols is NULL).  y and bound are m x ncols (a
 * product's output from the functions above); bias has one value per column
 * (NULL: none); residual is m rows of res_stride values (NULL: none).
 */
void q8o_epilogue(const double *y, const double *bound, int64_t m, int64_t ncols,
                  const int64_t *cols, const float *bias, const float *residual,
                  int64_t res_stride, double *z, double *zbound) {
  for (int64_t r = 0; r < m; ++r) {
    for (int64_t j = 0; j < ncols; ++j) {
      const int64_t n = col_at(cols, j);
      double v = y[r * ncols + j];
      double b = bound[r * ncols + j];
      if (bias) {
        v += (double)bias[n];
        b += fabs((double)bias[n]);
      }
      if (residual) {
        v += (double)residual[r * res_stride + n];
        b += fabs((double)residual[r * res_stride + n]);
      }
      z[r * ncols + j] = v;
      zbound[r * ncols + j] = b;
    }
  }
}
