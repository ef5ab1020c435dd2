/*
 * oracle.c -- plain, slow, CPU reference for the NVFP4 "Four-Over-Six"
 * KV-cache smooth-quantize path, its dequantize, and attention over the cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  The GPU library shares no
 * source, header, table or helper with it, and neither links the other.
 *
 * What is computed comes from the summary page "LongLive-2.0: An NVFP4
 * Parallel Infrastructure for Long Video Generation" (paper.rainbus.top,
 * paper 2605.18739), cited below as [LL2]:
 *   - [LL2] inference pipeline, step 7: the cache is built chunk by chunk
 *     (F_c = 8 frames, T_c = F_c * L_f tokens); K of each chunk is smoothed by
 *     removing its mean, then K and V go into an NVFP4 cache with the 4/6
 *     adaptive block scale.
 *   - [LL2] full-stack NVFP4: the 4/6 block scale compares the MSE of two FP8
 *     block-scale candidates, keeping the +-6 range or switching to +-4 so that
 *     values near 75 % of the block maximum are represented more finely.
 *   - [LL2] training pipeline, step 4: NVFP4 GEMMs use 2D block scales for
 *     weights, 1D block scales for activations, and a random Hadamard
 *     transform (RHT) against outliers.
   - [LL2] inference pipeline, steps 7 and 9: the cache feeds attention over
 *     sink frames plus the current window (the attention function below).
 * The page does not define the number formats or the arithmetic.  The
 * readings used here (each marked "convention" where it is used):
 *   E2M1 codes in 16-element blocks, OCP E4M3FN block scales, an FP32 tensor
 *   scale per (chunk, tensor) built from the constant C (1792 = 4 * 448 for
 *   the 4/6 and fixed-4 modes, 2688 = 6 * 448 for fixed-6), round to nearest
 *   even everywhere, fp32 MSE in the tensor-scaled domain with two
 *   sequential fused halves, ties to the +-6 candidate, low nibble = even
 *   element, and the mean over the chunk's tokens per (head, channel).
 *
 * Style: scalar loops, codecs by nearest search over value tables, every
 * fp32 operation written out one at a time.  Build with -O2
 * -ffp-contract=off (no fast-math, no FMA contraction); the only fused
 * multiply-adds are the explicit fmaf() calls of the MSE accumulation.
 * Threads only split independent (head, row-range) work items.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define ORA_API __attribute__((visibility("default")))

enum { ORA_MODE_4OVER6 = 0, ORA_MODE_FIXED6 = 1, ORA_MODE_FIXED4 = 2 };

/* ------------------------------------------------------------------------ */
/* Number formats (convention: OCP FP4 E2M1 and FP8 E4M3FN)                  */
/* ------------------------------------------------------------------------ */

/* E2M1 magnitudes by 3-bit code: 0, 0.5, 1, 1.5, 2, 3, 4, 6 (the +-6 range
 * [LL2] full-stack NVFP4 refers to). */
static const double E2M1_MAG[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

ORA_API float ora_e2m1_decode(uint8_t code) {
  double m = E2M1_MAG[code & 7u];
  return (float)((code & 8u) ? -m : m);
}

/* Nearest E2M1 value to y; a tie goes to the even code; |y| >= 6 gives the
 * largest magnitude (saturation); the sign bit is y's sign bit, so a negative
 * value that rounds to zero gives code 0x8. */
ORA_API uint8_t ora_e2m1_encode(float y) {
  uint8_t sign = signbit(y) ? 8u : 0u;
  double a = fabs((double)y);
  if (a >= 6.0) return (uint8_t)(sign | 7u);
  uint8_t best = 0;
  double bestd = a;
  for (uint8_t k = 1; k < 8; ++k) {
    double d = fabs(a - E2M1_MAG[k]);
    if (d < bestd || (d == bestd && (k % 2u) == 0u)) {
      best = k;
      bestd = d;
    }
  }
  return (uint8_t)(sign | best);
}

/* OCP E4M3FN: bias 7, 3 mantissa bits, subnormals m * 2^-9, no infinity,
 * 0x7F / 0xFF are NaN, largest finite 448. */
ORA_API float ora_e4m3_decode(uint8_t b) {
  int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = (double)m * ldexp(1.0, -9);
  else
    v = (1.0 + (double)m / 8.0) * ldexp(1.0, e - 7);
  return (float)(s ? -v : v);
}

static double e4m3_mag_table[127];
static pthread_once_t e4m3_once = PTHREAD_ONCE_INIT;
static void e4m3_build(void) {
  for (int c = 0; c < 127; ++c) e4m3_mag_table[c] = (double)ora_e4m3_decode((uint8_t)c);
}

/* Nearest finite E4M3FN value to r (codes 0x00..0x7E scanned in increasing
 * order), a tie goes to the even code, magnitudes above 448 give 448. */
ORA_API uint8_t ora_e4m3_encode(float r) {
  pthread_once(&e4m3_once, e4m3_build);
  uint8_t sign = signbit(r) ? 0x80u : 0u;
  double a = fabs((double)r);
  if (a >= 448.0) return (uint8_t)(sign | 0x7Eu);
  int best = 0;
  double bestd = a;
  for (int c = 1; c < 127; ++c) {
    double d = fabs(a - e4m3_mag_table[c]);
    if (d < bestd || (d == bestd && (c % 2) == 0)) {
      best = c;
      bestd = d;
    } else if (e4m3_mag_table[c] > a) {
      break; /* table is increasing: every later value is farther away */
    }
  }
  return (uint8_t)(sign | (uint8_t)best);
}

/* bf16 is the upper half of an fp32 pattern. */
ORA_API float ora_bf16_to_float(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* Value of a bf16 magnitude pattern, reading the all-ones exponent as the
 * finite power 2^128 so that rounding up past the largest finite bf16 lands on
 * infinity exactly as IEEE round-to-nearest does. */
static double bf16_mag_ext(uint16_t h) {
  int e = (h >> 7) & 0xFF, m = h & 0x7F;
  if (e == 0) return (double)m * ldexp(1.0, -133);
  return (1.0 + (double)m / 128.0) * ldexp(1.0, e - 127);
}

/* Nearest bf16 to x, ties to the even pattern (IEEE round to nearest even). */
ORA_API uint16_t ora_float_to_bf16(float x) {
  uint32_t u;
  memcpy(&u, &x, sizeof u);
  if (isnan(x)) return (uint16_t)((u >> 16) | 0x40u);
  if (isinf(x)) return (uint16_t)(u >> 16); /* already a bf16 value */
  uint16_t lo = (uint16_t)(u >> 16); /* same sign, magnitude <= |x| */
  uint16_t hi = (uint16_t)(lo + 1u); /* next magnitude up           */
  double a = fabs((double)x);
  double dlo = a - bf16_mag_ext((uint16_t)(lo & 0x7FFFu));
  double dhi = bf16_mag_ext((uint16_t)(hi & 0x7FFFu)) - a;
  if (dlo < dhi) return lo;
  if (dhi < dlo) return hi;
  return (lo & 1u) ? hi : lo;
}

/* ------------------------------------------------------------------------ */
/* Thread helper: run fn(ctx, item) for item in [0, n) on up to nthreads      */
/* ------------------------------------------------------------------------ */

typedef void (*item_fn)(void* ctx, long item);
typedef struct {
  item_fn fn;
  void* ctx;
  long n;
  long next;
  pthread_mutex_t mu;
} pool_t;

static void* pool_worker(void* arg) {
  pool_t* p = (pool_t*)arg;
  for (;;) {
    pthread_mutex_lock(&p->mu);
    long i = p->next++;
    pthread_mutex_unlock(&p->mu);
    if (i >= p->n) break;
    p->fn(p->ctx, i);
  }
  return NULL;
}

static int resolve_threads(int nthreads) {
  if (nthreads > 0) return nthreads;
  long c = sysconf(_SC_NPROCESSORS_ONLN);
  return c > 0 ? (int)c : 1;
}

static void parallel_items(item_fn fn, void* ctx, long n, int nthreads) {
  int nt = resolve_threads(nthreads);
  if (nt > 256) nt = 256;
  if ((long)nt > n) nt = (int)(n > 0 ? n : 1);
  pool_t p = {fn, ctx, n, 0, PTHREAD_MUTEX_INITIALIZER};
  if (nt <= 1) {
    pool_worker(&p);
    return;
  }
  pthread_t th[256];
  int started = 0;
  for (int t = 0; t < nt; ++t)
    if (pthread_create(&th[t], NULL, pool_worker, &p) == 0) ++started;
  if (started == 0) pool_worker(&p);
  for (int t = 0; t < started; ++t) pthread_join(th[t], NULL);
}

/* ------------------------------------------------------------------------ */
/* Per-chunk K mean ([LL2] inference pipeline, step 7)                      */
/* ------------------------------------------------------------------------ */

/* Convention: the mean is over the chunk's tokens, one value per (head,
 * channel), accumulated in double and rounded to float once at the end. */
typedef struct {
  const uint16_t* x;
  int H, T, D, L;
  float* mean;
} mean_ctx;

static void mean_item(void* vctx, long item) {
  mean_ctx* c = (mean_ctx*)vctx;
  int nchunks = c->T / c->L;
  int h = (int)(item / nchunks), ch = (int)(item % nchunks);
  for (int d = 0; d < c->D; ++d) {
    double s = 0.0;
    for (int t = ch * c->L; t < (ch + 1) * c->L; ++t)
      s += (double)ora_bf16_to_float(c->x[((size_t)h * c->T + t) * c->D + d]);
    c->mean[((size_t)ch * c->H + h) * c->D + d] = (float)(s / (double)c->L);
  }
}

/* mean: [T/L, H, D] */
ORA_API int ora_kv_mean(const uint16_t* x, int H, int T, int D, int L, float* mean, int nthreads) {
  if (!x || !mean || H <= 0 || T <= 0 || D <= 0 || L <= 0 || T % L) return -1;
  mean_ctx c = {x, H, T, D, L, mean};
  parallel_items(mean_item, &c, (long)H * (T / L), nthreads);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Random Hadamard transform of one 16-element block ([LL2] training step 4) */
/* ------------------------------------------------------------------------ */

/* Convention: u_j = s_j * x_j with s_j = -1 where bit j of sign_mask is set;
 * the fast Walsh-Hadamard butterflies with strides 1, 2, 4, 8 turn each pair
 * (u_i, u_{i+h}), i & h == 0, into (u_i + u_{i+h}, u_i - u_{i+h}); the result
 * is multiplied by 1/4 so that the transform (H_16 in natural Sylvester order,
 * times diag(s), over 4) is orthonormal. */
ORA_API void ora_rht16_block(const float* in, uint32_t sign_mask, float* out) {
  float u[16];
  for (int j = 0; j < 16; ++j) u[j] = ((sign_mask >> j) & 1u) ? -in[j] : in[j];
  for (int h = 1; h < 16; h <<= 1) {
    for (int i = 0; i < 16; ++i) {
      if (i & h) continue;
      float a = u[i], b = u[i + h];
      u[i] = a + b;
      u[i + h] = a - b;
    }
  }
  for (int j = 0; j < 16; ++j) out[j] = u[j] * 0.25f;
}

ORA_API void ora_rht16(const float* in, long nblocks, uint32_t sign_mask, float* out) {
  for (long b = 0; b < nblocks; ++b) ora_rht16_block(in + 16 * b, sign_mask, out + 16 * b);
}

/* ------------------------------------------------------------------------ */
/* Four-Over-Six block quantization ([LL2] full-stack NVFP4)                 */
/* ------------------------------------------------------------------------ */

/* Tensor-scale constant C (convention): the encode scale maps the tensor's
 * largest magnitude to C, so a block scale t_b / c never exceeds the E4M3
 * maximum 448 for the candidates the mode uses. */
static float mode_constant(int mode) { return mode == ORA_MODE_FIXED6 ? 2688.0f : 1792.0f; }

/* Encode one row segment of 16 values z (already in the encode domain) under
 * block scale S with reciprocal R: codes q[16] and the fp32 errors of the two
 * 8-element halves.  Convention: y = z * R, E2M1 by nearest; the error is
 * e = z - v * S (v * S is exact: at most 6 significant bits); each half sums
 * e^2 with a sequential fused multiply-add starting from 0. */
static void encode_row16(const float* z, float S, float R, uint8_t* q, float* e_lo, float* e_hi) {
  float lo = 0.0f, hi = 0.0f;
  for (int i = 0; i < 16; ++i) {
    float y = z[i] * R;
    q[i] = ora_e2m1_encode(y);
    float v = ora_e2m1_decode(q[i]);
    float vs = v * S;
    float e = z[i] - vs;
    if (i < 8)
      lo = fmaf(e, e, lo);
    else
      hi = fmaf(e, e, hi);
  }
  *e_lo = lo;
  *e_hi = hi;
}

/* Candidate block scale for divisor c (6 or 4): s = E4M3(t_b / c), with an
 * IEEE fp32 division; R = 1 / S (0 when S is 0). */
static void candidate_scale(float t_b, float c, uint8_t* s, float* S, float* R) {
  float r = t_b / c;
  *s = ora_e4m3_encode(r);
  *S = ora_e4m3_decode(*s);
  *R = (*S > 0.0f) ? 1.0f / *S : 0.0f;
}

/* 1D block: 16 consecutive values x (smoothed / rotated, fp32).  Writes 8 code
 * bytes (low nibble = even element), the scale byte, and the two candidates'
 * errors (NaN for a candidate the mode does not evaluate).  Returns 1 when the
 * +-4 candidate was kept. */
static int quantize_block16(const float* x, float g_enc, int mode, uint8_t* code_bytes, uint8_t* scale,
                            float* err6_out, float* err4_out) {
  float z[16];
  float t_b = 0.0f;
  for (int i = 0; i < 16; ++i) {
    z[i] = x[i] * g_enc;
    float a = fabsf(z[i]);
    if (a > t_b) t_b = a;
  }
  uint8_t s6 = 0, s4 = 0, q6[16], q4[16];
  float err6 = NAN, err4 = NAN;
  if (mode != ORA_MODE_FIXED4) {
    float S, R, lo, hi;
    candidate_scale(t_b, 6.0f, &s6, &S, &R);
    encode_row16(z, S, R, q6, &lo, &hi);
    err6 = lo + hi;
  }
  if (mode != ORA_MODE_FIXED6) {
    float S, R, lo, hi;
    candidate_scale(t_b, 4.0f, &s4, &S, &R);
    encode_row16(z, S, R, q4, &lo, &hi);
    err4 = lo + hi;
  }
  /* Convention: keep +-4 only when its error is strictly lower (ties -> +-6). */
  int use4 = (mode == ORA_MODE_FIXED4) || (mode == ORA_MODE_4OVER6 && err4 < err6);
  const uint8_t* q = use4 ? q4 : q6;
  for (int j = 0; j < 8; ++j) code_bytes[j] = (uint8_t)(q[2 * j] | (q[2 * j + 1] << 4));
  *scale = use4 ? s4 : s6;
  if (err6_out) *err6_out = err6;
  if (err4_out) *err4_out = err4;
  return use4;
}

/* ------------------------------------------------------------------------ */
/* Chunked quantization of [H, T, D] (KV cache) and of [rows, cols] (1D)     */
/* ------------------------------------------------------------------------ */

/* Work item = (head, run of rows) inside one chunk. */
#define ROWS_PER_ITEM 64

typedef struct {
  const uint16_t* x;
  int H, T, D, L, chunk;
  const float* mean; /* [H, D] of this chunk, or NULL */
  int hadamard;
  uint32_t sign_mask;
  float* xp;         /* prepared fp32 chunk [H, L, D] */
  float* item_amax;  /* per item */
  float g_enc;
  int mode;
  uint8_t *codes, *scales;
  float *err6, *err4;
  long* item_use4;
  int items_per_head;
} chunk_ctx;

/* Step 1 of a chunk: smoothing ([LL2] inference step 7; x' = x - m in fp32,
 * never re-rounded to bf16) or the RHT (1D activations), and the largest
 * magnitude of the prepared values. */
static void prepare_item(void* vctx, long item) {
  chunk_ctx* c = (chunk_ctx*)vctx;
  int h = (int)(item / c->items_per_head);
  int r0 = (int)(item % c->items_per_head) * ROWS_PER_ITEM;
  int r1 = r0 + ROWS_PER_ITEM < c->L ? r0 + ROWS_PER_ITEM : c->L;
  float amax = 0.0f;
  for (int r = r0; r < r1; ++r) {
    size_t t = (size_t)c->chunk * c->L + r;
    const uint16_t* src = c->x + ((size_t)h * c->T + t) * c->D;
    float* dst = c->xp + ((size_t)h * c->L + r) * c->D;
    for (int d = 0; d < c->D; ++d) {
      float v = ora_bf16_to_float(src[d]);
      if (c->mean) v = v - c->mean[(size_t)h * c->D + d];
      dst[d] = v;
    }
    if (c->hadamard)
      for (int b = 0; b < c->D / 16; ++b) ora_rht16_block(dst + 16 * b, c->sign_mask, dst + 16 * b);
    for (int d = 0; d < c->D; ++d) {
      float a = fabsf(dst[d]);
      if (a > amax) amax = a;
    }
  }
  c->item_amax[item] = amax;
}

/* Step 2 of a chunk: quantize every 16-element block of the rows. */
static void quant_item(void* vctx, long item) {
  chunk_ctx* c = (chunk_ctx*)vctx;
  int h = (int)(item / c->items_per_head);
  int r0 = (int)(item % c->items_per_head) * ROWS_PER_ITEM;
  int r1 = r0 + ROWS_PER_ITEM < c->L ? r0 + ROWS_PER_ITEM : c->L;
  int nb = c->D / 16;
  long use4 = 0;
  for (int r = r0; r < r1; ++r) {
    size_t t = (size_t)c->chunk * c->L + r;
    size_t row = (size_t)h * c->T + t; /* row index in [H, T] */
    const float* src = c->xp + ((size_t)h * c->L + r) * c->D;
    for (int b = 0; b < nb; ++b) {
      size_t blk = row * nb + b;
      float e6, e4;
      use4 += quantize_block16(src + 16 * b, c->g_enc, c->mode, c->codes + blk * 8, c->scales + blk, &e6, &e4);
      if (c->err6) c->err6[blk] = e6;
      if (c->err4) c->err4[blk] = e4;
    }
  }
  c->item_use4[item] = use4;
}

/*
 * Quantize x [H, T, D] (bf16 bit patterns) chunk by chunk along T.
 *   mean       : NULL (no smoothing) or [T/L, H, D] per-chunk channel means to
 *                subtract first (K; the caller computes them with ora_kv_mean
 *                or passes the GPU's values for a parity run).
 *   hadamard   : apply the 16-point RHT with sign_mask to every block first.
 *   codes      : [H, T, D/2]  scales: [H, T, D/16] (E4M3FN bits)
 *   tensor_scale: [T/L] decode scale g_dec = A / C per chunk.
 *   err6/err4  : NULL or [H*T*D/16] per-block candidate errors.
 *   use4_count : NULL or number of blocks that kept +-4.
 * Convention: the tensor scale spans one chunk of one tensor (all heads);
 * A = largest |x'| in the chunk; g_enc = C / A and g_dec = A / C (both 0 when
 * A = 0), each one IEEE fp32 division.
 */
ORA_API int ora_quantize_chunks(const uint16_t* x, int H, int T, int D, int L, int mode, const float* mean,
                                int hadamard, uint32_t sign_mask, uint8_t* codes, uint8_t* scales,
                                float* tensor_scale, float* err6, float* err4, long long* use4_count,
                                int nthreads) {
  if (!x || !codes || !scales || !tensor_scale) return -1;
  if (H <= 0 || T <= 0 || D <= 0 || L <= 0 || T % L || D % 16) return -2;
  if (mode < 0 || mode > 2) return -6;
  int items_per_head = (L + ROWS_PER_ITEM - 1) / ROWS_PER_ITEM;
  long nitems = (long)H * items_per_head;
  float* xp = (float*)malloc(sizeof(float) * (size_t)H * L * D);
  float* amax = (float*)malloc(sizeof(float) * (size_t)nitems);
  long* u4 = (long*)malloc(sizeof(long) * (size_t)nitems);
  if (!xp || !amax || !u4) {
    free(xp);
    free(amax);
    free(u4);
    return -5;
  }
  float C = mode_constant(mode);
  long long total4 = 0;
  for (int ch = 0; ch < T / L; ++ch) {
    chunk_ctx c;
    memset(&c, 0, sizeof c);
    c.x = x;
    c.H = H;
    c.T = T;
    c.D = D;
    c.L = L;
    c.chunk = ch;
    c.mean = mean ? mean + (size_t)ch * H * D : NULL;
    c.hadamard = hadamard;
    c.sign_mask = sign_mask;
    c.xp = xp;
    c.item_amax = amax;
    c.mode = mode;
    c.codes = codes;
    c.scales = scales;
    c.err6 = err6;
    c.err4 = err4;
    c.item_use4 = u4;
    c.items_per_head = items_per_head;
    parallel_items(prepare_item, &c, nitems, nthreads);
    float A = 0.0f;
    for (long i = 0; i < nitems; ++i)
      if (amax[i] > A) A = amax[i];
    c.g_enc = A > 0.0f ? C / A : 0.0f;
    tensor_scale[ch] = A / C;
    parallel_items(quant_item, &c, nitems, nthreads);
    for (long i = 0; i < nitems; ++i) total4 += u4[i];
  }
  if (use4_count) *use4_count = total4;
  free(xp);
  free(amax);
  free(u4);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* 2D 16x16 tiles (weights, [LL2] training pipeline step 4)                  */
/* ------------------------------------------------------------------------ */

/* Convention: one E4M3 scale and one 4/6 choice per 16x16 tile of w [rows,
 * cols]; t_b is the tile's largest |z|; each tile row's error is computed as
 * in the 1D block (two fused halves added), and the tile error adds the 16
 * row errors as a pairwise tree ((r0+r1)+(r2+r3))+... . */
static float tile_error(const float* z, int ld, float S, float R, uint8_t* q /* [16][16] */) {
  float rows[16];
  for (int r = 0; r < 16; ++r) {
    float lo, hi;
    encode_row16(z + (size_t)r * ld, S, R, q + 16 * r, &lo, &hi);
    rows[r] = lo + hi;
  }
  for (int width = 16; width > 1; width /= 2)
    for (int k = 0; k < width / 2; ++k) rows[k] = rows[2 * k] + rows[2 * k + 1];
  return rows[0];
}

typedef struct {
  const uint16_t* w;
  int rows, cols, mode;
  float g_enc;
  uint8_t *codes, *scales;
  float *err6, *err4;
  float* tile_amax;
  long* tile_use4;
} tile_ctx;

static void tile_amax_item(void* vctx, long item) {
  tile_ctx* c = (tile_ctx*)vctx;
  int tr = (int)(item / (c->cols / 16)), tc = (int)(item % (c->cols / 16));
  float a = 0.0f;
  for (int r = 0; r < 16; ++r)
    for (int j = 0; j < 16; ++j) {
      float v = fabsf(ora_bf16_to_float(c->w[(size_t)(tr * 16 + r) * c->cols + tc * 16 + j]));
      if (v > a) a = v;
    }
  c->tile_amax[item] = a;
}

static void tile_quant_item(void* vctx, long item) {
  tile_ctx* c = (tile_ctx*)vctx;
  int tr = (int)(item / (c->cols / 16)), tc = (int)(item % (c->cols / 16));
  float z[256];
  float t_b = 0.0f;
  for (int r = 0; r < 16; ++r)
    for (int j = 0; j < 16; ++j) {
      float v = ora_bf16_to_float(c->w[(size_t)(tr * 16 + r) * c->cols + tc * 16 + j]);
      z[r * 16 + j] = v * c->g_enc;
      float a = fabsf(z[r * 16 + j]);
      if (a > t_b) t_b = a;
    }
  uint8_t s6 = 0, s4 = 0, q6[256], q4[256];
  float err6 = NAN, err4 = NAN;
  if (c->mode != ORA_MODE_FIXED4) {
    float S, R;
    candidate_scale(t_b, 6.0f, &s6, &S, &R);
    err6 = tile_error(z, 16, S, R, q6);
  }
  if (c->mode != ORA_MODE_FIXED6) {
    float S, R;
    candidate_scale(t_b, 4.0f, &s4, &S, &R);
    err4 = tile_error(z, 16, S, R, q4);
  }
  int use4 = (c->mode == ORA_MODE_FIXED4) || (c->mode == ORA_MODE_4OVER6 && err4 < err6);
  const uint8_t* q = use4 ? q4 : q6;
  for (int r = 0; r < 16; ++r)
    for (int j = 0; j < 8; ++j)
      c->codes[(size_t)(tr * 16 + r) * (c->cols / 2) + tc * 8 + j] =
          (uint8_t)(q[r * 16 + 2 * j] | (q[r * 16 + 2 * j + 1] << 4));
  c->scales[item] = use4 ? s4 : s6;
  if (c->err6) c->err6[item] = err6;
  if (c->err4) c->err4[item] = err4;
  c->tile_use4[item] = use4;
}

/* codes [rows, cols/2], scales [rows/16, cols/16], tensor_scale [1]. */
ORA_API int ora_quantize_2d(const uint16_t* w, int rows, int cols, int mode, uint8_t* codes, uint8_t* scales,
                            float* tensor_scale, float* err6, float* err4, long long* use4_count, int nthreads) {
  if (!w || !codes || !scales || !tensor_scale) return -1;
  if (rows <= 0 || cols <= 0 || rows % 16 || cols % 16) return -2;
  if (mode < 0 || mode > 2) return -6;
  long ntiles = (long)(rows / 16) * (cols / 16);
  float* ta = (float*)malloc(sizeof(float) * (size_t)ntiles);
  long* tu = (long*)malloc(sizeof(long) * (size_t)ntiles);
  if (!ta || !tu) {
    free(ta);
    free(tu);
    return -5;
  }
  tile_ctx c = {w, rows, cols, mode, 0.0f, codes, scales, err6, err4, ta, tu};
  parallel_items(tile_amax_item, &c, ntiles, nthreads);
  float A = 0.0f;
  for (long i = 0; i < ntiles; ++i)
    if (ta[i] > A) A = ta[i];
  float C = mode_constant(mode);
  c.g_enc = A > 0.0f ? C / A : 0.0f;
  tensor_scale[0] = A / C;
  parallel_items(tile_quant_item, &c, ntiles, nthreads);
  long long total4 = 0;
  for (long i = 0; i < ntiles; ++i) total4 += tu[i];
  if (use4_count) *use4_count = total4;
  free(ta);
  free(tu);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Dequantization                                                            */
/* ------------------------------------------------------------------------ */

/* Convention: x_hat = bf16( ((v * S) * g_dec) [+ m] ), each product and the
 * sum one fp32 rounding (v * S is exact), bf16 by round to nearest even. */
typedef struct {
  const uint8_t *codes, *scales;
  const float *tensor_scale, *mean;
  int H, T, D, L;
  uint16_t* out;
} deq_ctx;

static void deq_item(void* vctx, long row) {
  deq_ctx* c = (deq_ctx*)vctx;
  int h = (int)(row / c->T), t = (int)(row % c->T), ch = t / c->L;
  float g = c->tensor_scale[ch];
  for (int d = 0; d < c->D; ++d) {
    uint8_t byte = c->codes[(size_t)row * (c->D / 2) + d / 2];
    uint8_t q = (d & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15u);
    float S = ora_e4m3_decode(c->scales[(size_t)row * (c->D / 16) + d / 16]);
    float v = ora_e2m1_decode(q);
    float vs = v * S;
    float xh = vs * g;
    if (c->mean) xh = xh + c->mean[((size_t)ch * c->H + h) * c->D + d];
    c->out[(size_t)row * c->D + d] = ora_float_to_bf16(xh);
  }
}

ORA_API int ora_dequantize(const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                           const float* mean, int H, int T, int D, int L, uint16_t* out, int nthreads) {
  if (!codes || !scales || !tensor_scale || !out) return -1;
  if (H <= 0 || T <= 0 || D <= 0 || L <= 0 || T % L || D % 16) return -2;
  deq_ctx c = {codes, scales, tensor_scale, mean, H, T, D, L, out};
  parallel_items(deq_item, &c, (long)H * T, nthreads);
  return 0;
}

ORA_API int ora_dequantize_2d(const uint8_t* codes, const uint8_t* scales, const float* tensor_scale, int rows,
                              int cols, uint16_t* out) {
  if (!codes || !scales || !tensor_scale || !out) return -1;
  if (rows <= 0 || cols <= 0 || rows % 16 || cols % 16) return -2;
  float g = tensor_scale[0];
  for (int r = 0; r < rows; ++r)
    for (int d = 0; d < cols; ++d) {
      uint8_t byte = codes[(size_t)r * (cols / 2) + d / 2];
      uint8_t q = (d & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15u);
      float S = ora_e4m3_decode(scales[(size_t)(r / 16) * (cols / 16) + d / 16]);
      float v = ora_e2m1_decode(q);
      float vs = v * S;
      out[(size_t)r * cols + d] = ora_float_to_bf16(vs * g);
    }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* 3-bit and 2-bit KV ([LL2] directions to extend, item 6: a 3-bit / 2-bit  */
/* KV cache)                                                                 */
/* ------------------------------------------------------------------------ */

/* The page names a 3-bit / 2-bit KV cache as a direction without defining a
 * format.  Reading (convention): the NVFP4 layout with fewer element bits.
 *   element: sign bit + (bits - 1) magnitude bits, a minifloat grid:
 *            3 bits: E1M1 (bias 1, with subnormal), magnitudes {0, .5, 1, 1.5};
 *            2 bits: E1M0, magnitudes {0, 1};
 *            nearest magnitude, ties to the even code, saturating at the
 *            largest, sign bit = y's sign bit (so -0 is possible).
 *   block  : 16 consecutive channels, one E4M3FN scale, fp32 tensor scale per
 *            (chunk, tensor), the same smoothing as the 4-bit path.
 *   choice : two candidate scales t_b / c for divisors c_a (maps the block
 *            maximum onto the grid's largest magnitude) and c_b = c_a / 1.5
 *            (3 bits: 1.5 and 1) or c_a * 1.5 (2 bits: 1 and 1.5), the same
 *            3 : 2 ratio as 6 : 4; the lower fp32 error wins, ties keep c_a;
 *            mode 1 uses c_a only, mode 2 c_b only.
 *   C      : 448 * the smallest divisor the mode uses (the largest candidate
 *            scale stays within E4M3's 448).
 *   codes  : element i of a block at bits [bits*i, bits*i + bits) of the
 *            block's little-endian bit field: 6 bytes per block (3 bits), 4
 *            bytes (2 bits); rows of D / 16 blocks.
 * The error, its summation order, the encode domain and the dequantize are
 * those of the 4-bit path. */

static const double FP3_MAG[4] = {0.0, 0.5, 1.0, 1.5};
static const double FP2_MAG[2] = {0.0, 1.0};

static int lowbit_nmag(int bits) { return bits == 3 ? 4 : 2; }
static const double* lowbit_mag(int bits) { return bits == 3 ? FP3_MAG : FP2_MAG; }

ORA_API float ora_lowbit_decode(int bits, uint8_t code) {
  int sbit = bits - 1;
  double m = lowbit_mag(bits)[code & ((1u << sbit) - 1u)];
  return (float)(((code >> sbit) & 1u) ? -m : m);
}

ORA_API uint8_t ora_lowbit_encode(int bits, float y) {
  int sbit = bits - 1, n = lowbit_nmag(bits);
  const double* mag = lowbit_mag(bits);
  uint8_t sign = signbit(y) ? (uint8_t)(1u << sbit) : 0u;
  double a = fabs((double)y);
  if (a >= mag[n - 1]) return (uint8_t)(sign | (n - 1));
  int best = 0;
  double bestd = a;
  for (int k = 1; k < n; ++k) {
    double d = fabs(a - mag[k]);
    if (d < bestd || (d == bestd && (k % 2) == 0)) {
      best = k;
      bestd = d;
    }
  }
  return (uint8_t)(sign | best);
}

static void lowbit_divisors(int bits, float* ca, float* cb) {
  *ca = bits == 3 ? 1.5f : 1.0f;
  *cb = bits == 3 ? 1.0f : 1.5f;
}

static float lowbit_constant(int bits, int mode) {
  float ca, cb;
  lowbit_divisors(bits, &ca, &cb);
  float c = mode == ORA_MODE_FIXED6 ? ca : (mode == ORA_MODE_FIXED4 ? cb : (ca < cb ? ca : cb));
  return 448.0f * c;
}

/* One 16-element block in the encode domain under scale S (reciprocal R):
 * codes q[16] and the fp32 error, two sequential fused halves added. */
static float lowbit_encode16(int bits, const float* z, float S, float R, uint8_t* q) {
  float lo = 0.0f, hi = 0.0f;
  for (int i = 0; i < 16; ++i) {
    float y = z[i] * R;
    q[i] = ora_lowbit_encode(bits, y);
    float v = ora_lowbit_decode(bits, q[i]);
    float vs = v * S;
    float e = z[i] - vs;
    if (i < 8)
      lo = fmaf(e, e, lo);
    else
      hi = fmaf(e, e, hi);
  }
  return lo + hi;
}

static void lowbit_pack(int bits, const uint8_t* q, uint8_t* out) {
  int nbytes = 2 * bits;
  for (int j = 0; j < nbytes; ++j) out[j] = 0;
  for (int i = 0; i < 16; ++i)
    for (int b = 0; b < bits; ++b)
      if ((q[i] >> b) & 1u) {
        int pos = bits * i + b;
        out[pos / 8] |= (uint8_t)(1u << (pos % 8));
      }
}

/* Returns 1 when the c_b candidate was kept. */
static int lowbit_block16(int bits, const float* x, float g_enc, int mode, uint8_t* code_bytes, uint8_t* scale,
                          float* erra_out, float* errb_out) {
  float z[16], t_b = 0.0f, ca, cb;
  lowbit_divisors(bits, &ca, &cb);
  for (int i = 0; i < 16; ++i) {
    z[i] = x[i] * g_enc;
    float a = fabsf(z[i]);
    if (a > t_b) t_b = a;
  }
  uint8_t sa = 0, sb = 0, qa[16], qb[16];
  float erra = NAN, errb = NAN;
  if (mode != ORA_MODE_FIXED4) {
    float S, R;
    candidate_scale(t_b, ca, &sa, &S, &R);
    erra = lowbit_encode16(bits, z, S, R, qa);
  }
  if (mode != ORA_MODE_FIXED6) {
    float S, R;
    candidate_scale(t_b, cb, &sb, &S, &R);
    errb = lowbit_encode16(bits, z, S, R, qb);
  }
  int useb = (mode == ORA_MODE_FIXED4) || (mode == ORA_MODE_4OVER6 && errb < erra);
  lowbit_pack(bits, useb ? qb : qa, code_bytes);
  *scale = useb ? sb : sa;
  if (erra_out) *erra_out = erra;
  if (errb_out) *errb_out = errb;
  return useb;
}

typedef struct {
  int bits, mode, D, L, T, H, chunk, items_per_head;
  const float* xp;  /* prepared (smoothed) fp32 chunk [H, L, D] */
  float g_enc;
  uint8_t *codes, *scales;
  float *erra, *errb;
  long* item_useb;
} lowbit_ctx;

static void lowbit_item(void* vctx, long item) {
  lowbit_ctx* c = (lowbit_ctx*)vctx;
  int h = (int)(item / c->items_per_head);
  int r0 = (int)(item % c->items_per_head) * ROWS_PER_ITEM;
  int r1 = r0 + ROWS_PER_ITEM < c->L ? r0 + ROWS_PER_ITEM : c->L;
  int nb = c->D / 16, cb = 2 * c->bits;
  long useb = 0;
  for (int r = r0; r < r1; ++r) {
    size_t row = (size_t)h * c->T + (size_t)c->chunk * c->L + r;
    const float* src = c->xp + ((size_t)h * c->L + r) * c->D;
    for (int b = 0; b < nb; ++b) {
      size_t blk = row * nb + b;
      float ea, eb;
      useb += lowbit_block16(c->bits, src + 16 * b, c->g_enc, c->mode, c->codes + blk * cb, c->scales + blk, &ea,
                             &eb);
      if (c->erra) c->erra[blk] = ea;
      if (c->errb) c->errb[blk] = eb;
    }
  }
  c->item_useb[item] = useb;
}

/*
 * 3-bit / 2-bit quantization of x [H, T, D] (bf16 bits), chunk by chunk,
 * smoothed by `mean` when given (as ora_quantize_chunks).
 *   codes [H, T, D * bits / 8], scales [H, T, D / 16], tensor_scale [T / L].
 *   erra / errb: NULL or per-block errors of the c_a / c_b candidates.
 */
ORA_API int ora_quantize_chunks_lowbit(const uint16_t* x, int H, int T, int D, int L, int bits, int mode,
                                       const float* mean, uint8_t* codes, uint8_t* scales, float* tensor_scale,
                                       float* erra, float* errb, long long* useb_count, int nthreads) {
  if (!x || !codes || !scales || !tensor_scale) return -1;
  if (H <= 0 || T <= 0 || D <= 0 || L <= 0 || T % L || D % 16) return -2;
  if (bits != 3 && bits != 2) return -2;
  if (mode < 0 || mode > 2) return -6;
  int items_per_head = (L + ROWS_PER_ITEM - 1) / ROWS_PER_ITEM;
  long nitems = (long)H * items_per_head;
  float* xp = (float*)malloc(sizeof(float) * (size_t)H * L * D);
  float* amax = (float*)malloc(sizeof(float) * (size_t)nitems);
  long* ub = (long*)malloc(sizeof(long) * (size_t)nitems);
  if (!xp || !amax || !ub) {
    free(xp);
    free(amax);
    free(ub);
    return -5;
  }
  float C = lowbit_constant(bits, mode);
  long long total = 0;
  for (int ch = 0; ch < T / L; ++ch) {
    /* step 1: smoothing and the chunk's largest magnitude, as the 4-bit path */
    chunk_ctx pc;
    memset(&pc, 0, sizeof pc);
    pc.x = x;
    pc.H = H;
    pc.T = T;
    pc.D = D;
    pc.L = L;
    pc.chunk = ch;
    pc.mean = mean ? mean + (size_t)ch * H * D : NULL;
    pc.xp = xp;
    pc.item_amax = amax;
    pc.items_per_head = items_per_head;
    parallel_items(prepare_item, &pc, nitems, nthreads);
    float A = 0.0f;
    for (long i = 0; i < nitems; ++i)
      if (amax[i] > A) A = amax[i];
    /* step 2: the blocks */
    lowbit_ctx c = {bits, mode, D, L, T, H, ch, items_per_head, xp, A > 0.0f ? C / A : 0.0f,
                    codes, scales, erra, errb, ub};
    tensor_scale[ch] = A / C;
    parallel_items(lowbit_item, &c, nitems, nthreads);
    for (long i = 0; i < nitems; ++i) total += ub[i];
  }
  if (useb_count) *useb_count = total;
  free(xp);
  free(amax);
  free(ub);
  return 0;
}

/* x_hat = bf16( ((v * S) * g_dec) [+ m] ), as the 4-bit dequantize. */
typedef struct {
  const uint8_t *codes, *scales;
  const float *tensor_scale, *mean;
  int H, T, D, L, bits;
  uint16_t* out;
} deq_lowbit_ctx;

static void deq_lowbit_item(void* vctx, long row) {
  deq_lowbit_ctx* c = (deq_lowbit_ctx*)vctx;
  int h = (int)(row / c->T), t = (int)(row % c->T), ch = t / c->L;
  float g = c->tensor_scale[ch];
  int rowbytes = c->D * c->bits / 8;
  for (int d = 0; d < c->D; ++d) {
    int pos = c->bits * d, q = 0;
    for (int b = 0; b < c->bits; ++b) {
      int bit = pos + b;
      q |= ((c->codes[(size_t)row * rowbytes + bit / 8] >> (bit % 8)) & 1) << b;
    }
    float S = ora_e4m3_decode(c->scales[(size_t)row * (c->D / 16) + d / 16]);
    float v = ora_lowbit_decode(c->bits, (uint8_t)q);
    float vs = v * S;
    float xh = vs * g;
    if (c->mean) xh = xh + c->mean[((size_t)ch * c->H + h) * c->D + d];
    c->out[(size_t)row * c->D + d] = ora_float_to_bf16(xh);
  }
}

ORA_API int ora_dequantize_lowbit(const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                                  const float* mean, int H, int T, int D, int L, int bits, uint16_t* out,
                                  int nthreads) {
  if (!codes || !scales || !tensor_scale || !out) return -1;
  if (H <= 0 || T <= 0 || D <= 0 || L <= 0 || T % L || D % 16 || (bits != 3 && bits != 2)) return -2;
  deq_lowbit_ctx c = {codes, scales, tensor_scale, mean, H, T, D, L, bits, out};
  parallel_items(deq_lowbit_item, &c, (long)H * T, nthreads);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Attention over the NVFP4 cache (consumer of [LL2] inference pipeline,     */
/* steps 7 and 9)                                                            */
/* ------------------------------------------------------------------------ */

/* The page builds the cache for attention (step 7) and attends to a key set
 * made of sink frames and the current window (step 9), but prints no
 * attention formula.  Reading (convention): ordinary softmax attention of
 * each query over the listed keys, with K and V the values the cache
 * represents, taken exactly (no bf16 step):
 *   K[j][d] = v * S * g_K[c] + m[c][d],   V[j][d] = v * S * g_V[c],
 * c = j / L the key's chunk, v the E2M1 value, S the E4M3 block scale.
 *   s_j = scale * sum_d q[d] K[j][d],   p_j = exp(s_j) / sum_j' exp(s_j'),
 *   out[d] = sum_j p_j V[j][d],   lse = log sum_j exp(s_j).
 * The key set is the concatenation of the ranges [start, start + len) (a key
 * listed twice counts twice); an empty set gives out = 0 and lse = -inf.
 * Query head h reads cache head h / (H / H_kv).  Everything in double. */
typedef struct {
  const uint16_t* q;
  int H, Tq, D;
  const uint8_t *kc, *ks, *vc, *vs;
  const float *kg, *vg, *km;
  int Hkv, T, L;
  const int* ranges;
  int nr;
  double scale;
  const long* rows;
  double *out, *lse;
} att_ctx;

/* Row j of one cache tensor of head kvh, decoded exactly into x[0..D). */
static void att_decode_row(const uint8_t* codes, const uint8_t* scales, const float* g, const float* mean, int Hkv,
                           int T, int D, int L, int kvh, long j, double* x) {
  long row = (long)kvh * T + j;
  int c = (int)(j / L);
  for (int d = 0; d < D; ++d) {
    uint8_t byte = codes[row * (D / 2) + d / 2];
    uint8_t code = (d & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15u);
    double v = (double)ora_e2m1_decode(code);
    double S = (double)ora_e4m3_decode(scales[row * (D / 16) + d / 16]);
    x[d] = v * S * (double)g[c];
    if (mean) x[d] += (double)mean[((size_t)c * Hkv + kvh) * D + d];
  }
}

static void att_item(void* vctx, long item) {
  att_ctx* c = (att_ctx*)vctx;
  long r = c->rows ? c->rows[item] : item;
  int h = (int)(r / c->Tq), i = (int)(r % c->Tq), D = c->D;
  int kvh = h / (c->H / c->Hkv);
  long nk = 0;
  for (int k = 0; k < c->nr; ++k) nk += c->ranges[2 * k + 1];
  double* out = c->out + (size_t)item * D;
  for (int d = 0; d < D; ++d) out[d] = 0.0;
  if (nk == 0) {
    c->lse[item] = -INFINITY;
    return;
  }
  double* s = (double*)malloc(sizeof(double) * (size_t)nk);
  double* x = (double*)malloc(sizeof(double) * (size_t)D);
  double* qd = (double*)malloc(sizeof(double) * (size_t)D);
  if (!s || !x || !qd) { /* out of memory: the row reads NaN */
    for (int d = 0; d < D; ++d) out[d] = NAN;
    c->lse[item] = NAN;
    free(s);
    free(x);
    free(qd);
    return;
  }
  for (int d = 0; d < D; ++d) qd[d] = (double)ora_bf16_to_float(c->q[((size_t)h * c->Tq + i) * D + d]);
  /* scores */
  long n = 0;
  for (int k = 0; k < c->nr; ++k)
    for (long j = c->ranges[2 * k]; j < (long)c->ranges[2 * k] + c->ranges[2 * k + 1]; ++j) {
      att_decode_row(c->kc, c->ks, c->kg, c->km, c->Hkv, c->T, D, c->L, kvh, j, x);
      double dot = 0.0;
      for (int d = 0; d < D; ++d) dot += qd[d] * x[d];
      s[n++] = c->scale * dot;
    }
  /* softmax with the largest score subtracted, then the weighted sum of V */
  double mx = s[0];
  for (long j = 1; j < nk; ++j)
    if (s[j] > mx) mx = s[j];
  double l = 0.0;
  for (long j = 0; j < nk; ++j) {
    s[j] = exp(s[j] - mx);
    l += s[j];
  }
  n = 0;
  for (int k = 0; k < c->nr; ++k)
    for (long j = c->ranges[2 * k]; j < (long)c->ranges[2 * k] + c->ranges[2 * k + 1]; ++j) {
      att_decode_row(c->vc, c->vs, c->vg, NULL, c->Hkv, c->T, D, c->L, kvh, j, x);
      double p = s[n++] / l;
      for (int d = 0; d < D; ++d) out[d] += p * x[d];
    }
  c->lse[item] = mx + log(l);
  free(s);
  free(x);
  free(qd);
}

/* q bf16 [H, Tq, D]; cache tensors as the quantizer writes them ([H_kv, T, D/2]
 * codes, [H_kv, T, D/16] scales, [T/L] tensor scales, k_mean [T/L, H_kv, D] or
 * NULL); ranges [n_ranges][2] = (start, len).  rows: NULL for every (h, i) in
 * order, else n_rows flat indices h * Tq + i.  out double [rows][D], lse
 * double [rows]. */
ORA_API int ora_kv_attention(const uint16_t* q, int H, int Tq, int D, const uint8_t* k_codes,
                             const uint8_t* k_scales, const float* k_tensor_scale, const float* k_mean,
                             const uint8_t* v_codes, const uint8_t* v_scales, const float* v_tensor_scale, int Hkv,
                             int T, int L, const int* ranges, int n_ranges, double scale, const long* rows,
                             long n_rows, double* out, double* lse, int nthreads) {
  if (!q || !k_codes || !k_scales || !k_tensor_scale || !v_codes || !v_scales || !v_tensor_scale || !out || !lse)
    return -1;
  if (H <= 0 || Tq < 0 || D <= 0 || D % 16 || Hkv <= 0 || H % Hkv || T < 0 || L <= 0 || T % L || n_ranges < 0)
    return -2;
  if (n_ranges > 0 && !ranges) return -1;
  for (int k = 0; k < n_ranges; ++k)
    if (ranges[2 * k] < 0 || ranges[2 * k + 1] < 0 || (long)ranges[2 * k] + ranges[2 * k + 1] > T) return -2;
  long n = rows ? n_rows : (long)H * Tq;
  for (long r = 0; rows && r < n_rows; ++r)
    if (rows[r] < 0 || rows[r] >= (long)H * Tq) return -2;
  att_ctx c = {q, H, Tq, D, k_codes, k_scales, v_codes, v_scales, k_tensor_scale, v_tensor_scale, k_mean,
               Hkv, T, L, ranges, n_ranges, scale, rows, out, lse};
  parallel_items(att_item, &c, n, nthreads);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* W4A4 GEMM on NVFP4 operands ([LL2] training pipeline, step 4; inference   */
/* pipeline, step 6)                                                         */
/* ------------------------------------------------------------------------ */

/* The page runs its linear layers as NVFP4 GEMMs with 1D block scales on the
 * activation and 2D block scales on the weight, and gives no formula.
 * Reading (convention): the product of the two dequantized operands along
 * their shared K axis, taken exactly,
 *   out[m][n] = sum_k A[m][k] * W[n][k],
 *   A[m][k] = v * S_A(m, k/16) * g_A,   W[n][k] = v * S_W(blk) * g_W,
 * with blk = (n, k/16) for 1D weight blocks or (n/16, k/16) for 2D tiles.
 * A rotation applied before quantization (the RHT) is not undone: the
 * product is that of the stored operands.  Everything in double. */
typedef struct {
  const uint8_t *ac, *as, *wc, *ws;
  double ga, gw;
  int M, N, K, w2d;
  double* out;
} gemm_ctx;

static void gemm_row(void* vctx, long m) {
  gemm_ctx* c = (gemm_ctx*)vctx;
  int K = c->K;
  double* a = (double*)malloc(sizeof(double) * (size_t)K);
  double* out = c->out + (size_t)m * c->N;
  if (!a) {
    for (int n = 0; n < c->N; ++n) out[n] = NAN;
    return;
  }
  for (int k = 0; k < K; ++k) {
    uint8_t byte = c->ac[(size_t)m * (K / 2) + k / 2];
    uint8_t code = (k & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15u);
    a[k] = (double)ora_e2m1_decode(code) * (double)ora_e4m3_decode(c->as[(size_t)m * (K / 16) + k / 16]) * c->ga;
  }
  for (int n = 0; n < c->N; ++n) {
    double acc = 0.0;
    for (int k = 0; k < K; ++k) {
      uint8_t byte = c->wc[(size_t)n * (K / 2) + k / 2];
      uint8_t code = (k & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15u);
      size_t si = c->w2d ? (size_t)(n / 16) * (K / 16) + k / 16 : (size_t)n * (K / 16) + k / 16;
      double w = (double)ora_e2m1_decode(code) * (double)ora_e4m3_decode(c->ws[si]) * c->gw;
      acc += a[k] * w;
    }
    out[n] = acc;
  }
  free(a);
}

/* a: codes [M, K/2], scales [M, K/16], tensor scale; w: codes [N, K/2],
 * scales [N, K/16] (w2d = 0) or [N/16, K/16] (w2d = 1), tensor scale.
 * out double [M, N]. */
ORA_API int ora_gemm_w4a4(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_tensor_scale, int M,
                          int K, const uint8_t* w_codes, const uint8_t* w_scales, const float* w_tensor_scale,
                          int N, int w2d, double* out, int nthreads) {
  if (!a_codes || !a_scales || !a_tensor_scale || !w_codes || !w_scales || !w_tensor_scale || !out) return -1;
  if (M < 0 || N < 0 || K <= 0 || K % 16 || (w2d && N % 16)) return -2;
  gemm_ctx c = {a_codes, a_scales, w_codes, w_scales, (double)a_tensor_scale[0], (double)w_tensor_scale[0],
                M, N, K, w2d != 0, out};
  parallel_items(gemm_row, &c, M, nthreads);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Array helpers for the tests                                              */
/* ------------------------------------------------------------------------ */

typedef struct {
  const void* in;
  void* out;
  long n;
  int kind;
} arr_ctx;

#define ARR_SPAN 65536
static void arr_item(void* vctx, long item) {
  arr_ctx* c = (arr_ctx*)vctx;
  long i0 = item * ARR_SPAN, i1 = i0 + ARR_SPAN < c->n ? i0 + ARR_SPAN : c->n;
  for (long i = i0; i < i1; ++i) {
    switch (c->kind) {
      case 0: ((uint8_t*)c->out)[i] = ora_e2m1_encode(((const float*)c->in)[i]); break;
      case 1: ((uint8_t*)c->out)[i] = ora_e4m3_encode(((const float*)c->in)[i]); break;
      case 2: ((uint16_t*)c->out)[i] = ora_float_to_bf16(((const float*)c->in)[i]); break;
      case 3: ((float*)c->out)[i] = ora_e2m1_decode(((const uint8_t*)c->in)[i]); break;
      case 4: ((float*)c->out)[i] = ora_e4m3_decode(((const uint8_t*)c->in)[i]); break;
      case 5: ((uint8_t*)c->out)[i] = ora_lowbit_encode(3, ((const float*)c->in)[i]); break;
      case 6: ((uint8_t*)c->out)[i] = ora_lowbit_encode(2, ((const float*)c->in)[i]); break;
      default: break;
    }
  }
}

static void run_array(const void* in, void* out, long n, int kind, int nthreads) {
  arr_ctx c = {in, out, n, kind};
  parallel_items(arr_item, &c, (n + ARR_SPAN - 1) / ARR_SPAN, nthreads);
}

ORA_API void ora_e2m1_encode_array(const float* y, long n, uint8_t* out, int nt) { run_array(y, out, n, 0, nt); }
ORA_API void ora_e4m3_encode_array(const float* r, long n, uint8_t* out, int nt) { run_array(r, out, n, 1, nt); }
ORA_API void ora_float_to_bf16_array(const float* x, long n, uint16_t* out, int nt) { run_array(x, out, n, 2, nt); }
ORA_API void ora_e2m1_decode_array(const uint8_t* q, long n, float* out, int nt) { run_array(q, out, n, 3, nt); }
ORA_API void ora_e4m3_decode_array(const uint8_t* s, long n, float* out, int nt) { run_array(s, out, n, 4, nt); }
ORA_API void ora_lowbit_encode_array(int bits, const float* y, long n, uint8_t* out, int nt) {
  run_array(y, out, n, bits == 3 ? 5 : 6, nt);
}

/* E4M3 code of the candidate t / c (c = 6 or 4), as the quantizer forms it. */
ORA_API void ora_candidate_codes(const float* t, long n, float c, uint8_t* out) {
  for (long i = 0; i < n; ++i) {
    float r = t[i] / c;
    out[i] = ora_e4m3_encode(r);
  }
}
