/*
 * Codec-Gauge CPU ORACLE -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously-correct C implementation of the integer and
 * fixed-precision parts of the Codec-Gauge KV-cache round trip, used only by
 * the tests, by the package's smoke check and by the benchmark's CPU-baseline
 * leg.  It shares no code, header, table or constant generator with the HIP
 * library; nothing on the product path may load it.
 *
 * Sources (page titles; the arXiv HTML page has lost its headings, so its
 * paragraphs are named by topic):
 *  - "Codec-Gauge: Learning Compression-Friendly Gauges for Transformer KV
 *    Caches" (arXiv 2607.20538 HTML): gauge parameterization paragraph
 *    (G = exp(A - A^T), orthogonal, per layer / cache type / head / group);
 *    evaluation-protocol paragraph on backends (fixed-rate zfp on contiguous
 *    FP32-transformed tensors presented as a 2D field with n_x = d_l and
 *    n_y = numel / d_l; block-uniform ranges per T_b x d_l block; KIVI-style
 *    per-channel key / per-token value ranges).
 *  - The Chinese translation of the same paper ("Codec-Gauge：为Transformer
 *    KV缓存学习压缩友好的变换框架"), problem statement: X[b,h,t,r] in R^g,
 *    the gauge mixes channels within a group only, never tokens/heads/layers.
 *  - The zfp block coder the paper cites (Lindstrom 2014) is not on the
 *    pages; the reading used here (exponent header, block-floating-point
 *    quantization, the 4-point decorrelating transform with matrix
 *    F = 1/16 [[4,4,4,4],[5,1,-1,-5],[-4,4,4,-4],[-2,6,-6,2]], total-sequency
 *    ordering, negabinary, group-tested embedded bit planes) follows that
 *    published method's steps in order; the choices it leaves open are
 *    stated where they are made below.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -shared -fPIC.
 * FMA contraction is off so every multiply and add below rounds as written;
 * fmaf() is used exactly where a fused multiply-add is specified.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* bf16 helpers (storage format only)                                        */
/* ------------------------------------------------------------------------ */

/* bf16 -> fp32 is exact: the bf16 bits are the top half of the fp32 bits. */
float oracle_bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* fp32 -> bf16, round to nearest, ties to even (finite inputs). */
uint16_t oracle_f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  uint32_t keep = u >> 16;
  uint32_t rest = u & 0xFFFFu;
  if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u))) keep += 1u;
  return (uint16_t)keep;
}

void oracle_bf16_to_f32_array(int64_t n, const uint16_t *in, float *out) {
  for (int64_t i = 0; i < n; i++) out[i] = oracle_bf16_to_f32(in[i]);
}

void oracle_f32_to_bf16_array(int64_t n, const float *in, uint16_t *out) {
  for (int64_t i = 0; i < n; i++) out[i] = oracle_f32_to_bf16(in[i]);
}

/* ------------------------------------------------------------------------ */
/* Gauge application (arXiv page, gauge parameterization paragraph: X' = G X */
/* per token and per g-channel group; the inverse of an orthogonal G is G^T) */
/* ------------------------------------------------------------------------ */

/*
 * x: [T][d] fp32, G: [d/g][g][g] fp32 row-major.  For each token t and group
 * r: y[t][r*g+i] = sum_k G[r][i][k] * x[t][r*g+k], evaluated as a chain of
 * fmaf over k = 0..g-1 starting from +0.0f.  g == 0 means the identity gauge
 * (a plain copy, no arithmetic).
 */
void oracle_gauge_forward(int64_t T, int d, int g, const float *G,
                          const float *x, float *y) {
  if (g == 0) {
    memcpy(y, x, (size_t)T * (size_t)d * sizeof(float));
    return;
  }
  int R = d / g;
  for (int64_t t = 0; t < T; t++) {
    const float *xt = x + t * d;
    float *yt = y + t * d;
    for (int r = 0; r < R; r++) {
      const float *Gr = G + (size_t)r * g * g;
      for (int i = 0; i < g; i++) {
        float acc = 0.0f;
        for (int k = 0; k < g; k++) acc = fmaf(Gr[i * g + k], xt[r * g + k], acc);
        yt[r * g + i] = acc;
      }
    }
  }
}

/*
 * Inverse gauge: x[t][r*g+k] = sum_i G[r][i][k] * y[t][r*g+i] (that is G^T y),
 * as an fmaf chain over i = 0..g-1 from +0.0f.
 */
void oracle_gauge_inverse(int64_t T, int d, int g, const float *G,
                          const float *y, float *x) {
  if (g == 0) {
    memcpy(x, y, (size_t)T * (size_t)d * sizeof(float));
    return;
  }
  int R = d / g;
  for (int64_t t = 0; t < T; t++) {
    const float *yt = y + t * d;
    float *xt = x + t * d;
    for (int r = 0; r < R; r++) {
      const float *Gr = G + (size_t)r * g * g;
      for (int k = 0; k < g; k++) {
        float acc = 0.0f;
        for (int i = 0; i < g; i++) acc = fmaf(Gr[i * g + k], yt[r * g + i], acc);
        xt[r * g + k] = acc;
      }
    }
  }
}

/* ------------------------------------------------------------------------ */
/* Bit stream: bit p of the stream is bit (p mod 8) of byte p / 8, which is  */
/* the same as bit (p mod 64) of little-endian 64-bit word p / 64.            */
/* ------------------------------------------------------------------------ */

typedef struct {
  uint8_t *buf;
  uint64_t pos;
} bitwriter;

static void put_bit(bitwriter *w, unsigned bit) {
  if (bit & 1u) w->buf[w->pos >> 3] |= (uint8_t)(1u << (w->pos & 7u));
  else w->buf[w->pos >> 3] &= (uint8_t)~(1u << (w->pos & 7u));
  w->pos++;
}

/* n low bits of v, least significant first */
static void put_bits(bitwriter *w, uint64_t v, int n) {
  for (int i = 0; i < n; i++) put_bit(w, (unsigned)(v >> i) & 1u);
}

typedef struct {
  const uint8_t *buf;
  uint64_t pos;
} bitreader;

static unsigned get_bit(bitreader *r) {
  unsigned b = (r->buf[r->pos >> 3] >> (r->pos & 7u)) & 1u;
  r->pos++;
  return b;
}

static uint64_t get_bits(bitreader *r, int n) {
  uint64_t v = 0;
  for (int i = 0; i < n; i++) v |= (uint64_t)get_bit(r) << i;
  return v;
}

/* ------------------------------------------------------------------------ */
/* zfp-style fixed-rate 4x4 block coder                                      */
/* ------------------------------------------------------------------------ */

/*
 * Total-sequency order of the 16 coefficients (i = channel frequency,
 * j = token frequency, stored at index i + 4 j): sort by i + j, then by
 * i^2 + j^2, then larger i first.  Built once by brute-force sorting.
 */
static int seq_order[16];
static int seq_ready = 0;
static void build_seq_order(void);
/* built once when the library is loaded, before any thread can use it */
__attribute__((constructor)) static void seq_order_init(void) { build_seq_order(); }

static int seq_key_less(int a, int b) {
  int ia = a & 3, ja = a >> 2, ib = b & 3, jb = b >> 2;
  if (ia + ja != ib + jb) return ia + ja < ib + jb;
  if (ia * ia + ja * ja != ib * ib + jb * jb) return ia * ia + ja * ja < ib * ib + jb * jb;
  return ia > ib;
}

static void build_seq_order(void) {
  if (seq_ready) return;
  for (int k = 0; k < 16; k++) seq_order[k] = k;
  for (int a = 0; a < 16; a++)          /* plain selection sort */
    for (int b = a + 1; b < 16; b++)
      if (seq_key_less(seq_order[b], seq_order[a])) {
        int t = seq_order[a];
        seq_order[a] = seq_order[b];
        seq_order[b] = t;
      }
  seq_ready = 1;
}

void oracle_sequency_order(int32_t out[16]) {
  build_seq_order();
  for (int k = 0; k < 16; k++) out[k] = seq_order[k];
}

/*
 * One 4-point forward transform on p[0], p[s], p[2s], p[3s]: an integer
 * lifting realization of F = 1/16 [[4,4,4,4],[5,1,-1,-5],[-4,4,4,-4],
 * [-2,6,-6,2]], derived by factoring F into pairwise means / half
 * differences followed by one lifting rotation (>> is an arithmetic shift,
 * i.e. floor division by a power of two):
 *   1. outer pair:        a <- (a+d)>>1,   d <- d - a
 *   2. inner pair:        c <- (b+c)>>1,   b <- b - c
 *   3. the two means:     a <- (a+c)>>1,   c <- c - a      (DC, F row 2)
 *   4. the two halves:    d <- (d+b)>>1,   b <- b - d
 *   5. rotation:          d <- d + (b>>1), b <- b - (d>>1)  (F rows 3, 1)
 * Output order (a, b, c, d) = (F row 0, row 1, row 2, row 3) applied to the
 * input, up to the floor roundings.  Every intermediate stays inside int32
 * for |inputs| < 2^30.
 */
static int32_t wadd(int32_t a, int32_t b) { return (int32_t)((uint32_t)a + (uint32_t)b); }
static int32_t wsub(int32_t a, int32_t b) { return (int32_t)((uint32_t)a - (uint32_t)b); }
static int32_t wdbl(int32_t a) { return (int32_t)((uint32_t)a << 1); }

static void fwd_lift(int32_t *p, int s) {
  int32_t a = p[0], b = p[s], c = p[2 * s], d = p[3 * s];
  a = wadd(a, d) >> 1;  d = wsub(d, a);
  c = wadd(b, c) >> 1;  b = wsub(b, c);
  a = wadd(a, c) >> 1;  c = wsub(c, a);
  d = wadd(d, b) >> 1;  b = wsub(b, d);
  d = wadd(d, b >> 1);  b = wsub(b, d >> 1);
  p[0] = a; p[s] = b; p[2 * s] = c; p[3 * s] = d;
}

/*
 * Exact inverse of each lifting step above, applied in reverse order (a
 * mean step x <- (x+y)>>1, y <- y - x is undone by y <- y + x, x <- 2x - y,
 * which restores the pair up to the bit the shift dropped).  Arithmetic
 * wraps modulo 2^32 so that arbitrary (corrupt) streams decode without
 * undefined behaviour.
 */
static void inv_lift(int32_t *p, int s) {
  int32_t a = p[0], b = p[s], c = p[2 * s], d = p[3 * s];
  b = wadd(b, d >> 1);  d = wsub(d, b >> 1);      /* undo 5 */
  b = wadd(b, d);       d = wsub(wdbl(d), b);     /* undo 4 */
  c = wadd(c, a);       a = wsub(wdbl(a), c);     /* undo 3 */
  b = wadd(b, c);       c = wsub(wdbl(c), b);     /* undo 2 */
  d = wadd(d, a);       a = wsub(wdbl(a), d);     /* undo 1 */
  p[0] = a; p[s] = b; p[2 * s] = c; p[3 * s] = d;
}

/* test exports of the 1D transforms */
void oracle_fwd_lift4(int32_t v[4]) { fwd_lift(v, 1); }
void oracle_inv_lift4(int32_t v[4]) { inv_lift(v, 1); }

#define NEGA_MASK 0xAAAAAAAAu

/*
 * Steps 1-5 for one 4x4 block v[j*4+i] (j = token row, i = channel): block
 * exponent, block-floating-point integers, 2D transform, total-sequency
 * order, negabinary.  Returns 0 for an all-zero block (u, *emax untouched).
 */
static int block_words(const float v[16], uint32_t u[16], int *emax_out) {
  /* step 1: block exponent (frexp convention, |m| in [0.5, 1)), clamped */
  int nonzero = 0, emax = -100000;
  for (int k = 0; k < 16; k++) {
    if (v[k] != 0.0f) {
      int e;
      frexpf(v[k], &e);
      nonzero = 1;
      if (e > emax) emax = e;
    }
  }
  if (!nonzero) return 0;
  if (emax < -126) emax = -126;

  /* step 2: block floating point -> int32 (truncation toward zero) */
  int32_t q[16];
  for (int k = 0; k < 16; k++) q[k] = (int32_t)ldexpf(v[k], 30 - emax);

  /* step 3: transform along channels (each token row), then along tokens */
  for (int j = 0; j < 4; j++) fwd_lift(q + 4 * j, 1);
  for (int i = 0; i < 4; i++) fwd_lift(q + i, 4);

  /* steps 4-5: total-sequency order, negabinary */
  for (int k = 0; k < 16; k++)
    u[k] = ((uint32_t)q[seq_order[k]] + NEGA_MASK) ^ NEGA_MASK;
  *emax_out = emax;
  return 1;
}

/*
 * Step 6: embedded coding of bit planes 31..0 of u[] with `beta` bits.
 * Plane k is the 16-bit word whose bit i is bit k of u[i].  Per plane: the
 * bits of the n coefficients already significant are sent verbatim; then
 * group tests ("is any further bit of this plane set?"), each positive one
 * followed by a unary scan up to the next set bit, which makes that
 * coefficient significant.  A scan that reaches position 15 stops: the one
 * there is implied.  Emission stops the moment the budget is spent.
 */
static void code_planes(const uint32_t u[16], int beta, bitwriter *w) {
  int n = 0;
  for (int k = 31; k >= 0 && beta > 0; k--) {
    uint32_t x = 0;
    for (int i = 0; i < 16; i++) x |= ((u[i] >> k) & 1u) << i;
    /* (a) verbatim bits of the n coefficients already significant */
    int m = n < beta ? n : beta;
    put_bits(w, x, m);
    beta -= m;
    x >>= m;
    /* (b) group tests, each followed by a unary scan to the next one */
    while (n < 16 && beta > 0) {
      unsigned t = x != 0;
      put_bit(w, t);
      beta--;
      if (!t) break;
      while (n < 15 && beta > 0) {
        unsigned bit = x & 1u;
        put_bit(w, bit);
        beta--;
        if (bit) break;
        x >>= 1;
        n++;
      }
      x >>= 1;
      n++;
    }
  }
}

/*
 * Encode one block at rate R (bits per value) into exactly 16*R bits at the
 * writer position: a 1-bit nonzero flag, the 8-bit biased exponent
 * emax + 127 (LSB first), the plane code under the budget 16R - 9, zero
 * padding.  An all-zero block is a single 0 bit followed by padding.
 */
static void zfp_encode_block(const float v[16], int R, bitwriter *w) {
  const uint64_t end = w->pos + 16u * (uint64_t)R;
  uint32_t u[16];
  int emax;
  if (!block_words(v, u, &emax)) {
    put_bit(w, 0);
    while (w->pos < end) put_bit(w, 0);
    return;
  }
  put_bit(w, 1);
  put_bits(w, (uint64_t)(emax + 127), 8);
  code_planes(u, 16 * R - 9, w);
  while (w->pos < end) put_bit(w, 0);
}

/* Mirror of code_planes: rebuild the negabinary words from `beta` bits. */
static void decode_planes(bitreader *r, int beta, uint32_t u[16]) {
  memset(u, 0, 16 * sizeof(uint32_t));
  int n = 0;
  for (int k = 31; k >= 0 && beta > 0; k--) {
    int m = n < beta ? n : beta;
    uint32_t x = (uint32_t)get_bits(r, m);
    beta -= m;
    while (n < 16 && beta > 0) {
      unsigned t = get_bit(r);
      beta--;
      if (!t) break;
      while (n < 15 && beta > 0) {
        unsigned bit = get_bit(r);
        beta--;
        if (bit) break;
        n++;
      }
      /* the one ends the scan; when the budget ran out inside the scan the
         bit at the current position is still set */
      x |= 1u << n;
      n++;
    }
    for (int i = 0; i < 16; i++) u[i] |= ((x >> i) & 1u) << k;
  }
}

/* Inverse of steps 5..2: negabinary -> int, natural order, inverse
   transform (tokens first, then channels), scale by 2^(emax-30). */
static void block_values(const uint32_t u[16], int emax, float v[16]) {
  int32_t q[16];
  for (int k = 0; k < 16; k++)
    q[seq_order[k]] = (int32_t)((u[k] ^ NEGA_MASK) - NEGA_MASK); /* mod 2^32 */
  for (int i = 0; i < 4; i++) inv_lift(q + i, 4);
  for (int j = 0; j < 4; j++) inv_lift(q + 4 * j, 1);
  for (int k = 0; k < 16; k++) v[k] = ldexpf((float)q[k], emax - 30);
}

static void zfp_decode_block(bitreader *r, int R, float v[16]) {
  const uint64_t end = r->pos + 16u * (uint64_t)R;
  if (!get_bit(r)) {
    for (int k = 0; k < 16; k++) v[k] = 0.0f;
    r->pos = end;
    return;
  }
  int emax = (int)get_bits(r, 8) - 127;
  uint32_t u[16];
  decode_planes(r, 16 * R - 9, u);
  r->pos = end;
  block_values(u, emax, v);
}

/* stage test exports */
int oracle_zfp_block_words(const float v[16], uint32_t u[16], int32_t *emax) {
  int e = 0;
  int nz = block_words(v, u, &e);
  *emax = e;
  return nz;
}

/* decode the plane code of one block; returns the nonzero flag */
int oracle_zfp_decode_block_words(const uint8_t *in, int R, uint32_t u[16], int32_t *emax) {
  bitreader r = {in, 0};
  if (!get_bit(&r)) {
    memset(u, 0, 16 * sizeof(uint32_t));
    *emax = 0;
    return 0;
  }
  *emax = (int)get_bits(&r, 8) - 127;
  decode_planes(&r, 16 * R - 9, u);
  return 1;
}

/* single-block test exports: out holds 2*R bytes */
void oracle_zfp_encode_block(const float v[16], int R, uint8_t *out) {
  bitwriter w = {out, 0};
  zfp_encode_block(v, R, &w);
}

void oracle_zfp_decode_block(const uint8_t *in, int R, float v[16]) {
  bitreader r = {in, 0};
  zfp_decode_block(&r, R, v);
}

/*
 * Encode token rows [t0, t0+nt) of one field x[T][d] (T and d multiples of
 * 4).  Blocks are taken in raster order (channel block bx fastest, then token
 * block by); block (bx, by) occupies stream bits
 * [(by*(d/4)+bx)*16R, +16R) of `out`, so a field occupies T*d*R/8 bytes and
 * an append of rows [t0, t0+nt) touches only its own block rows.
 */
void oracle_zfp_encode_field(int64_t t0, int64_t nt, int d, int R,
                             const float *x, uint8_t *out) {
  int nbx = d / 4;
  for (int64_t by = t0 / 4; by < (t0 + nt) / 4; by++)
    for (int bx = 0; bx < nbx; bx++) {
      float v[16];
      for (int j = 0; j < 4; j++)
        for (int i = 0; i < 4; i++) v[4 * j + i] = x[(4 * by + j) * d + 4 * bx + i];
      bitwriter w = {out, ((uint64_t)by * nbx + bx) * 16u * (uint64_t)R};
      zfp_encode_block(v, R, &w);
    }
}

void oracle_zfp_decode_field(int64_t t0, int64_t nt, int d, int R,
                             const uint8_t *in, float *x) {
  int nbx = d / 4;
  for (int64_t by = t0 / 4; by < (t0 + nt) / 4; by++)
    for (int bx = 0; bx < nbx; bx++) {
      float v[16];
      bitreader r = {in, ((uint64_t)by * nbx + bx) * 16u * (uint64_t)R};
      zfp_decode_block(&r, R, v);
      for (int j = 0; j < 4; j++)
        for (int i = 0; i < 4; i++) x[(4 * by + j) * d + 4 * bx + i] = v[4 * j + i];
    }
}

/* ------------------------------------------------------------------------ */
/* Uniform min/max quantizer shared by the block-uniform and KIVI-style      */
/* backends (arXiv page, evaluation protocol: one range per group of values) */
/* ------------------------------------------------------------------------ */

/*
 * Quantize the n values vals[] with one range.  Range: mn, mx in fp32.
 * L = 2^bits - 1.  mx == mn (or L/(mx-mn) not finite in fp32) gives scale 0
 * and all codes 0; otherwise
 * scale = (mx-mn)/L and inv = L/(mx-mn) (fp32 divisions, the difference
 * itself rounded to fp32), q = clamp(rint((x-mn)*inv), 0, L) with ties to
 * even.  Codes are written to q[0..n-1]; meta = (mn, scale).
 */
static void quant_range(int n, const float *vals, int bits, uint32_t *q, float meta[2]) {
  float mn = vals[0], mx = vals[0];
  for (int i = 1; i < n; i++) {
    if (vals[i] < mn) mn = vals[i];
    if (vals[i] > mx) mx = vals[i];
  }
  int L = (1 << bits) - 1;
  float scale = 0.0f;
  float diff = mx - mn;
  float inv = diff > 0.0f ? (float)L / diff : 0.0f;
  if (mx == mn || !(inv <= 3.4028234663852886e38f)) {
    /* constant group, or a range so small that L/(mx-mn) overflows fp32:
       every code is 0 and the group decodes to mn */
    for (int i = 0; i < n; i++) q[i] = 0;
  } else {
    scale = diff / (float)L;
    for (int i = 0; i < n; i++) {
      float s = vals[i] - mn;
      float p = s * inv;
      float rq = rintf(p);          /* default rounding mode: ties to even */
      long iq = (long)rq;
      if (iq < 0) iq = 0;
      if (iq > L) iq = L;
      q[i] = (uint32_t)iq;
    }
  }
  meta[0] = mn;
  meta[1] = scale;
}

/* x_hat = mn + (float)q * scale, as a separate multiply then add */
static float dequant(uint32_t q, const float meta[2]) {
  float p = (float)q * meta[1];
  return meta[0] + p;
}

/* b-bit codes packed least-significant-bit first at bit offset `bitpos` */
static void pack_code(uint8_t *buf, uint64_t bitpos, uint32_t code, int bits) {
  bitwriter w = {buf, bitpos};
  put_bits(&w, code, bits);
}

static uint32_t unpack_code(const uint8_t *buf, uint64_t bitpos, int bits) {
  bitreader r = {buf, bitpos};
  return (uint32_t)get_bits(&r, bits);
}

/*
 * Block-uniform: one range per block of Bt tokens x d channels.  Field
 * x[T][d] (T a multiple of Bt).  Block m's codes are packed token-major
 * (value (t, c) of the block at index t*d + c) at payload bit offset
 * m*Bt*d*bits; meta[2m], meta[2m+1] = (mn, scale).  Token rows
 * [t0, t0+nt) (multiples of Bt) are encoded.
 */
void oracle_bu_encode_field(int64_t t0, int64_t nt, int d, int Bt, int bits,
                            const float *x, uint8_t *payload, float *meta) {
  int n = Bt * d;
  uint32_t *q = (uint32_t *)malloc((size_t)n * sizeof(uint32_t));
  for (int64_t m = t0 / Bt; m < (t0 + nt) / Bt; m++) {
    const float *blk = x + m * (int64_t)n;
    quant_range(n, blk, bits, q, meta + 2 * m);
    for (int v = 0; v < n; v++)
      pack_code(payload, ((uint64_t)m * n + v) * bits, q[v], bits);
  }
  free(q);
}

void oracle_bu_decode_field(int64_t t0, int64_t nt, int d, int Bt, int bits,
                            const uint8_t *payload, const float *meta, float *x) {
  int n = Bt * d;
  for (int64_t m = t0 / Bt; m < (t0 + nt) / Bt; m++)
    for (int v = 0; v < n; v++) {
      uint32_t q = unpack_code(payload, ((uint64_t)m * n + v) * bits, bits);
      x[m * (int64_t)n + v] = dequant(q, meta + 2 * m);
    }
}

/*
 * KIVI-style.  Tokens [0, Tq) are quantized, Tq = T - residual (a multiple
 * of `group`); the last `residual` tokens are returned to the caller to be
 * kept in the storage format.  Keys (kind 0): one range per channel per
 * `group` consecutive tokens; meta index ((t/group)*d + c).  Values (kind 1):
 * one range per token per `group` consecutive channels; meta index
 * (t*(d/group) + c/group).  Codes of value (t, c) sit at bit (t*d + c)*bits
 * of the payload.
 */
void oracle_kivi_encode_field(int64_t Tq, int d, int kind, int group, int bits,
                              const float *x, uint8_t *payload, float *meta) {
  float vals[1024];
  uint32_t q[1024];
  if (group > 1024) return;
  if (kind == 0) {
    for (int64_t tg = 0; tg < Tq / group; tg++)
      for (int c = 0; c < d; c++) {
        for (int k = 0; k < group; k++) vals[k] = x[(tg * group + k) * d + c];
        float *mt = meta + 2 * (tg * d + c);
        quant_range(group, vals, bits, q, mt);
        for (int k = 0; k < group; k++)
          pack_code(payload, ((uint64_t)(tg * group + k) * d + c) * bits, q[k], bits);
      }
  } else {
    int ng = d / group;
    for (int64_t t = 0; t < Tq; t++)
      for (int cg = 0; cg < ng; cg++) {
        for (int k = 0; k < group; k++) vals[k] = x[t * d + cg * group + k];
        float *mt = meta + 2 * (t * ng + cg);
        quant_range(group, vals, bits, q, mt);
        for (int k = 0; k < group; k++)
          pack_code(payload, ((uint64_t)t * d + cg * group + k) * bits, q[k], bits);
      }
  }
}

void oracle_kivi_decode_field(int64_t Tq, int d, int kind, int group, int bits,
                              const uint8_t *payload, const float *meta, float *x) {
  int ng = d / group;
  for (int64_t t = 0; t < Tq; t++)
    for (int c = 0; c < d; c++) {
      int64_t mi = kind == 0 ? (t / group) * d + c : t * ng + c / group;
      uint32_t q = unpack_code(payload, ((uint64_t)t * d + c) * bits, bits);
      x[t * d + c] = dequant(q, meta + 2 * mi);
    }
}

/* raw integer codes of a block-uniform / KIVI payload, for comparisons */
void oracle_unpack_codes(int64_t n, int bits, const uint8_t *payload, uint32_t *codes) {
  for (int64_t v = 0; v < n; v++) codes[v] = unpack_code(payload, (uint64_t)v * bits, bits);
}
