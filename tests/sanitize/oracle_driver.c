/* Drives every C function of the oracle over random, special-value and
 * corrupted inputs with exactly sized heap buffers, for a build under
 * AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_oracle_sanitize.py).
 * Test harness only. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

float oracle_bf16_to_f32(uint16_t h);
uint16_t oracle_f32_to_bf16(float f);
void oracle_bf16_to_f32_array(int64_t n, const uint16_t *in, float *out);
void oracle_f32_to_bf16_array(int64_t n, const float *in, uint16_t *out);
void oracle_gauge_forward(int64_t T, int d, int g, const float *G, const float *x, float *y);
void oracle_gauge_inverse(int64_t T, int d, int g, const float *G, const float *y, float *x);
void oracle_sequency_order(int32_t out[16]);
void oracle_fwd_lift4(int32_t v[4]);
void oracle_inv_lift4(int32_t v[4]);
int oracle_zfp_block_words(const float v[16], uint32_t u[16], int32_t *emax);
int oracle_zfp_decode_block_words(const uint8_t *in, int R, uint32_t u[16], int32_t *emax);
void oracle_zfp_encode_block(const float v[16], int R, uint8_t *out);
void oracle_zfp_decode_block(const uint8_t *in, int R, float v[16]);
void oracle_zfp_encode_field(int64_t t0, int64_t nt, int d, int R, const float *x, uint8_t *out);
void oracle_zfp_decode_field(int64_t t0, int64_t nt, int d, int R, const uint8_t *in, float *x);
void oracle_bu_encode_field(int64_t t0, int64_t nt, int d, int Bt, int bits, const float *x,
                            uint8_t *payload, float *meta);
void oracle_bu_decode_field(int64_t t0, int64_t nt, int d, int Bt, int bits, const uint8_t *payload,
                            const float *meta, float *x);
void oracle_kivi_encode_field(int64_t Tq, int d, int kind, int group, int bits, const float *x,
                              uint8_t *payload, float *meta);
void oracle_kivi_decode_field(int64_t Tq, int d, int kind, int group, int bits,
                              const uint8_t *payload, const float *meta, float *x);
void oracle_unpack_codes(int64_t n, int bits, const uint8_t *payload, uint32_t *codes);

static uint64_t rs = 88172645463325252ull;
static uint32_t rnd(void) { rs ^= rs << 13; rs ^= rs >> 7; rs ^= rs << 17; return (uint32_t)rs; }
static float rndf(void) { return ((float)(rnd() & 0xFFFFFF) / 8388608.0f) - 1.0f; }

/* random field: mostly normal values, some zeros, -0, subnormals, large values */
static float *field(int64_t n) {
  float *x = (float *)malloc((size_t)n * sizeof(float));
  for (int64_t i = 0; i < n; i++) {
    uint32_t k = rnd() % 64;
    x[i] = k == 0 ? 0.0f : k == 1 ? -0.0f : k == 2 ? 1e-40f * rndf() : k == 3 ? 3e37f * rndf()
                                                                                : 50.0f * rndf();
  }
  return x;
}

int main(void) {
  const int d = 128;
  /* bf16 conversions */
  {
    int64_t n = 1000;
    float *x = field(n);
    uint16_t *h = (uint16_t *)malloc(n * sizeof(uint16_t));
    float *y = (float *)malloc(n * sizeof(float));
    oracle_f32_to_bf16_array(n, x, h);
    oracle_bf16_to_f32_array(n, h, y);
    for (int64_t i = 0; i < n; i++) (void)oracle_bf16_to_f32(oracle_f32_to_bf16(x[i]));
    free(x); free(h); free(y);
  }
  /* gauge */
  {
    const int gs[4] = {8, 16, 32, 128};
    for (int gi = 0; gi < 4; gi++) {
      int g = gs[gi];
      int64_t T = 37;
      float *G = (float *)malloc((size_t)(d / g) * g * g * sizeof(float));
      for (int i = 0; i < (d / g) * g * g; i++) G[i] = rndf();
      float *x = field(T * d), *y = (float *)malloc(T * d * sizeof(float));
      float *z = (float *)malloc(T * d * sizeof(float));
      oracle_gauge_forward(T, d, g, G, x, y);
      oracle_gauge_inverse(T, d, g, G, y, z);
      oracle_gauge_forward(T, d, 0, G, x, y);
      free(G); free(x); free(y); free(z);
    }
  }
  /* block primitives */
  {
    int32_t ord[16], v[4] = {(int32_t)rnd() >> 2, -(int32_t)(rnd() >> 3), 7, -1};
    oracle_sequency_order(ord);
    oracle_fwd_lift4(v);
    oracle_inv_lift4(v);
  }
  /* zfp blocks and fields, including corrupted streams */
  {
    const int Rs[8] = {1, 2, 3, 4, 6, 8, 16, 32};
    for (int ri = 0; ri < 8; ri++) {
      int R = Rs[ri];
      for (int it = 0; it < 200; it++) {
        float *v = field(16), w[16];
        uint32_t u[16];
        int32_t e;
        uint8_t *code = (uint8_t *)malloc(2 * (size_t)R);
        memset(code, 0, 2 * (size_t)R);
        (void)oracle_zfp_block_words(v, u, &e);
        oracle_zfp_encode_block(v, R, code);
        oracle_zfp_decode_block(code, R, w);
        (void)oracle_zfp_decode_block_words(code, R, u, &e);
        for (int b = 0; b < 2 * R; b++) code[b] = (uint8_t)rnd();   /* corrupted stream */
        oracle_zfp_decode_block(code, R, w);
        free(v); free(code);
      }
      int64_t T = 36;
      size_t nbytes = (size_t)T * d * R / 8;
      float *x = field(T * d), *y = (float *)malloc(T * d * sizeof(float));
      uint8_t *pay = (uint8_t *)calloc(nbytes, 1);
      oracle_zfp_encode_field(0, T, d, R, x, pay);
      oracle_zfp_encode_field(8, 12, d, R, x, pay);            /* an append */
      oracle_zfp_decode_field(0, T, d, R, pay, y);
      for (size_t b = 0; b < nbytes; b++) pay[b] = (uint8_t)rnd();
      oracle_zfp_decode_field(4, 16, d, R, pay, y);
      free(x); free(y); free(pay);
    }
  }
  /* block-uniform and KIVI-style quantizers */
  for (int bits = 1; bits <= 8; bits++) {
    const int Bts[3] = {16, 32, 64};
    for (int bi = 0; bi < 3; bi++) {
      int Bt = Bts[bi];
      int64_t T = 128;
      size_t nbytes = (size_t)T * d * bits / 8;
      float *x = field(T * d), *y = (float *)malloc(T * d * sizeof(float));
      uint8_t *pay = (uint8_t *)calloc(nbytes, 1);
      float *meta = (float *)malloc((size_t)(T / Bt) * 2 * sizeof(float));
      oracle_bu_encode_field(0, T, d, Bt, bits, x, pay, meta);
      oracle_bu_decode_field(0, T, d, Bt, bits, pay, meta, y);
      uint32_t *codes = (uint32_t *)malloc((size_t)T * d * sizeof(uint32_t));
      oracle_unpack_codes(T * d, bits, pay, codes);
      free(x); free(y); free(pay); free(meta); free(codes);
    }
    for (int kind = 0; kind < 2; kind++) {
      int64_t Tq = 96;
      int group = 32;
      size_t nbytes = (size_t)Tq * d * bits / 8;
      size_t nmeta = kind == 0 ? (size_t)(Tq / group) * d : (size_t)Tq * (d / group);
      float *x = field(Tq * d), *y = (float *)malloc(Tq * d * sizeof(float));
      uint8_t *pay = (uint8_t *)calloc(nbytes, 1);
      float *meta = (float *)malloc(nmeta * 2 * sizeof(float));
      oracle_kivi_encode_field(Tq, d, kind, group, bits, x, pay, meta);
      oracle_kivi_decode_field(Tq, d, kind, group, bits, pay, meta, y);
      free(x); free(y); free(pay); free(meta);
    }
  }
  printf("oracle driver done\n");
  return 0;
}
