// Host-only build of the HIP library's block codec (zfp_block.hpp), used by
// the CPU tests to compare the exact code the kernels run against the oracle
// without a GPU.  Test harness only: nothing on the product path loads it.
#include <string.h>

#include "../../fixed_rate_compression_amd/csrc/zfp_block.hpp"

static cgz::PlaneTables g_tab;
static bool g_tab_ready = false;

template <int R, bool GENERAL>
static void enc(const float *v, unsigned char *out) {
  if (!g_tab_ready) {
    for (uint32_t i = 0; i < 256; i++) cgz::plane_tables_entry(g_tab, i);
    g_tab_ready = true;
  }
  float b[16];
  memcpy(b, v, sizeof b);
  uint64_t acc[cgz::Rate<R>::kAcc];
  cgz::encode_block<R, GENERAL>(b, acc, g_tab);
  for (int i = 0; i < 2 * R; i++) out[i] = (unsigned char)(acc[i / 8] >> (8 * (i % 8)));
}

template <int R, bool GENERAL>
static void dec(const unsigned char *in, float *v) {
  uint64_t acc[cgz::Rate<R>::kAcc];
  for (int a = 0; a < cgz::Rate<R>::kAcc; a++) acc[a] = 0;
  for (int i = 0; i < 2 * R; i++) acc[i / 8] |= (uint64_t)in[i] << (8 * (i % 8));
  float b[16];
  cgz::decode_block<R, GENERAL>(acc, b);
  memcpy(v, b, sizeof b);
}

#define RATES(X) X(1) X(2) X(3) X(4) X(5) X(6) X(7) X(8) X(12) X(16)

// the encoder as the kernels run it (planes 0..7 from the 8x8 transposes
// whenever they apply to the block), and with the 16x16 transposes forced
extern "C" int hc_encode_block(const float *v, int R, unsigned char *out) {
  switch (R) {
#define C(r) case r: enc<r, false>(v, out); return 0;
    RATES(C)
#undef C
  }
  return -1;
}

extern "C" int hc_encode_block_general(const float *v, int R, unsigned char *out) {
  switch (R) {
#define C(r) case r: enc<r, true>(v, out); return 0;
    RATES(C)
#undef C
  }
  return -1;
}

// the decoder as the kernels run it (8-plane reconstruction whenever it
// applies to the block), and with the 32-plane reconstruction forced
extern "C" int hc_decode_block(const unsigned char *in, int R, float *v) {
  switch (R) {
#define C(r) case r: dec<r, false>(in, v); return 0;
    RATES(C)
#undef C
  }
  return -1;
}

extern "C" int hc_decode_block_general(const unsigned char *in, int R, float *v) {
  switch (R) {
#define C(r) case r: dec<r, true>(in, v); return 0;
    RATES(C)
#undef C
  }
  return -1;
}

// n consecutive blocks v[16 b + 4 j + i] into 2R bytes each (GENERAL != 0:
// the 16x16 transposes forced)
extern "C" int hc_encode_blocks(const float *v, long n, int R, int general, unsigned char *out) {
  for (long b = 0; b < n; b++) {
    const float *p = v + 16 * b;
    unsigned char *o = out + b * 2 * R;
    int rc = general ? hc_encode_block_general(p, R, o) : hc_encode_block(p, R, o);
    if (rc) return rc;
  }
  return 0;
}

// n consecutive blocks of 2R bytes each into v[16 b + 4 j + i] (GENERAL != 0:
// the 32-plane reconstruction forced)
extern "C" int hc_decode_blocks(const unsigned char *in, long n, int R, int general, float *v) {
  for (long b = 0; b < n; b++) {
    const unsigned char *p = in + b * 2 * R;
    float *o = v + 16 * b;
    int rc = general ? hc_decode_block_general(p, R, o) : hc_decode_block(p, R, o);
    if (rc) return rc;
  }
  return 0;
}

template <int R>
static int dec_lifted(const unsigned char *in, float *v) {
  uint64_t acc[cgz::Rate<R>::kAcc];
  for (int a = 0; a < cgz::Rate<R>::kAcc; a++) acc[a] = 0;
  for (int i = 0; i < 2 * R; i++) acc[i / 8] |= (uint64_t)in[i] << (8 * (i % 8));
  float b[16];
  const bool applied = cgz::decode_block_lifted<R>(acc, b);
  memcpy(v, b, sizeof b);
  return applied ? 1 : 0;
}

// the lifted (matrix-core) reconstruction's arithmetic on the CPU: 1 where it
// applies to the block (v written), 0 where the kernels take another path
extern "C" int hc_decode_block_lifted(const unsigned char *in, int R, float *v) {
  switch (R) {
#define C(r) case r: return dec_lifted<r>(in, v);
    RATES(C)
#undef C
  }
  return -1;
}

// the integer matrix of the lifted reconstruction, A[p][k] (row p = output
// position 4j + i, column k = sequency index)
extern "C" void hc_lift_matrix(int *a) {
  for (int p = 0; p < 16; p++)
    for (int k = 0; k < 16; k++) a[16 * p + k] = cgz::kLift.a[p][k];
}
