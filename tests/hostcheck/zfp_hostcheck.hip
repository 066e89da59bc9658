// Host-only build of the HIP library's block codec (zfp_block.hpp), used by
// the CPU tests to compare the exact code the kernels run against the oracle
// without a GPU.  Test harness only: nothing on the product path loads it.
#include <string.h>

#include "../../fixed_rate_compression_amd/csrc/zfp_block.hpp"

static uint16_t g_dbl[256];
static bool g_dbl_ready = false;

template <int R>
static void enc(const float *v, unsigned char *out) {
  if (!g_dbl_ready) {
    for (int i = 0; i < 256; i++) g_dbl[i] = cgz::dbl8_entry((uint32_t)i);
    g_dbl_ready = true;
  }
  float b[16];
  memcpy(b, v, sizeof b);
  uint64_t acc[cgz::Rate<R>::kAcc];
  cgz::encode_block<R>(b, acc, g_dbl);
  for (int i = 0; i < 2 * R; i++) out[i] = (unsigned char)(acc[i / 8] >> (8 * (i % 8)));
}

template <int R>
static void dec(const unsigned char *in, float *v) {
  uint64_t acc[cgz::Rate<R>::kAcc];
  for (int a = 0; a < cgz::Rate<R>::kAcc; a++) acc[a] = 0;
  for (int i = 0; i < 2 * R; i++) acc[i / 8] |= (uint64_t)in[i] << (8 * (i % 8));
  float b[16];
  cgz::decode_block<R>(acc, b);
  memcpy(v, b, sizeof b);
}

#define RATES(X) X(1) X(2) X(3) X(4) X(5) X(6) X(7) X(8) X(12) X(16)

extern "C" int hc_encode_block(const float *v, int R, unsigned char *out) {
  switch (R) {
#define C(r) case r: enc<r>(v, out); return 0;
    RATES(C)
#undef C
  }
  return -1;
}

extern "C" int hc_decode_block(const unsigned char *in, int R, float *v) {
  switch (R) {
#define C(r) case r: dec<r>(in, v); return 0;
    RATES(C)
#undef C
  }
  return -1;
}
