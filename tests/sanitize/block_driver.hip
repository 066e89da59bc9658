// Drives the HIP library's block coder (zfp_block.hpp, host build) over
// random, special-value and corrupted blocks at every rate, for a build under
// AddressSanitizer and UndefinedBehaviorSanitizer
// (tests/test_oracle_sanitize.py).  Test harness only.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../fixed_rate_compression_amd/csrc/zfp_block.hpp"

static uint64_t rs = 0x9E3779B97F4A7C15ull;
static uint32_t rnd() { rs ^= rs << 13; rs ^= rs >> 7; rs ^= rs << 17; return (uint32_t)rs; }
static float rndf() { return ((float)(rnd() & 0xFFFFFF) / 8388608.0f) - 1.0f; }

template <int R>
static void run(const cgz::PlaneTables &tab) {
  constexpr int NA = cgz::Rate<R>::kAcc;
  for (int it = 0; it < 2000; it++) {
    float v[16], w[16];
    for (int i = 0; i < 16; i++) {
      const uint32_t k = rnd() % 64;
      v[i] = k == 0 ? 0.0f : k == 1 ? -0.0f : k == 2 ? 1e-40f * rndf() : k == 3 ? 3e37f * rndf()
                                                                                  : 50.0f * rndf();
    }
    if (it % 7 == 0) for (int i = 0; i < 16; i++) v[i] = v[0];     // constant block
    uint64_t acc[NA];
    cgz::encode_block<R>(v, acc, tab);
    cgz::decode_block<R>(acc, w);
    for (int a = 0; a < NA; a++) acc[a] = ((uint64_t)rnd() << 32) | rnd();   // corrupted stream
    constexpr int top = 16 * R - 64 * (NA - 1);
    if (top < 64) acc[NA - 1] &= (1ull << top) - 1ull;               // bits past 16R are zero
    cgz::decode_block<R>(acc, w);
  }
}

int main() {
  // the encoder's lookup tables on the heap, exactly as large as they are
  cgz::PlaneTables *tab = (cgz::PlaneTables *)malloc(sizeof(cgz::PlaneTables));
  for (uint32_t i = 0; i < 256; i++) cgz::plane_tables_entry(*tab, i);
  run<1>(*tab); run<2>(*tab); run<3>(*tab); run<4>(*tab); run<5>(*tab); run<6>(*tab); run<7>(*tab);
  run<8>(*tab); run<12>(*tab); run<16>(*tab);
  free(tab);
  printf("block driver done\n");
  return 0;
}
