// zfp-style fixed-rate coding of one 4x4 token x channel block, in registers.
//
// The Codec-Gauge paper ("Codec-Gauge: Learning Compression-Friendly Gauges
// for Transformer KV Caches", arXiv HTML, evaluation-protocol paragraph)
// uses fixed-rate zfp (Lindstrom 2014) on the gauged FP32 field presented as
// a 2D array with n_x = d_l.  One block is 4 tokens x 4 channels and always
// occupies exactly 16*R bits:
//   bit 0            nonzero flag (0: all values are +-0, rest is zero)
//   bits 1..8        emax + 127, emax = largest frexp exponent, >= -126
//   bits 9..16R-1    embedded bit-plane code of the 16 transformed integers
// Steps: block-floating-point integers q = trunc(x * 2^(30-emax)); the
// 4-point integer lifting transform along channels, then along tokens;
// total-sequency reordering; negabinary; bit planes 31..0 coded with group
// tests until the 16R-9 bit budget is spent.
//
// GPU formulation (one block per lane, everything in VGPRs):
//  * the leading all-zero planes cost one 0 bit each, so they are skipped in
//    one step with a count-leading-zeros of the OR of the 16 words, and the
//    words are shifted so that the first nonzero plane sits at bit 31;
//  * all bit planes are produced at once by a 16x16 bit-matrix transpose
//    applied to both 16-bit halves of the 16 words (4 butterfly stages);
//  * a plane's verbatim part is one masked shift into the output, and its
//    group-test/scan part costs one step per coefficient that becomes
//    significant (each coefficient does so at most once per block);
//  * the block's bits live in ceil(16R/64) 64-bit accumulators; bits past
//    16R are dropped, which equals stopping at the budget because the code
//    of a block is a prefix code emitted strictly left to right.
// The functions are __host__ __device__ so the same code can be checked on
// the CPU; they use only portable integer operations.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cgz {

constexpr uint32_t kNegaMask = 0xAAAAAAAAu;

// total-sequency order: coefficient (i, j) stored at i + 4j, visited by
// i + j, then i^2 + j^2, then larger i first
__host__ __device__ constexpr int seq_index(int k) {
  constexpr int order[16] = {0, 1, 4, 5, 2, 8, 6, 9, 3, 12, 10, 7, 13, 11, 14, 15};
  return order[k];
}

template <int R>
struct Rate {
  static constexpr int kBits = 16 * R;
  static constexpr int kAcc = (kBits + 63) / 64;   // 64-bit accumulators
};

__host__ __device__ __forceinline__ int32_t shr1(uint32_t s) { return ((int32_t)s) >> 1; }

// forward 4-point lifting transform (integer realization of
// F = 1/16 [[4,4,4,4],[5,1,-1,-5],[-4,4,4,-4],[-2,6,-6,2]])
__host__ __device__ __forceinline__ void fwd_xform4(int32_t &a, int32_t &b, int32_t &c,
                                                    int32_t &d) {
  a = shr1((uint32_t)a + (uint32_t)d);
  d = (int32_t)((uint32_t)d - (uint32_t)a);
  c = shr1((uint32_t)b + (uint32_t)c);
  b = (int32_t)((uint32_t)b - (uint32_t)c);
  a = shr1((uint32_t)a + (uint32_t)c);
  c = (int32_t)((uint32_t)c - (uint32_t)a);
  d = shr1((uint32_t)d + (uint32_t)b);
  b = (int32_t)((uint32_t)b - (uint32_t)d);
  d = (int32_t)((uint32_t)d + (uint32_t)(b >> 1));
  b = (int32_t)((uint32_t)b - (uint32_t)(d >> 1));
}

// exact inverse of every lifting step, in reverse order (mod 2^32)
__host__ __device__ __forceinline__ void inv_xform4(int32_t &a, int32_t &b, int32_t &c,
                                                    int32_t &d) {
  b = (int32_t)((uint32_t)b + (uint32_t)(d >> 1));
  d = (int32_t)((uint32_t)d - (uint32_t)(b >> 1));
  b = (int32_t)((uint32_t)b + (uint32_t)d);
  d = (int32_t)(((uint32_t)d << 1) - (uint32_t)b);
  c = (int32_t)((uint32_t)c + (uint32_t)a);
  a = (int32_t)(((uint32_t)a << 1) - (uint32_t)c);
  b = (int32_t)((uint32_t)b + (uint32_t)c);
  c = (int32_t)(((uint32_t)c << 1) - (uint32_t)b);
  d = (int32_t)((uint32_t)d + (uint32_t)a);
  a = (int32_t)(((uint32_t)a << 1) - (uint32_t)d);
}

// Transpose the two 16x16 bit matrices held in the low and high halves of
// w[0..15] (row i = word i, column c = bit c of the half).  Afterwards the low
// half of w[k] is the word whose bit i was bit k of the old w[i], and the high
// half likewise for bit 16 + k.  The transform is an involution.
__host__ __device__ __forceinline__ void swap_stage(uint32_t &a, uint32_t &b, int s, uint32_t m) {
  // exchange the columns selected by (m << s) of row a with the columns m of row b
  const uint32_t na = (a & ~(m << s)) | ((b << s) & (m << s));
  const uint32_t nb = (b & ~m) | ((a >> s) & m);
  a = na;
  b = nb;
}

// the 8-bit stage of swap_stage: a' = (a0, b0, a2, b2), b' = (a1, b1, a3, b3)
// (bytes from least significant); one byte permute per output on the GPU
__host__ __device__ __forceinline__ void swap_bytes(uint32_t &a, uint32_t &b) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint32_t na = __builtin_amdgcn_perm(a, b, 0x02060004u);
  const uint32_t nb = __builtin_amdgcn_perm(a, b, 0x03070105u);
#else
  const uint32_t na = (a & 0x00FF00FFu) | ((b << 8) & 0xFF00FF00u);
  const uint32_t nb = ((a >> 8) & 0x00FF00FFu) | (b & 0xFF00FF00u);
#endif
  a = na;
  b = nb;
}

__host__ __device__ __forceinline__ void transpose16x2(uint32_t (&w)[16]) {
#pragma unroll
  for (int i = 0; i < 8; i++) swap_bytes(w[i], w[i + 8]);
#pragma unroll
  for (int i = 0; i < 16; i++)
    if (!(i & 4)) swap_stage(w[i], w[i + 4], 4, 0x0F0F0F0Fu);
#pragma unroll
  for (int i = 0; i < 16; i++)
    if (!(i & 2)) swap_stage(w[i], w[i + 2], 2, 0x33333333u);
#pragma unroll
  for (int i = 0; i < 16; i += 2) swap_stage(w[i], w[i + 1], 1, 0x55555555u);
}

__host__ __device__ __forceinline__ int ctz32(uint32_t x) {  // x != 0
  return __builtin_ctz(x);
}

__host__ __device__ __forceinline__ int clz32(uint32_t x) {  // x != 0
  return __builtin_clz(x);
}

// number of significant bits of x (0 for x = 0)
__host__ __device__ __forceinline__ int bitlen32(uint32_t x) {
#if defined(__HIP_DEVICE_COMPILE__)
  return 32 - __clz((int)x);  // __clz(0) = 32
#else
  return x ? 32 - __builtin_clz(x) : 0;
#endif
}

// Append `len` (<= 32) bits of `code` at bit `pos`; bits at or past 16R are
// dropped.
template <int R>
__host__ __device__ __forceinline__ void put(uint64_t (&acc)[Rate<R>::kAcc], int pos,
                                             uint32_t code) {
  constexpr int NA = Rate<R>::kAcc;
  if (pos >= Rate<R>::kBits) return;
#pragma unroll
  for (int a = 0; a < NA; a++) {
    int sh = pos - 64 * a;
    if (sh >= 0 && sh < 64)
      acc[a] |= (uint64_t)code << sh;
    else if (sh < 0 && sh > -32)
      acc[a] |= (uint64_t)code >> (-sh);
  }
}

// OR a 64-bit code into the block's bits at `pos` (bits at or past 16R are
// dropped by the final mask).
template <int R>
__host__ __device__ __forceinline__ void put64(uint64_t (&acc)[Rate<R>::kAcc], int pos,
                                               uint64_t code) {
  constexpr int NA = Rate<R>::kAcc;
  // pos is in [0, 16R): the first word never needs a right shift
  if (pos < 64) acc[0] |= code << pos;
#pragma unroll
  for (int a = 1; a < NA; a++) {
    const int sh = pos - 64 * a;
    if (sh >= 0 && sh < 64)
      acc[a] |= code << sh;
    else if (sh < 0 && sh > -64)
      acc[a] |= code >> (-sh);
  }
}

// 8-bit expansion table entry: every 1 followed by an inserted 1, LSB first
__host__ __device__ constexpr uint16_t dbl8_entry(uint32_t s) {
  uint32_t out = 0;
  int p = 0;
  for (int i = 0; i < 8; i++) {
    if ((s >> i) & 1u) {
      out |= 3u << p;
      p += 2;
    } else {
      p += 1;
    }
  }
  return (uint16_t)out;
}

// 32 stream bits starting at `pos` (< 16R); bits past 16R read as 0
template <int R>
__host__ __device__ __forceinline__ uint32_t window(const uint64_t (&acc)[Rate<R>::kAcc],
                                                    int pos) {
  constexpr int NA = Rate<R>::kAcc;
  if (NA == 1) return (uint32_t)(acc[0] >> pos);
  uint32_t r = 0;
#pragma unroll
  for (int a = 0; a < NA; a++) {
    int sh = pos - 64 * a;
    if (sh >= 0 && sh < 64)
      r |= (uint32_t)(acc[a] >> sh);
    else if (sh < 0 && sh > -32)
      r |= (uint32_t)(acc[a] << (-sh));
  }
  return r;
}

// Encode 16 fp32 values v[4j + i] (j = token row, i = channel) at rate R.
template <int R>
__host__ __device__ __forceinline__ void encode_block(const float (&v)[16],
                                                      uint64_t (&acc)[Rate<R>::kAcc],
                                                      const uint16_t *__restrict__ dbl) {
  constexpr int NA = Rate<R>::kAcc;
  constexpr int LIMIT = Rate<R>::kBits;
#pragma unroll
  for (int a = 0; a < NA; a++) acc[a] = 0;

  // block exponent from the largest magnitude (bit patterns of |x| order like
  // the values): frexp exponent = biased exponent - 126, clamped at -126
  float fm = 0.0f;
#pragma unroll
  for (int k = 0; k < 16; k++) fm = fmaxf(fm, fabsf(v[k]));
  const uint32_t mx = __builtin_bit_cast(uint32_t, fm);
  if (mx == 0) return;
  int ebiased = (int)(mx >> 23);
  int emax = ebiased ? ebiased - 126 : -126;

  int32_t q[16];
#pragma unroll
  for (int k = 0; k < 16; k++) q[k] = (int32_t)ldexpf(v[k], 30 - emax);
#pragma unroll
  for (int j = 0; j < 4; j++) fwd_xform4(q[4 * j], q[4 * j + 1], q[4 * j + 2], q[4 * j + 3]);
#pragma unroll
  for (int i = 0; i < 4; i++) fwd_xform4(q[i], q[4 + i], q[8 + i], q[12 + i]);

  uint32_t u[16];
  uint32_t any = 0;
#pragma unroll
  for (int k = 0; k < 16; k++) {
    u[k] = ((uint32_t)q[seq_index(k)] + kNegaMask) ^ kNegaMask;
    any |= u[k];
  }
  acc[0] = 1u | ((uint64_t)(uint32_t)(emax + 127) << 1);
  if (any == 0) return;
  const int s = clz32(any);            // planes 31..32-s are all zero
  int pos = 9 + s;                      // one failed group test per zero plane
#pragma unroll
  for (int k = 0; k < 16; k++) u[k] <<= s;
  transpose16x2(u);                     // u[m]: plane m (low), plane m+16 (high)

  // Planes from the top, one fixed-cost step each.  For plane word w with n
  // coefficients already significant the code is: the n verbatim bits, then
  // (if n < 16) either a failed group test (0) or a 1 followed by the bits
  // w[n..min(hb,14)] with every 1 among them followed by one more bit -- 1 if
  // another one follows in the plane, 0 after the last one (hb = highest set
  // bit; a one at position 15 is implied and not sent).  The "1 after every
  // 1" expansion comes from the 256-entry table `dbl`.
  int n = 0;                            // coefficients already significant
#pragma unroll
  for (int j = 0; j < 32; j++) {        // plane 31-j of the shifted words
    if (pos < LIMIT) {                  // (no early exit: keeps the loop unrollable)
      const uint32_t w = j < 16 ? (u[15 - j] >> 16) : (u[31 - j] & 0xFFFFu);
      const uint32_t rest = w >> n;
      const int hb1 = 32 - clz32(w | 1u);   // highest set bit + 1 (1 when w <= 1)
      // scanned positions n .. min(hb, 14); when rest == 0 the code below is
      // replaced by the failed test
      const int L = max(min(hb1, 15), n) - n;
      const uint32_t S = rest & ((1u << L) - 1u);
      const uint32_t lo = S & 0xFFu, hi = S >> 8;
      const int pclo = __builtin_popcount(lo), pc = pclo + __builtin_popcount(hi);
      const uint32_t D = (uint32_t)dbl[lo] | ((uint32_t)dbl[hi] << (8 + pclo));
      uint32_t code = 1u | (D << 1);
      if (hb1 <= 15) code &= ~(1u << (L + pc));
      int len = 1 + L + pc;
      if (rest == 0) {
        code = 0u;
        len = n < 16 ? 1 : 0;
      }
      const uint64_t full = (uint64_t)(w & ((1u << n) - 1u)) | ((uint64_t)code << n);
      put64<R>(acc, pos, full);
      pos += n + len;
      n = rest ? hb1 : n;
    }
  }
  if (LIMIT % 64) acc[NA - 1] &= (~0ull) >> (64 - LIMIT % 64);
}

// Group-test/scan part of one bit plane, read bit-parallel.  On entry `pos`
// is at the plane's first group test and `n` (< 16) coefficients are
// significant.  The code there is a run of pairs "1 0^gap 1" (a positive
// group test, zeros scanned over, the newly significant coefficient's 1) and
// ends with a 0 (failed test), or with the budget, or with the implicit 1 of
// coefficient 15 (a scan reaching index 15 reads no bit).  With P the
// inclusive prefix parity of the window, a 1 at odd parity is a test, a 1 at
// even parity ends a scan and a 0 at even parity is the failed test; the k-th
// scan-ending 1 (k from 0) at window bit t is coefficient n + t - (k + 1).
// Returns the new coefficients' bits relative to n; advances pos and n.
template <int R>
__host__ __device__ __forceinline__ uint32_t group_part(const uint64_t (&acc)[Rate<R>::kAcc],
                                                        int &pos, int &n) {
  constexpr int LIMIT = Rate<R>::kBits;
  const uint32_t W = window<R>(acc, pos);
  uint32_t P = W;
  P ^= P << 1;
  P ^= P << 2;
  P ^= P << 4;
  P ^= P << 8;
  P ^= P << 16;
  const uint32_t tests = W & P;
  const uint32_t fails = ~(W | P);
  const uint32_t ef = fails ? (uint32_t)ctz32(fails) : 32u;  // first failed test
  const uint32_t room = (uint32_t)(LIMIT - pos);              // >= 1
  const uint32_t m = 15u - (uint32_t)n;                       // index of coefficient 15
  // a plane's group part never spans more than 2m+1 bits
  uint32_t E = ef < room ? ef : room;
  E = E < 2u * m + 2u ? E : 2u * m + 2u;                      // <= 32
  const uint32_t below = (uint32_t)~(~0ull << E);            // E <= 32
  uint32_t term = W & ~P & below;
  uint32_t y = 0u, bias = 1u;
  while (term) {                        // two newly significant coefficients per step
    const uint32_t low1 = term & (0u - term);
    const uint32_t rest = term ^ low1;
    const uint32_t low2 = rest & (0u - rest);   // 0 when only one was left
    y |= (low1 >> bias) | (low2 >> (bias + 1u));
    term = rest ^ low2;
    bias += 2u;
  }
  const uint32_t cnt = (uint32_t)__builtin_popcount(below & ~tests);     // bits scanned before E
  // three ways the part ends, selected without branches (lanes diverge here):
  //  cap    the scan reaches coefficient 15, whose 1 is implicit;
  //  fail   a failed group test at ef;
  //  budget the budget ends at room (<= ef <= 32); inside a scan the scanned
  //         index is set
  const bool cap = cnt > m;
  const bool fail = ef < room;
  const uint32_t ycap = (y & ((1u << m) - 1u)) | (1u << m);
  const uint32_t inscan = (P >> ((room - 1u) & 31u)) & 1u;
  const uint32_t ybud = y | (inscan << (cnt & 31u));
  y = cap ? ycap : (fail ? y : ybud);
  const uint32_t used = cap ? m + (uint32_t)__builtin_popcount(ycap) : (fail ? ef + 1u : room);
  pos += (int)used;
  n += bitlen32(y);                     // every index up to the last new one is now verbatim
  return y;
}

// Decode one block of 16R bits into 16 fp32 values v[4j + i].
template <int R>
__host__ __device__ __forceinline__ void decode_block(const uint64_t (&acc)[Rate<R>::kAcc],
                                                      float (&v)[16]) {
  constexpr int LIMIT = Rate<R>::kBits;
#pragma unroll
  for (int k = 0; k < 16; k++) v[k] = 0.0f;
  if (!(acc[0] & 1u)) return;
  const int emax = (int)((acc[0] >> 1) & 0xFFu) - 127;

  int pos = 9;
  uint32_t win = window<R>(acc, pos);
  const int s = win ? ctz32(win) : 32;  // leading failed group tests
  if (s >= 32 || pos + s >= LIMIT) return;  // no plane reached: all integers 0
  pos += s;

  uint32_t w[16];
#pragma unroll
  for (int k = 0; k < 16; k++) w[k] = 0;
  int n = 0;
#pragma unroll
  for (int j = 0; j < 32; j++) {
    uint32_t x = 0u;                    // plane word 31-j of the shifted words
    // planes past the last one (j > 31 - s) lie below bit s of the shifted
    // words, which the final shift drops; the encoder codes them as zeros
    if (pos < LIMIT) {                  // (no early exit: keeps the loop unrollable)
      x = window<R>(acc, pos) & ((1u << n) - 1u);   // verbatim bits (n <= 16)
      pos += n;
      const int n0 = n;
      if (n < 16 && pos < LIMIT) x |= group_part<R>(acc, pos, n) << n0;
    }
    if (j < 16)
      w[15 - j] |= x << 16;
    else
      w[31 - j] |= x;
  }
  transpose16x2(w);

  int32_t q[16];
#pragma unroll
  for (int k = 0; k < 16; k++)
    q[seq_index(k)] = (int32_t)(((w[k] >> s) ^ kNegaMask) - kNegaMask);
#pragma unroll
  for (int i = 0; i < 4; i++) inv_xform4(q[i], q[4 + i], q[8 + i], q[12 + i]);
#pragma unroll
  for (int j = 0; j < 4; j++) inv_xform4(q[4 * j], q[4 * j + 1], q[4 * j + 2], q[4 * j + 3]);
#pragma unroll
  for (int k = 0; k < 16; k++) v[k] = ldexpf((float)q[k], emax - 30);
}

}  // namespace cgz
