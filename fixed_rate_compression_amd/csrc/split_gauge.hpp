// Inverse gauge for groups of g = 16 and 32 channels with bf16 storage, on
// the bf16 matrix cores in split precision.
//
// "Codec-Gauge" (arXiv HTML, gauge parameterization and evaluation-protocol
// paragraphs): decoding applies G^T per group, y_c = sum_k G[k][c] x_k.
// With bf16 storage the result is rounded to bf16, so the product only has
// to be accurate far below bf16's 2^-9: every decoded value x is split into
// bf16 parts x = x_hi + x_lo (x_hi its top 8 significand bits, x_lo the
// remainder rounded to 8 bits: exact for the decoder's 16-bit values, error
// <= 2^-16 |x| otherwise), and G = G_hi + G_lo the same way (error <=
// 2^-17 |G|), and the products x_hi G_hi + x_hi G_lo + x_lo G_hi (+ x_lo
// G_lo at g = 16, where it is free) are summed on v_mfma_f32_16x16x32_bf16
// in fp32.  The bf16 matrix instructions run alongside the VALU work of
// other waves (the fp32 16x16x4 form does not), and take 2 (g = 16) or 3
// (g = 32) instructions per 16 x 16 output block instead of g / 4 fp32 ones.
//
// Tile layout: the fp32 tile (PITCH floats per row) is reused.  The 128 B of
// row r that hold channels [32w, 32w + 32) as fp32 first hold those 32
// values as bf16 hi parts (bytes 0..63) and lo parts (64..127), written by
// the decoder; wave w reads them as A operands and overwrites the same bytes
// with its fp32 results, so no other wave is involved and no barrier is
// needed between the two.
// Operand layout of 16x16x32: lane l holds A[m = l % 16][k = 8 (l / 16) ..
// + 7], B[k = 8 (l / 16) .. + 7][n = l % 16]; D[m][n] sits in lane
// n + 16 (m / 4), element m % 4.
//   g = 16 (output block nb = one group, inputs i = 0..15):
//     k = [hi of inputs 0..15 | lo of inputs 0..15]
//     D  = A B1 + A B2,  B1 = [G_hi; G_hi], B2 = [G_lo; G_lo]
//   g = 32 (the wave's 32 channels are one group, inputs k = 0..31):
//     D = A_hi B_hi + A_hi B_lo + A_lo B_hi   (B for output block nb)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cg_tile.hpp"

namespace cgk {

typedef __attribute__((ext_vector_type(8))) __bf16 sg_bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float sg_f32x4_t;
typedef __attribute__((ext_vector_type(4))) unsigned int sg_u32x4_t;

// top 16 bits of a and b (truncated bf16), packed a | b << 16
__device__ __forceinline__ uint32_t sg_hi2(float a, float b) {
  return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
}

// the remainders below those parts, rounded to bf16, packed
__device__ __forceinline__ uint32_t sg_lo2(float a, float b) {
  return pack_bf16x2(a - __uint_as_float(__float_as_uint(a) & 0xFFFF0000u),
                     b - __uint_as_float(__float_as_uint(b) & 0xFFFF0000u));
}

// the 4 values of one row of a decoded 4x4 block (channels c .. c + 3,
// c % 4 == 0) into the split layout of row `row`
__device__ __forceinline__ void split_store4(unsigned char *tile, int row, int c, float a, float b,
                                             float d, float e) {
  unsigned char *p = tile + (size_t)row * PITCH * 4 + (c >> 5) * 128 + (c & 31) * 2;
  *(uint2 *)p = make_uint2(sg_hi2(a, b), sg_hi2(d, e));
  *(uint2 *)(p + 64) = make_uint2(sg_lo2(a, b), sg_lo2(d, e));
}

// the 32 values of row `row`, channels 32 w .. 32 w + 31, into the split
// layout of that row's chunk w
__device__ __forceinline__ void split_store32(unsigned char *tile, int row, int w, const float (&v)[32]) {
  unsigned char *p = tile + (size_t)row * PITCH * 4 + w * 128;
#pragma unroll
  for (int q = 0; q < 4; q++) {
    *(uint4 *)(p + 16 * q) = make_uint4(sg_hi2(v[8 * q], v[8 * q + 1]), sg_hi2(v[8 * q + 2], v[8 * q + 3]),
                                        sg_hi2(v[8 * q + 4], v[8 * q + 5]), sg_hi2(v[8 * q + 6], v[8 * q + 7]));
    *(uint4 *)(p + 64 + 16 * q) =
        make_uint4(sg_lo2(v[8 * q], v[8 * q + 1]), sg_lo2(v[8 * q + 2], v[8 * q + 3]),
                   sg_lo2(v[8 * q + 4], v[8 * q + 5]), sg_lo2(v[8 * q + 6], v[8 * q + 7]));
  }
}

template <int G>
struct SplitGaugeFrags {
  sg_bf16x8_t b[2][2];  // [output block nb][g = 16: B1, B2 | g = 32: B_hi, B_lo]
};

__device__ __forceinline__ sg_bf16x8_t sg_pack8(const uint32_t (&h)[8]) {
  sg_u32x4_t u;
  u.x = h[0] | (h[1] << 16);
  u.y = h[2] | (h[3] << 16);
  u.z = h[4] | (h[5] << 16);
  u.w = h[6] | (h[7] << 16);
  return __builtin_bit_cast(sg_bf16x8_t, u);
}

// B operands of this wave for G^T (inverse): B[k][n] = G[input k][output c]
template <int G>
__device__ __forceinline__ void load_split_gauge(const float *__restrict__ Gf, SplitGaugeFrags<G> &f) {
  static_assert(G == 16 || G == 32, "split gauge handles g = 16 and 32");
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, kg = lane >> 4, n = lane & 15;
#pragma unroll
  for (int nb = 0; nb < 2; nb++) {
    const int col = 32 * wave + 16 * nb + n;
    const float *Gr = Gf + (col / G) * G * G;
    const int c = col % G;
    const int i0 = G == 16 ? 8 * (kg & 1) : 8 * kg;   // first input of this lane's k range
    uint32_t h[8], l[8];
#pragma unroll
    for (int e = 0; e < 8; e++) {
      const float gv = Gr[(i0 + e) * G + c];
      h[e] = bf16_rne(gv);
      l[e] = bf16_rne(gv - __uint_as_float(h[e] << 16));
    }
    f.b[nb][0] = sg_pack8(h);
    f.b[nb][1] = sg_pack8(l);
  }
}

// Inverse gauge of the split tile, results as fp32 in place (see the layout
// above).  Row blocks of 16 up to nrows; rows past nrows hold whatever the
// tile holds there and are never stored by the callers.
template <int G>
__device__ __forceinline__ void gauge_tile_split(unsigned char *tile, int nrows,
                                                 const SplitGaugeFrags<G> &f) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, kg = lane >> 4, n = lane & 15;
  unsigned char *wbase = tile + wave * 128;
  constexpr int TP = 2;  // row blocks per pass
  for (int rb0 = 0; rb0 < TILE_T / 16 && 16 * rb0 < nrows; rb0 += TP) {
    sg_bf16x8_t a[TP][2];
#pragma unroll
    for (int p = 0; p < TP; p++) {
      const unsigned char *r = wbase + (size_t)(16 * (rb0 + p) + n) * PITCH * 4;
      if constexpr (G == 16) {
        // a[p][nb]: hi (kg < 2) or lo (kg >= 2) parts of inputs 16 nb + 8 (kg & 1) ..
        const int off = (kg >> 1) * 64 + 16 * (kg & 1);
        a[p][0] = *(const sg_bf16x8_t *)(r + off);
        a[p][1] = *(const sg_bf16x8_t *)(r + off + 32);
      } else {
        // a[p][0]: hi parts of inputs 8 kg .. + 7, a[p][1]: lo parts
        a[p][0] = *(const sg_bf16x8_t *)(r + 16 * kg);
        a[p][1] = *(const sg_bf16x8_t *)(r + 64 + 16 * kg);
      }
    }
    sg_f32x4_t acc[TP][2];
#pragma unroll
    for (int p = 0; p < TP; p++)
#pragma unroll
      for (int nb = 0; nb < 2; nb++) {
        const sg_f32x4_t z = {0.f, 0.f, 0.f, 0.f};
        if constexpr (G == 16) {
          acc[p][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[p][nb], f.b[nb][0], z, 0, 0, 0);
          acc[p][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[p][nb], f.b[nb][1], acc[p][nb], 0, 0, 0);
        } else {
          acc[p][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[p][0], f.b[nb][0], z, 0, 0, 0);
          acc[p][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[p][0], f.b[nb][1], acc[p][nb], 0, 0, 0);
          acc[p][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[p][1], f.b[nb][0], acc[p][nb], 0, 0, 0);
        }
      }
    // every A operand of these rows is in registers: overwrite them with fp32
#pragma unroll
    for (int p = 0; p < TP; p++)
#pragma unroll
      for (int nb = 0; nb < 2; nb++)
#pragma unroll
        for (int j = 0; j < 4; j++)
          *(float *)(wbase + (size_t)(16 * (rb0 + p) + 4 * kg + j) * PITCH * 4 + (16 * nb + n) * 4) =
              acc[p][nb][j];
  }
}

}  // namespace cgk
