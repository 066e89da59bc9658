// Device building blocks shared by the Codec-Gauge kernels: the LDS token
// tile, storage-format conversion, and the VALU gauge (g <= 32).
//
// Tile: TILE_T tokens x 128 channels of one field, held in LDS as fp32 with a
// row pitch of 132 floats (the 4-float pad spreads the per-token rows of the
// gauge phase over the LDS banks).  Global traffic into and out of the tile
// is 16-byte vector loads/stores over whole rows, so every wave touches
// contiguous memory.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cg_launch.hpp"

namespace cgk {

constexpr int D = 128;        // head_dim this build is specialized for
constexpr int PITCH = D + 4;  // LDS row pitch in floats
constexpr int NT = 256;       // threads per workgroup (4 waves)

// gauge set index of a field: fields are (layer, kv, batch, head) row-major,
// gauges (layer, kv, head) -- shared by every sequence of the batch
__device__ __forceinline__ int64_t gauge_index(int64_t field, int B, int H) {
  const int64_t ls = field / ((int64_t)B * H);
  return ls * H + field % H;
}

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (finite values)
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Two values -> packed bf16 pair (lo in bits 0..15) with the gfx950 pair
// conversion (v_cvt_pk_bf16_f32).  For every non-NaN fp32 input it returns
// exactly bf16_rne (checked exhaustively over all 2^32 bit patterns on an
// MI355X), one instruction per pair instead of five.
typedef __bf16 cg_bf16x2_t __attribute__((ext_vector_type(2)));
typedef float cg_f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const cg_f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, cg_bf16x2_t));
}

// rows [0, nrows) of a [rows][128] storage-format array -> LDS fp32 tile
template <bool BF16>
__device__ __forceinline__ void load_tile(const void *__restrict__ src, int nrows, float *xs) {
  if (BF16) {
    const uint4 *s = (const uint4 *)src;  // 16 chunks of 8 values per row
    for (int i = threadIdx.x; i < nrows * 16; i += NT) {
      const uint4 r = s[i];
      float *dst = xs + (i >> 4) * PITCH + (i & 15) * 8;
      *(float4 *)dst = make_float4(bf16lo(r.x), bf16hi(r.x), bf16lo(r.y), bf16hi(r.y));
      *(float4 *)(dst + 4) = make_float4(bf16lo(r.z), bf16hi(r.z), bf16lo(r.w), bf16hi(r.w));
    }
  } else {
    const float4 *s = (const float4 *)src;  // 32 chunks of 4 values per row
    for (int i = threadIdx.x; i < nrows * 32; i += NT)
      *(float4 *)(xs + (i >> 5) * PITCH + (i & 31) * 4) = s[i];
  }
}

// LDS fp32 tile -> rows [0, nrows) of a [rows][128] storage-format array
template <bool BF16>
__device__ __forceinline__ void store_tile(void *__restrict__ dst, int nrows, const float *xs) {
  if (BF16) {
    uint4 *d = (uint4 *)dst;
    for (int i = threadIdx.x; i < nrows * 16; i += NT) {
      const float *s = xs + (i >> 4) * PITCH + (i & 15) * 8;
      const float4 a = *(const float4 *)s, b = *(const float4 *)(s + 4);
      d[i] = make_uint4(pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w), pack_bf16x2(b.x, b.y),
                        pack_bf16x2(b.z, b.w));
    }
  } else {
    float4 *d = (float4 *)dst;
    for (int i = threadIdx.x; i < nrows * 32; i += NT)
      d[i] = *(const float4 *)(xs + (i >> 5) * PITCH + (i & 31) * 4);
  }
}

// Gauge (INV = false: y = G x) or inverse gauge (INV = true: y = G^T x) of
// every token row of the tile, in place, for group size G in {8, 16, 32}.
// Each output is an fmaf chain over the group's inputs in index order from
// +0.  A wave owns whole groups (the group index is wave-uniform), so the
// g x g matrix is read through the scalar cache and every FMA takes its
// matrix operand from an SGPR; lane = token row.
template <int G, bool INV>
__device__ __forceinline__ void gauge_tile(float *xs, int nrows, const float *__restrict__ Gf) {
  static_assert(G == 8 || G == 16 || G == 32, "VALU gauge handles g = 8, 16 and 32");
  constexpr int NG = D / G;      // groups per head
  constexpr int GPW = NG / 4;    // groups per wave
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int gg = 0; gg < GPW; gg++) {
    const int r = wave * GPW + gg;
    const float *__restrict__ Gr = Gf + r * G * G;
    if (lane < nrows) {
      float *row = xs + lane * PITCH + r * G;
      float x[G], y[G];
#pragma unroll
      for (int k = 0; k < G; k += 4) {
        const float4 t = *(const float4 *)(row + k);
        x[k] = t.x; x[k + 1] = t.y; x[k + 2] = t.z; x[k + 3] = t.w;
      }
#pragma unroll
      for (int o = 0; o < G; o++) {
        float acc = 0.0f;
#pragma unroll
        for (int m = 0; m < G; m++) acc = __builtin_fmaf(INV ? Gr[m * G + o] : Gr[o * G + m], x[m], acc);
        y[o] = acc;
      }
#pragma unroll
      for (int k = 0; k < G; k += 4) *(float4 *)(row + k) = make_float4(y[k], y[k + 1], y[k + 2], y[k + 3]);
    }
  }
}

}  // namespace cgk
