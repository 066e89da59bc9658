// Full-head (g = 128) gauge on the matrix cores.
//
// "Codec-Gauge" (arXiv HTML, gauge parameterization paragraph): full-head
// gauges are the most expressive setting; explicit application costs g
// multiply-adds per value, which at g = 128 is a dense contraction:
// X'(64 x 128 tile) = X (64 x 128) * G^T (128 x 128).
//
// MFMA v_mfma_f32_16x16x32_bf16 with fp32 accumulation, split precision:
// G = G_hi + G_lo with G_hi = bf16(G), G_lo = bf16(G - G_hi), and likewise X
// when it is not already a bf16 value, so that
//   X G^T ~= X_hi G_hi^T + X_hi G_lo^T + X_lo G_hi^T
// carries ~16 significand bits of every product (the dropped X_lo G_lo term
// is ~2^-16 of the smallest kept one).  A bf16 input has X_lo = 0 and takes
// two passes.
//
// Work split: wave w owns output channels [32w, 32w+32) (two 16-wide column
// tiles) for all 64 rows; its B fragments (G_hi, G_lo: 2 column tiles x 4
// k-steps) stay in VGPRs for every tile a workgroup processes, so the 64 KB
// matrix is read once per workgroup.  Operand layout of the 16x16x32
// instruction: lane l holds A row (l & 15), k = 8 (l >> 4) .. +7; B column
// (l & 15), same k; D column (l & 15), rows 4 (l >> 4) .. +3.
// Results are deterministic for a given tile, so the fused kernels and the
// exported gauge routine produce identical values.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cg_tile.hpp"

namespace cgk {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;

// round-to-nearest-even bf16 of x, and the bf16 of the remainder
__device__ __forceinline__ void split_bf16(float x, uint32_t &hi, uint32_t &lo) {
  hi = bf16_rne(x);
  lo = bf16_rne(x - __uint_as_float(hi << 16));
}

__device__ __forceinline__ bf16x8_t pack8(const uint32_t (&h)[8]) {
  u32x4_t u;
  u.x = h[0] | (h[1] << 16);
  u.y = h[2] | (h[3] << 16);
  u.z = h[4] | (h[5] << 16);
  u.w = h[6] | (h[7] << 16);
  return __builtin_bit_cast(bf16x8_t, u);
}

struct G128Frags {
  bf16x8_t hi[2][4];
  bf16x8_t lo[2][4];
};

// B fragments of this wave: forward B[k][n] = G[n][k]; inverse B[k][n] = G[k][n]
template <bool INV>
__device__ __forceinline__ void load_g128(const float *__restrict__ Gf, G128Frags &f) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int ntl = 0; ntl < 2; ntl++) {
    const int n = 32 * wave + 16 * ntl + (lane & 15);
#pragma unroll
    for (int ks = 0; ks < 4; ks++) {
      const int k0 = 32 * ks + 8 * (lane >> 4);
      uint32_t h[8], l[8];
#pragma unroll
      for (int e = 0; e < 8; e++) {
        const float gv = INV ? Gf[(k0 + e) * D + n] : Gf[n * D + k0 + e];
        split_bf16(gv, h[e], l[e]);
      }
      f.hi[ntl][ks] = pack8(h);
      f.lo[ntl][ks] = pack8(l);
    }
  }
}

// In-place X <- X G^T (forward fragments) or X G (inverse fragments) on the
// 64-row LDS tile.  EXACT: every tile value is a bf16 number (X_lo = 0).
// Contains two workgroup barriers.
template <bool EXACT>
__device__ __forceinline__ void gauge128_tile(float *xs, const G128Frags &f) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  f32x4_t acc[4][2];
#pragma unroll
  for (int mt = 0; mt < 4; mt++) {
    acc[mt][0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    acc[mt][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ks++) {
      const float *src = xs + (16 * mt + (lane & 15)) * PITCH + 32 * ks + 8 * (lane >> 4);
      const float4 v0 = *(const float4 *)src, v1 = *(const float4 *)(src + 4);
      const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
      uint32_t h[8], l[8];
#pragma unroll
      for (int e = 0; e < 8; e++) {
        if (EXACT) {
          h[e] = __float_as_uint(v[e]) >> 16;
          l[e] = 0;
        } else {
          split_bf16(v[e], h[e], l[e]);
        }
      }
      const bf16x8_t ah = pack8(h);
#pragma unroll
      for (int ntl = 0; ntl < 2; ntl++) {
        acc[mt][ntl] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, f.hi[ntl][ks], acc[mt][ntl], 0, 0, 0);
        acc[mt][ntl] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, f.lo[ntl][ks], acc[mt][ntl], 0, 0, 0);
      }
      if (!EXACT) {
        const bf16x8_t al = pack8(l);
#pragma unroll
        for (int ntl = 0; ntl < 2; ntl++)
          acc[mt][ntl] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, f.hi[ntl][ks], acc[mt][ntl], 0, 0, 0);
      }
    }
  }
  __syncthreads();  // every wave has read the whole tile
#pragma unroll
  for (int mt = 0; mt < 4; mt++)
#pragma unroll
    for (int ntl = 0; ntl < 2; ntl++) {
      const int n = 32 * wave + 16 * ntl + (lane & 15);
      const int m0 = 16 * mt + 4 * (lane >> 4);
      xs[(m0 + 0) * PITCH + n] = acc[mt][ntl].x;
      xs[(m0 + 1) * PITCH + n] = acc[mt][ntl].y;
      xs[(m0 + 2) * PITCH + n] = acc[mt][ntl].z;
      xs[(m0 + 3) * PITCH + n] = acc[mt][ntl].w;
    }
  __syncthreads();
}

}  // namespace cgk
