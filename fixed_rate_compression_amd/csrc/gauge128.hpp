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

// The tile as MFMA A operands: bf16 "hi" and "lo" parts of its 64 x 128
// values in LDS, row pitch HP bf16 (272 B = 17 x 16 B, so the 16 lanes of a
// fragment read, 16 B each from 16 rows, hit 64 distinct banks).  Every tile
// value is split exactly once, by the thread that produced it; the waves then
// read their fragments with plain 16-B loads.  The fp32 result tile (pitch
// PITCH floats) overlays the same LDS after all waves have read the operands.
constexpr int HP = 136;
constexpr int SPLIT_BYTES = 2 * TILE_T * HP * 2;                 // hi + lo tiles
constexpr int TILE_BYTES = TILE_T * PITCH * 4;                   // fp32 tile
constexpr int LDS_TILE_BYTES = SPLIT_BYTES > TILE_BYTES ? SPLIT_BYTES : TILE_BYTES;

// two values -> packed bf16 hi parts and packed bf16 remainders (each part
// round-to-nearest-even, as split_bf16)
__device__ __forceinline__ void split_pair(float a, float b, uint32_t &hi, uint32_t &lo) {
  hi = pack_bf16x2(a, b);
  lo = pack_bf16x2(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xFFFF0000u));
}

// One tile of a storage-format [rows][128] array held in registers between
// its global load and its LDS store, so that a workgroup can fetch tile i+1
// while the matrix cores work on tile i.  Thread i of the NTH threads holds
// the 16-B pieces i, i + NTH, ... (coalesced); rows past nrows read as zero.
template <bool BF16, int NTH = NT>
struct TileFetch {
  static constexpr int N = (BF16 ? TILE_T * D * 2 : TILE_T * D * 4) / 16 / NTH;  // pieces per thread
  uint4 r[N];

  __device__ __forceinline__ void fetch(const void *__restrict__ src, int nrows) {
    const uint4 *s = (const uint4 *)src;
#pragma unroll
    for (int k = 0; k < N; k++) {
      const int i = threadIdx.x + NTH * k;
      const int row = BF16 ? (i >> 4) : (i >> 5);
      r[k] = row < nrows ? s[i] : make_uint4(0u, 0u, 0u, 0u);
    }
  }

  // -> the fp32 LDS tile (pitch PITCH floats), bf16 widened exactly
  __device__ __forceinline__ void put_f32(float *xs) const {
#pragma unroll
    for (int k = 0; k < N; k++) {
      const int i = threadIdx.x + NTH * k;
      if (BF16) {
        float *d = xs + (i >> 4) * PITCH + 8 * (i & 15);
        *(float4 *)d = make_float4(bf16lo(r[k].x), bf16hi(r[k].x), bf16lo(r[k].y), bf16hi(r[k].y));
        *(float4 *)(d + 4) = make_float4(bf16lo(r[k].z), bf16hi(r[k].z), bf16lo(r[k].w), bf16hi(r[k].w));
      } else {
        *(uint4 *)(xs + (i >> 5) * PITCH + 4 * (i & 31)) = r[k];
      }
    }
  }

  // -> split tiles (bf16 inputs are their own hi part; lo is not used)
  __device__ __forceinline__ void put(uint16_t *sh, uint16_t *sl) const {
#pragma unroll
    for (int k = 0; k < N; k++) {
      const int i = threadIdx.x + NTH * k;
      if (BF16) {
        *(uint4 *)(sh + (i >> 4) * HP + 8 * (i & 15)) = r[k];
      } else {
        uint2 h, l;
        split_pair(__uint_as_float(r[k].x), __uint_as_float(r[k].y), h.x, l.x);
        split_pair(__uint_as_float(r[k].z), __uint_as_float(r[k].w), h.y, l.y);
        *(uint2 *)(sh + (i >> 5) * HP + 4 * (i & 31)) = h;
        *(uint2 *)(sl + (i >> 5) * HP + 4 * (i & 31)) = l;
      }
    }
  }
};

// the 32 values of row t, channels 32 j .. 32 j + 31 -> split tiles
__device__ __forceinline__ void split32(uint16_t *sh, uint16_t *sl, int t, int j, const float (&v)[32]) {
#pragma unroll
  for (int q = 0; q < 4; q++) {
    uint4 h, l;
    split_pair(v[8 * q], v[8 * q + 1], h.x, l.x);
    split_pair(v[8 * q + 2], v[8 * q + 3], h.y, l.y);
    split_pair(v[8 * q + 4], v[8 * q + 5], h.z, l.z);
    split_pair(v[8 * q + 6], v[8 * q + 7], h.w, l.w);
    *(uint4 *)(sh + t * HP + 32 * j + 8 * q) = h;
    *(uint4 *)(sl + t * HP + 32 * j + 8 * q) = l;
  }
}

// X G^T (forward fragments) or X G (inverse fragments) of the split tile into
// the fp32 tile xs, which may overlay sh/sl.  EXACT: every tile value is a
// bf16 number (no lo part: two passes instead of three).  Each accumulator
// takes its products in the order ks = 0..3, and within a ks hi*G_hi,
// hi*G_lo, lo*G_hi, so results depend on the tile only.  Contains two
// workgroup barriers; the caller has synchronized after writing sh/sl.
// AFFINE: the tile holds integer codes q and the result is written as
// scale_r (q G)[r][n] + min_r cs[n], with (min_r, scale_r) = rowp[r] and
// cs[n] the column sums of the matrix (the dequantized tile min + q scale
// times the matrix, with the range applied after the product).
template <bool EXACT, bool AFFINE = false>
__device__ __forceinline__ void gauge128_tile(const uint16_t *sh, const uint16_t *sl, float *xs,
                                              const G128Frags &f, const float2 *rowp = nullptr,
                                              const float *cs = nullptr) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  f32x4_t acc[4][2];
#pragma unroll
  for (int mt = 0; mt < 4; mt++) {
    acc[mt][0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    acc[mt][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  // k-step outermost: the eight accumulators advance together, so every
  // instruction is eight issues away from the previous one on its accumulator
#pragma unroll
  for (int ks = 0; ks < 4; ks++) {
    bf16x8_t ah[4], al[4];
#pragma unroll
    for (int mt = 0; mt < 4; mt++) {
      const int off = (16 * mt + (lane & 15)) * HP + 8 * (lane >> 4) + 32 * ks;
      ah[mt] = *(const bf16x8_t *)(sh + off);
      if (!EXACT) al[mt] = *(const bf16x8_t *)(sl + off);
    }
#pragma unroll
    for (int mt = 0; mt < 4; mt++)
#pragma unroll
      for (int ntl = 0; ntl < 2; ntl++)
        acc[mt][ntl] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[mt], f.hi[ntl][ks], acc[mt][ntl], 0, 0, 0);
#pragma unroll
    for (int mt = 0; mt < 4; mt++)
#pragma unroll
      for (int ntl = 0; ntl < 2; ntl++)
        acc[mt][ntl] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[mt], f.lo[ntl][ks], acc[mt][ntl], 0, 0, 0);
    if (!EXACT) {
#pragma unroll
      for (int mt = 0; mt < 4; mt++)
#pragma unroll
        for (int ntl = 0; ntl < 2; ntl++)
          acc[mt][ntl] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[mt], f.hi[ntl][ks], acc[mt][ntl], 0, 0, 0);
    }
  }
  __syncthreads();  // every wave has read its operands: xs may overwrite them
  if constexpr (AFFINE) {
    const float c0 = cs[32 * wave + (lane & 15)], c1 = cs[32 * wave + 16 + (lane & 15)];
#pragma unroll
    for (int mt = 0; mt < 4; mt++) {
      const int m0 = 16 * mt + 4 * (lane >> 4);
      const float4 pa = *(const float4 *)(rowp + m0), pb = *(const float4 *)(rowp + m0 + 2);
      const float mn[4] = {pa.x, pa.z, pb.x, pb.z}, sc[4] = {pa.y, pa.w, pb.y, pb.w};
#pragma unroll
      for (int ntl = 0; ntl < 2; ntl++) {
        const int n = 32 * wave + 16 * ntl + (lane & 15);
        const float c = ntl ? c1 : c0;
#pragma unroll
        for (int i = 0; i < 4; i++) xs[(m0 + i) * PITCH + n] = fmaf(sc[i], acc[mt][ntl][i], mn[i] * c);
      }
    }
  } else {
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
  }
  __syncthreads();
}

}  // namespace cgk
