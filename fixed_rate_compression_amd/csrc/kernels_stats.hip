// Gauge-fit statistics of the frequency objective and their gradient
// ("Codec-Gauge", arXiv HTML, frequency-objective and gauge-training
// paragraphs).  For X' = G X, each block of 16 tokens x 128 channels gets an
// orthonormal 2D DCT-II  U = C16 X'_blk C128^T;  E = U^2;  per block
// L_b = sum(r E) / sum(E);  rate terms log(1 + U^2 / tau^2).  Gradient:
//   dU  = (lambda_f / N_b) 2 U (r - L_b) / sum(E) + (lambda_r / N_c) 2 U / (tau^2 + U^2)
//   dX' = C16^T dU C128,   Gamma_r += sum_t dX'_t[r] x_t[r]^T   (= dL/dG_r)
// The chain through G = exp(A - A^T) is finished on the host (Frechet
// derivative, fp64).
//
// Both 128-point transforms are dense 16 x 128 x 128 contractions per block and
// run on the matrix cores in fp32 (v_mfma_f32_16x16x4_f32: A lane l holds
// row l%16, k-slot l/16; B lane l holds k-slot l/16, column l%16; D lane l
// holds column l%16, rows 4(l/16)..+3).  The 128-point matrix sits in LDS
// with row v rotated left by rot(v) = 16 (v & 3) + 4 ((v >> 2) & 3) columns,
// which keeps both of its access patterns (row varying across lanes in the
// forward transform, column varying in the adjoint) free of bank conflicts.  The 16-point token transforms, the
// adjoint and the Gamma update use the same instruction with the summation
// index permuted so that k-slot g at k-step s is row 4g + s: the B (or A)
// operand is then exactly element s of the previous D fragment, with no
// cross-lane data movement.  The 128-point matrix lives in LDS; the 16-point
// one in VGPRs.
//
// Workgroup: 4 waves over a chunk of 64-token tiles of one field; wave w owns
// block w (rows 16w..16w+15) of each tile.  Per-chunk partial sums (fp64
// scalars, fp32 Gamma) go to the workspace and are reduced in a fixed order
// by k_stats_reduce, so results are deterministic.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "cg_stats.hpp"
#include "cg_tile.hpp"

namespace cgs {

using namespace cgk;
typedef __attribute__((ext_vector_type(4))) float f4;

__device__ __forceinline__ f4 mma(float a, float b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

__device__ __forceinline__ int rot(int v) { return 16 * (v & 3) + 4 * ((v >> 2) & 3); }

__device__ __forceinline__ void zero_rows(float *xs, int from) {
  for (int i = threadIdx.x; i < (TILE_T - from) * 32; i += NT)
    *(float4 *)(xs + (from + (i >> 5)) * PITCH + (i & 31) * 4) = make_float4(0.f, 0.f, 0.f, 0.f);
}

template <bool BF16, int G, bool GRAD>
__global__ __launch_bounds__(NT) void k_dct_stats(const void *__restrict__ kv,
                                                  const float *__restrict__ gauges,
                                                  const float *__restrict__ C128,
                                                  const float *__restrict__ C16,
                                                  const float *__restrict__ rtab,
                                                  double *__restrict__ part,
                                                  float *__restrict__ gpart, StatsArgs a) {
  // gauged tile (then the adjoint Z), and with the gradient the raw tile
  __shared__ float buf[(GRAD ? 2 : 1) * TILE_T * PITCH];
  __shared__ float blk[4][4][2];  // per wave, per block: partial sum E, sum r E
  __shared__ double red[4][3];
  float *xs = buf, *xr = buf + TILE_T * PITCH;
  // Gamma tiles of this wave: g = 16 (and g = 8, the 8x8 diagonal blocks of
  // the g = 16 tiles): groups 2w, 2w + 1; g = 32: group w as 2 x 2 tiles
  constexpr int NGW = G == 32 ? 4 : (G == 16 || G == 8 ? 2 : 0);
  constexpr int NGT = 4 * NGW;    // tiles per field
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, lg = lane >> 4, lm = lane & 15;
  const int64_t f = (int64_t)blockIdx.x / a.chunks;
  const int64_t chunk = (int64_t)blockIdx.x % a.chunks;
  const int64_t ntiles = (a.tokens + TILE_T - 1) / TILE_T;
  TileGauge<G, false> tg;
  if constexpr (G != 0) tg.load(gauges + gauge_index(f, a.batch, a.heads) * D * G);

  // wave w owns DCT columns v (forward) and channels c (adjoint) 32w .. 32w + 31
  const int n0 = 32 * wave + lm;                  // + 16 nt
  float bw[2][32], ba[2][GRAD ? 32 : 1];          // B operands of C128^T and C128
#pragma unroll
  for (int nt = 0; nt < 2; nt++)
#pragma unroll
    for (int ks = 0; ks < 32; ks++) {
      bw[nt][ks] = C128[(n0 + 16 * nt) * D + 4 * ks + lg];
      if constexpr (GRAD) ba[nt][ks] = C128[(4 * ks + lg) * D + n0 + 16 * nt];
    }
  float cB[4], cBt[4];  // C16 operand fragments (permuted summation index)
#pragma unroll
  for (int s = 0; s < 4; s++) {
    cB[s] = C16[lm * 16 + 4 * lg + s];
    cBt[s] = C16[(4 * lg + s) * 16 + lm];
  }
  float rr[2][4];
#pragma unroll
  for (int nt = 0; nt < 2; nt++)
#pragma unroll
    for (int i = 0; i < 4; i++) rr[nt][i] = rtab[(4 * lg + i) * D + n0 + 16 * nt];

  double sLb = 0.0, sLog = 0.0, sE = 0.0;
  f4 gacc[NGW > 0 ? NGW : 1];
#pragma unroll
  for (int q = 0; q < (NGW > 0 ? NGW : 1); q++) gacc[q] = f4{0.f, 0.f, 0.f, 0.f};

  for (int64_t tile = chunk * a.tiles_per_chunk;
       tile < min(ntiles, (chunk + 1) * a.tiles_per_chunk); tile++) {
    const int64_t tb = tile * TILE_T;
    const int nrows = (int)min((int64_t)TILE_T, a.tokens - tb);
    const uint8_t *src = (const uint8_t *)kv + (size_t)(f * a.tcap + tb) * D * (BF16 ? 2 : 4);
    load_tile<BF16>(src, nrows, xs);
    if constexpr (GRAD) load_tile<BF16>(src, nrows, xr);
    if (nrows < TILE_T) {
      zero_rows(xs, nrows);
      if constexpr (GRAD) zero_rows(xr, nrows);
    }
    __syncthreads();
    if constexpr (G != 0) {
      tg.apply(xs, nrows);
      __syncthreads();
    }
    // channel DCT of the four 16-row blocks: Y = X' C128^T (this wave's columns)
    f4 y[4][2];
#pragma unroll
    for (int mt = 0; mt < 4; mt++) y[mt][0] = y[mt][1] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 32; ks++) {
      float av[4];
#pragma unroll
      for (int mt = 0; mt < 4; mt++) av[mt] = xs[(16 * mt + lm) * PITCH + 4 * ks + lg];
#pragma unroll
      for (int mt = 0; mt < 4; mt++)
#pragma unroll
        for (int nt = 0; nt < 2; nt++) y[mt][nt] = mma(av[mt], bw[nt][ks], y[mt][nt]);
    }
    // token DCT: U = C16 Y per block
    f4 U[4][2];
#pragma unroll
    for (int mt = 0; mt < 4; mt++)
#pragma unroll
      for (int nt = 0; nt < 2; nt++) {
        U[mt][nt] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; s++) U[mt][nt] = mma(cB[s], y[mt][nt][s], U[mt][nt]);
      }
    float slog = 0.f;
#pragma unroll
    for (int mt = 0; mt < 4; mt++) {
      float se = 0.f, sre = 0.f;
#pragma unroll
      for (int nt = 0; nt < 2; nt++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const float u = U[mt][nt][i];
          const float e = u * u;
          se += e;
          sre += rr[nt][i] * e;
          // log2(1 + U^2/tau^2) with the hardware log2 (~1 ulp; the argument is
          // >= 1, so no cancellation near 0 matters for the sum); times ln 2 below
          slog += __builtin_amdgcn_logf(1.0f + e * a.inv_tau2);
        }
      se = wave_sum(se);
      sre = wave_sum(sre);
      if (lane == 0) {
        blk[wave][mt][0] = se;
        blk[wave][mt][1] = sre;
      }
    }
    sLog += (double)(wave_sum(slog) * 0.693147180559945309f);
    __syncthreads();  // block partials visible; every wave is done reading X'
    float Lb[4], seb[4];
#pragma unroll
    for (int mt = 0; mt < 4; mt++) {
      const float se = ((blk[0][mt][0] + blk[1][mt][0]) + blk[2][mt][0]) + blk[3][mt][0];
      const float sre = ((blk[0][mt][1] + blk[1][mt][1]) + blk[2][mt][1]) + blk[3][mt][1];
      seb[mt] = se;
      Lb[mt] = se > 0.f ? sre / se : 0.f;
      if (wave == 0 && 16 * mt < nrows) {
        sLb += (double)Lb[mt];
        sE += (double)se;
      }
    }
    if constexpr (GRAD) {
#pragma unroll
      for (int mt = 0; mt < 4; mt++) {
        const float cf = seb[mt] > 0.f ? a.lam_f_nb * 2.0f / seb[mt] : 0.f;
#pragma unroll
        for (int nt = 0; nt < 2; nt++)
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const float u = U[mt][nt][i];
            // d/dU of (lambda_r / N_c) log(1 + U^2/tau^2), with a ~1-ulp reciprocal
            y[mt][nt][i] = cf * u * (rr[nt][i] - Lb[mt]) +
                           a.lam_r_nc * 2.0f * u * __builtin_amdgcn_rcpf(a.tau2 + u * u);
          }
      }
      // adjoint token DCT: Z = C16^T dU, into the tile (this wave's columns)
#pragma unroll
      for (int mt = 0; mt < 4; mt++)
#pragma unroll
        for (int nt = 0; nt < 2; nt++) {
          f4 z = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < 4; s++) z = mma(cBt[s], y[mt][nt][s], z);
#pragma unroll
          for (int i = 0; i < 4; i++) xs[(16 * mt + 4 * lg + i) * PITCH + n0 + 16 * nt] = z[i];
        }
      __syncthreads();
      // adjoint channel DCT: dX' = Z C128 (this wave's channels)
#pragma unroll
      for (int mt = 0; mt < 4; mt++) U[mt][0] = U[mt][1] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 32; ks++) {
        float av[4];
#pragma unroll
        for (int mt = 0; mt < 4; mt++) av[mt] = xs[(16 * mt + lm) * PITCH + 4 * ks + lg];
#pragma unroll
        for (int mt = 0; mt < 4; mt++)
#pragma unroll
          for (int nt = 0; nt < 2; nt++) U[mt][nt] = mma(av[mt], ba[nt][ks], U[mt][nt]);
      }
      // Gamma_r[i][k] += sum_t dX'_t[r][i] x_t[r][k] over the tile's rows
#pragma unroll
      for (int mt = 0; mt < 4; mt++)
#pragma unroll
        for (int s = 0; s < 4; s++) {
          const float *xrow = xr + (16 * mt + 4 * lg + s) * PITCH + 32 * wave + lm;
          if constexpr (G == 8 || G == 16) {
#pragma unroll
            for (int q = 0; q < 2; q++) gacc[q] = mma(U[mt][q][s], xrow[16 * q], gacc[q]);
          } else if constexpr (G == 32) {
#pragma unroll
            for (int ta = 0; ta < 2; ta++)
#pragma unroll
              for (int tb2 = 0; tb2 < 2; tb2++)
                gacc[ta * 2 + tb2] = mma(U[mt][ta][s], xrow[16 * tb2], gacc[ta * 2 + tb2]);
          }
        }
    }
    __syncthreads();  // the tile buffers are rewritten by the next tile
  }

  // partial sums of this chunk, in a fixed order
  if (lane == 0) {
    red[wave][0] = sLb;
    red[wave][1] = sLog;
    red[wave][2] = sE;
  }
  __syncthreads();
  const int64_t slot = f * a.chunks + chunk;
  if (threadIdx.x == 0) {
    double s0 = 0, s1 = 0, s2 = 0;
    for (int w = 0; w < 4; w++) {
      s0 += red[w][0];
      s1 += red[w][1];
      s2 += red[w][2];
    }
    part[slot * 4 + 0] = s0;
    part[slot * 4 + 1] = s1;
    part[slot * 4 + 2] = s2;
    part[slot * 4 + 3] = 0.0;
  }
  if constexpr (GRAD && NGW > 0) {
    // tile q of the field: g = 16 / 8: group 2w + q; g = 32: group w, tile q
    float *gp = gpart + slot * (NGT * 256) + wave * NGW * 256;
#pragma unroll
    for (int q = 0; q < NGW; q++)
#pragma unroll
      for (int i = 0; i < 4; i++) gp[q * 256 + (4 * lg + i) * 16 + lm] = gacc[q][i];
  }
}

// per field: sum the chunk partials in chunk order (fp64)
__global__ __launch_bounds__(NT) void k_stats_reduce(const double *__restrict__ part,
                                                     const float *__restrict__ gpart,
                                                     double *__restrict__ out, int64_t chunks,
                                                     int ng, int grad) {
  const int64_t f = blockIdx.x;
  const int width = 4 + ng;
  if (threadIdx.x < 4) {
    double s = 0.0;
    for (int64_t c = 0; c < chunks; c++) s += part[(f * chunks + c) * 4 + threadIdx.x];
    out[f * width + threadIdx.x] = s;
  }
  if (grad)
    for (int e = threadIdx.x; e < ng; e += NT) {
      double s = 0.0;
      for (int64_t c = 0; c < chunks; c++) s += (double)gpart[(f * chunks + c) * ng + e];
      out[f * width + 4 + e] = s;
    }
}

hipError_t stats_launch(bool bf16, int g, const void *kv, const float *gauges, const float *C128,
                        const float *C16, const float *rtab, double *part, float *gpart,
                        double *out, const StatsArgs &a, int64_t fields, hipStream_t s) {
  const dim3 grid((unsigned)(fields * a.chunks)), block(NT);
#define CG_S(BF, GG)                                                                           \
  if (bf16 == BF && g == GG) {                                                                 \
    if (a.grad)                                                                                \
      hipLaunchKernelGGL((k_dct_stats<BF, GG, true>), grid, block, 0, s, kv, gauges, C128, C16, \
                         rtab, part, gpart, a);                                                \
    else                                                                                       \
      hipLaunchKernelGGL((k_dct_stats<BF, GG, false>), grid, block, 0, s, kv, gauges, C128,     \
                         C16, rtab, part, gpart, a);                                           \
  }
  CG_S(true, 0) CG_S(true, 8) CG_S(true, 16) CG_S(true, 32)
  CG_S(false, 0) CG_S(false, 8) CG_S(false, 16) CG_S(false, 32)
#undef CG_S
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int ng = g == 32 ? 16 * 256 : (g == 16 || g == 8 ? 8 * 256 : 0);
  hipLaunchKernelGGL(k_stats_reduce, dim3((unsigned)fields), block, 0, s, part, gpart, out,
                     a.chunks, ng, a.grad && g != 0);
  return hipGetLastError();
}

}  // namespace cgs
