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
// The gauge and the 128-point channel transform are one linear map per head,
// X' C128^T = X M^T with M = C128 diag(G_r) (M[v][c] = sum_i C128[v][g r + i]
// G_r[i][c - g r], formed once per workgroup in fp64 and rounded to fp32).  It
// runs on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16, fp32 accumulate)
// in split precision: M = M_hi + M_mid + M_lo, three bf16 parts that hold all
// 24 significand bits of the fp32 value.  A bf16 input is exact in the A
// operand, so X M^T takes three passes with exact products; an fp32 input is
// split the same way and takes the six passes whose parts sum to at least
// 2^-16 of the leading product.  The adjoint channel transform Z C128 splits
// Z and C128 into hi + lo and takes three passes (only lo x lo dropped).
// The 16-point token transforms, their adjoint and the Gamma update stay on
// the fp32 matrix cores (v_mfma_f32_16x16x4_f32) with the summation index
// permuted so that k-slot j at k-step s is row 4j + s: the B (or A) operand
// is then element s of the previous D fragment, with no cross-lane moves.
// Operand layouts: 16x16x32 A lane l holds row l%16, k = 8(l/16)..+7; B
// column l%16, same k; 16x16x4 A row l%16, k-slot l/16; B k-slot l/16, column
// l%16; both D: column l%16, rows 4(l/16)..+3.
//
// Workgroup: 4 waves over a chunk of 64-token tiles of one field; wave w owns
// DCT columns (forward) and channels (adjoint) 32w..32w+31 of all four 16-row
// blocks of a tile, its operand fragments in VGPRs.  Per-block sums are
// exchanged through LDS and added in a fixed wave order; per-chunk partial
// sums (fp64 scalars, fp32 Gamma) go to the workspace and are reduced in a
// fixed order by k_stats_reduce, so results are deterministic.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "cg_stats.hpp"
#include "cg_tile.hpp"
#include "gauge128.hpp"

namespace cgs {

using namespace cgk;
typedef __attribute__((ext_vector_type(4))) float f4;

__device__ __forceinline__ f4 mma(float a, float b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f4 mma8(bf16x8_t a, bf16x8_t b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// sum over the 64 lanes, wave-uniform: each 16-lane row is summed with DPP
// (quad swaps, then row rotations by 4 and 8), the four row sums in row order
__device__ __forceinline__ float wave_total(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v += dpp<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  v += dpp<0x124>(v);  // row_ror:4
  v += dpp<0x128>(v);  // row_ror:8
  const int b = __float_as_int(v);
  return (__int_as_float(__builtin_amdgcn_readlane(b, 0)) + __int_as_float(__builtin_amdgcn_readlane(b, 16))) +
         (__int_as_float(__builtin_amdgcn_readlane(b, 32)) + __int_as_float(__builtin_amdgcn_readlane(b, 48)));
}

// x = hi + mid + lo exactly (each part round-to-nearest-even bf16 of what the
// previous parts leave; both remainders are exact in fp32)
__device__ __forceinline__ void split3(float x, uint32_t &h, uint32_t &m, uint32_t &l) {
  h = bf16_rne(x);
  const float r = x - bf16lo(h);
  m = bf16_rne(r);
  l = bf16_rne(r - bf16lo(m));
}

constexpr int PL = TILE_T * HP;  // bf16 elements per LDS tile plane

// B fragments of M = C128 diag(G_r) for this wave's DCT columns v, split in
// three: mf[part][nt][ks] holds M[cw + 16nt + (l & 15)][32ks + 8(l >> 4) + e]
template <int G, int NTL>
__device__ __forceinline__ void fused_frags(const float *__restrict__ C128,
                                            const float *__restrict__ Gf, int cw, int lane,
                                            bf16x8_t (&mf)[3][NTL][4]) {
#pragma unroll
  for (int nt = 0; nt < NTL; nt++)
#pragma unroll
    for (int ks = 0; ks < 4; ks++) {
      const int v = cw + 16 * nt + (lane & 15);
      const int c0 = 32 * ks + 8 * (lane >> 4);
      double m[8];
      if constexpr (G == 0) {
#pragma unroll
        for (int e = 0; e < 8; e++) m[e] = (double)C128[v * D + c0 + e];
      } else {
        // channels c0 .. c0 + 7 lie in one gauge group (g is a multiple of 8)
        const int base = c0 / G * G;
        const float *gr = Gf + (size_t)(c0 / G) * G * G + (c0 - base);
#pragma unroll
        for (int e = 0; e < 8; e++) m[e] = 0.0;
#pragma unroll 4
        for (int i = 0; i < G; i++) {
          const double cv = (double)C128[v * D + base + i];
          const float4 g0 = *(const float4 *)(gr + i * G);
          const float4 g1 = *(const float4 *)(gr + i * G + 4);
          m[0] = fma(cv, (double)g0.x, m[0]);
          m[1] = fma(cv, (double)g0.y, m[1]);
          m[2] = fma(cv, (double)g0.z, m[2]);
          m[3] = fma(cv, (double)g0.w, m[3]);
          m[4] = fma(cv, (double)g1.x, m[4]);
          m[5] = fma(cv, (double)g1.y, m[5]);
          m[6] = fma(cv, (double)g1.z, m[6]);
          m[7] = fma(cv, (double)g1.w, m[7]);
        }
      }
      uint32_t h[8], md[8], l[8];
#pragma unroll
      for (int e = 0; e < 8; e++) split3((float)m[e], h[e], md[e], l[e]);
      mf[0][nt][ks] = pack8(h);
      mf[1][nt][ks] = pack8(md);
      mf[2][nt][ks] = pack8(l);
    }
}

// B fragments of the adjoint channel transform, B[k = v][n = c] = C128[v][c]
// for this wave's channels c, split in two
template <int NTL>
__device__ __forceinline__ void adjoint_frags(const float *__restrict__ C128, int cw, int lane,
                                              bf16x8_t (&cf)[2][NTL][4]) {
#pragma unroll
  for (int nt = 0; nt < NTL; nt++)
#pragma unroll
    for (int ks = 0; ks < 4; ks++) {
      const int c = cw + 16 * nt + (lane & 15);
      const int v0 = 32 * ks + 8 * (lane >> 4);
      uint32_t h[8], l[8];
#pragma unroll
      for (int e = 0; e < 8; e++) split_bf16(C128[(v0 + e) * D + c], h[e], l[e]);
      cf[0][nt][ks] = pack8(h);
      cf[1][nt][ks] = pack8(l);
    }
}

// the fetched tile -> bf16 planes of the LDS tile (a bf16 input is its own
// single plane; fp32 values are split into hi, mid, lo planes)
template <bool BF16, int NTH>
__device__ __forceinline__ void put_planes(const TileFetch<BF16, NTH> &tf, uint16_t *sx) {
#pragma unroll
  for (int k = 0; k < TileFetch<BF16, NTH>::N; k++) {
    const int i = threadIdx.x + NTH * k;
    if constexpr (BF16) {
      *(uint4 *)(sx + (i >> 4) * HP + 8 * (i & 15)) = tf.r[k];
    } else {
      const uint32_t w[4] = {tf.r[k].x, tf.r[k].y, tf.r[k].z, tf.r[k].w};
      uint32_t h[4], m[4], l[4];
#pragma unroll
      for (int e = 0; e < 4; e++) split3(__uint_as_float(w[e]), h[e], m[e], l[e]);
      const int off = (i >> 5) * HP + 4 * (i & 31);
      *(uint2 *)(sx + off) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
      *(uint2 *)(sx + PL + off) = make_uint2(m[0] | (m[1] << 16), m[2] | (m[3] << 16));
      *(uint2 *)(sx + 2 * PL + off) = make_uint2(l[0] | (l[1] << 16), l[2] | (l[3] << 16));
    }
  }
}

// raw value x[t][c] from the planes (hi + mid + lo is exact)
template <bool BF16>
__device__ __forceinline__ float raw_at(const uint16_t *sx, int off) {
  if constexpr (BF16) return bf16lo(sx[off]);
  else return (bf16lo(sx[off]) + bf16lo(sx[PL + off])) + bf16lo(sx[2 * PL + off]);
}

template <bool BF16, int G, bool GRAD, int NW>
__global__ __launch_bounds__(64 * NW, 2) void k_dct_stats(const void *__restrict__ kv,
                                                  const float *__restrict__ gauges,
                                                  const float *__restrict__ C128,
                                                  const float *__restrict__ C16,
                                                  const float *__restrict__ rtab,
                                                  double *__restrict__ part,
                                                  float *__restrict__ gpart, StatsArgs a) {
  constexpr int NTH = 64 * NW;      // threads
  constexpr int NTL = 8 / NW;        // 16-wide column tiles per wave
  constexpr int NX = BF16 ? 1 : 3;   // bf16 planes of the raw tile
  __shared__ __align__(16) uint16_t sx[NX * PL];
  __shared__ __align__(16) uint16_t sz[GRAD ? 2 * PL : 8];  // Z hi, lo (gradient)
  __shared__ float blk[NW][4][2];  // per wave, per block: partial sum E, sum r E
  __shared__ double red[NW][3];
  // 16 x 16 Gamma tiles: g = 16 (and g = 8, the 8x8 diagonal blocks of the
  // g = 16 tiles): one per group, 8 per field, a wave has those of its
  // channel tiles; g = 32: four per group (2 x 2), 16 per field, a wave has
  // the two column tiles of each of its channel tiles
  constexpr int NGW = G == 32 ? 2 * NTL : (G == 16 || G == 8 ? NTL : 0);
  constexpr int NGT = G == 32 ? 16 : (G == 16 || G == 8 ? 8 : 0);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, lg = lane >> 4, lm = lane & 15;
  const int64_t f = (int64_t)blockIdx.x / a.chunks;
  const int64_t chunk = (int64_t)blockIdx.x % a.chunks;
  const int64_t ntiles = (a.tokens + TILE_T - 1) / TILE_T;
  const int64_t tile0 = chunk * a.tiles_per_chunk;
  const int64_t tile1 = min(ntiles, tile0 + a.tiles_per_chunk);
  const size_t esz = BF16 ? 2 : 4;
  const uint8_t *fbase = (const uint8_t *)kv + (size_t)f * a.tcap * D * esz;

  TileFetch<BF16, NTH> tf;
  if (tile0 < tile1)
    tf.fetch(fbase + (size_t)tile0 * TILE_T * D * esz, (int)min((int64_t)TILE_T, a.tokens - tile0 * TILE_T));

  // wave w owns DCT columns v (forward) and channels c (adjoint) cw .. cw + 16 NTL - 1
  const int cw = 16 * NTL * wave;
  const int n0 = cw + lm;  // + 16 nt
  bf16x8_t mf[3][NTL][4];
  fused_frags<G, NTL>(C128, G ? gauges + gauge_index(f, a.batch, a.heads) * D * (G ? G : 1) : nullptr,
                      cw, lane, mf);
  bf16x8_t cf[2][NTL][GRAD ? 4 : 1];
  if constexpr (GRAD) adjoint_frags<NTL>(C128, cw, lane, cf);
  float cB[4], cBt[4];  // C16 operand fragments (permuted summation index)
#pragma unroll
  for (int s = 0; s < 4; s++) {
    cB[s] = C16[lm * 16 + 4 * lg + s];
    cBt[s] = C16[(4 * lg + s) * 16 + lm];
  }
  float rr[NTL][4];
#pragma unroll
  for (int nt = 0; nt < NTL; nt++)
#pragma unroll
    for (int i = 0; i < 4; i++) rr[nt][i] = rtab[(4 * lg + i) * D + n0 + 16 * nt];

  double sLb = 0.0, sE = 0.0;
  double sLog = 0.0;  // per lane, log2 units
  const float lam2 = a.lam_r_nc * 2.0f;
  f4 gacc[NGW > 0 ? NGW : 1];
#pragma unroll
  for (int q = 0; q < (NGW > 0 ? NGW : 1); q++) gacc[q] = f4{0.f, 0.f, 0.f, 0.f};

  for (int64_t tile = tile0; tile < tile1; tile++) {
    const int nrows = (int)min((int64_t)TILE_T, a.tokens - tile * TILE_T);
    put_planes<BF16, NTH>(tf, sx);  // rows past nrows were fetched as zero
    __syncthreads();
    if (tile + 1 < tile1)
      tf.fetch(fbase + (size_t)(tile + 1) * TILE_T * D * esz,
               (int)min((int64_t)TILE_T, a.tokens - (tile + 1) * TILE_T));

    // gauge + channel DCT of the four 16-row blocks: Y = X M^T (this wave's columns)
    f4 y[4][NTL];
#pragma unroll
    for (int mt = 0; mt < 4; mt++)
#pragma unroll
      for (int nt = 0; nt < NTL; nt++) y[mt][nt] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ks++) {
      bf16x8_t ax[4][NX];
#pragma unroll
      for (int mt = 0; mt < 4; mt++)
#pragma unroll
        for (int p = 0; p < NX; p++)
          ax[mt][p] = *(const bf16x8_t *)(sx + p * PL + (16 * mt + lm) * HP + 32 * ks + 8 * lg);
      // smallest parts first: (X, M) part pairs whose order sums to at most 2
#pragma unroll
      for (int ord = 2; ord >= 0; ord--)
#pragma unroll
        for (int p = 0; p < NX; p++) {
          if (p > ord) continue;
#pragma unroll
          for (int mt = 0; mt < 4; mt++)
#pragma unroll
            for (int nt = 0; nt < NTL; nt++)
              y[mt][nt] = mma8(ax[mt][p], mf[ord - p][nt][ks], y[mt][nt]);
        }
    }
    // token DCT: U = C16 Y per block
    f4 U[4][NTL];
#pragma unroll
    for (int mt = 0; mt < 4; mt++)
#pragma unroll
      for (int nt = 0; nt < NTL; nt++) {
        U[mt][nt] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; s++) U[mt][nt] = mma(cB[s], y[mt][nt][s], U[mt][nt]);
      }
    float slog = 0.f;
#pragma unroll
    for (int mt = 0; mt < 4; mt++) {
      float se = 0.f, sre = 0.f;
#pragma unroll
      for (int nt = 0; nt < NTL; nt++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const float u = U[mt][nt][i];
          const float e = u * u;
          se += e;
          sre = fmaf(rr[nt][i], e, sre);
          // log2(1 + U^2/tau^2) with the hardware log2 (~1 ulp; the argument is
          // >= 1, so no cancellation near 0 matters for the sum); times ln 2 at the end
          slog += __builtin_amdgcn_logf(fmaf(e, a.inv_tau2, 1.0f));
        }
      se = wave_total(se);
      sre = wave_total(sre);
      if (lane == 0) {
        blk[wave][mt][0] = se;
        blk[wave][mt][1] = sre;
      }
    }
    sLog += (double)slog;
    __syncthreads();  // block partials visible
    float Lb[4], seb[4];
#pragma unroll
    for (int mt = 0; mt < 4; mt++) {
      float se = blk[0][mt][0], sre = blk[0][mt][1];
#pragma unroll
      for (int w = 1; w < NW; w++) {
        se += blk[w][mt][0];
        sre += blk[w][mt][1];
      }
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
        const float cf0 = seb[mt] > 0.f ? a.lam_f_nb * 2.0f / seb[mt] : 0.f;
#pragma unroll
        for (int nt = 0; nt < NTL; nt++)
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const float u = U[mt][nt][i];
            // u (centroid term + d/dU-over-U of (lambda_r / N_c) log(1 + U^2/tau^2)),
            // with a ~1-ulp reciprocal
            y[mt][nt][i] = u * fmaf(cf0, rr[nt][i] - Lb[mt],
                                    lam2 * __builtin_amdgcn_rcpf(fmaf(u, u, a.tau2)));
          }
      }
      // adjoint token DCT, transposed: Z^T = dU^T C16 puts four consecutive
      // channels of one row in each lane; split hi + lo into the Z planes
#pragma unroll
      for (int mt = 0; mt < 4; mt++)
#pragma unroll
        for (int nt = 0; nt < NTL; nt++) {
          f4 z = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < 4; s++) z = mma(y[mt][nt][s], cBt[s], z);
          const uint32_t h0 = pack_bf16x2(z[0], z[1]), h1 = pack_bf16x2(z[2], z[3]);
          const uint32_t l0 = pack_bf16x2(z[0] - bf16lo(h0), z[1] - bf16hi(h0));
          const uint32_t l1 = pack_bf16x2(z[2] - bf16lo(h1), z[3] - bf16hi(h1));
          const int off = (16 * mt + lm) * HP + cw + 16 * nt + 4 * lg;
          *(uint2 *)(sz + off) = make_uint2(h0, h1);
          *(uint2 *)(sz + PL + off) = make_uint2(l0, l1);
        }
      __syncthreads();
      // adjoint channel DCT: dX' = Z C128 (this wave's channels)
#pragma unroll
      for (int mt = 0; mt < 4; mt++)
#pragma unroll
        for (int nt = 0; nt < NTL; nt++) U[mt][nt] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ks++) {
        bf16x8_t zh[4], zl[4];
#pragma unroll
        for (int mt = 0; mt < 4; mt++) {
          const int off = (16 * mt + lm) * HP + 32 * ks + 8 * lg;
          zh[mt] = *(const bf16x8_t *)(sz + off);
          zl[mt] = *(const bf16x8_t *)(sz + PL + off);
        }
#pragma unroll
        for (int mt = 0; mt < 4; mt++)
#pragma unroll
          for (int nt = 0; nt < NTL; nt++) {
            U[mt][nt] = mma8(zl[mt], cf[0][nt][ks], U[mt][nt]);
            U[mt][nt] = mma8(zh[mt], cf[1][nt][ks], U[mt][nt]);
            U[mt][nt] = mma8(zh[mt], cf[0][nt][ks], U[mt][nt]);
          }
      }
      // Gamma_r[i][k] += sum_t dX'_t[r][i] x_t[r][k] over the tile's rows
#pragma unroll
      for (int mt = 0; mt < 4; mt++)
#pragma unroll
        for (int s = 0; s < 4; s++) {
          const int row = (16 * mt + 4 * lg + s) * HP + lm;
          if constexpr (G == 8 || G == 16) {
            // channel tile ta is group cw / 16 + ta
#pragma unroll
            for (int ta = 0; ta < NTL; ta++)
              gacc[ta] = mma(U[mt][ta][s], raw_at<BF16>(sx, row + cw + 16 * ta), gacc[ta]);
          } else if constexpr (G == 32) {
            // channel tiles of group cw / 32 (all of it when NTL = 2, half otherwise)
            const int gb = cw / 32 * 32;
            const float x0 = raw_at<BF16>(sx, row + gb), x1 = raw_at<BF16>(sx, row + gb + 16);
#pragma unroll
            for (int ta = 0; ta < NTL; ta++) {
              gacc[ta * 2 + 0] = mma(U[mt][ta][s], x0, gacc[ta * 2 + 0]);
              gacc[ta * 2 + 1] = mma(U[mt][ta][s], x1, gacc[ta * 2 + 1]);
            }
          }
        }
    }
    __syncthreads();  // the tile planes are rewritten by the next tile
  }

  // partial sums of this chunk, in a fixed order
  sLog = wave_sum(sLog) * 0.693147180559945309;
  if (lane == 0) {
    red[wave][0] = sLb;
    red[wave][1] = sLog;
    red[wave][2] = sE;
  }
  __syncthreads();
  const int64_t slot = f * a.chunks + chunk;
  if (threadIdx.x == 0) {
    double s0 = 0, s1 = 0, s2 = 0;
    for (int w = 0; w < NW; w++) {
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
    // the wave's tiles are contiguous in the field's list: g = 16 / 8 from
    // group cw / 16; g = 32 from tile 2 (cw / 16) (group cw / 32, row tile
    // (cw / 16) % 2, column tiles 0 and 1)
    float *gp = gpart + slot * (NGT * 256) + (G == 32 ? 2 : 1) * (cw / 16) * 256;
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

// waves per workgroup: with the gradient 8 (a wave owns 16 columns, which
// halves its operand fragments to fit two waves per SIMD; the 8 waves share
// one LDS tile); without it 4 (already two waves per SIMD at 4 per group,
// and half as many per-block cross-lane sums per tile)
constexpr int kWavesGrad = 8;
constexpr int kWavesStats = 4;

hipError_t stats_launch(bool bf16, int g, const void *kv, const float *gauges, const float *C128,
                        const float *C16, const float *rtab, double *part, float *gpart,
                        double *out, const StatsArgs &a, int64_t fields, hipStream_t s) {
  const dim3 grid((unsigned)(fields * a.chunks)), block(NT);
#define CG_S(BF, GG)                                                                         \
  if (bf16 == BF && g == GG) {                                                               \
    if (a.grad)                                                                              \
      hipLaunchKernelGGL((k_dct_stats<BF, GG, true, kWavesGrad>), grid, dim3(64 * kWavesGrad), \
                         0, s, kv, gauges, C128, C16, rtab, part, gpart, a);                 \
    else                                                                                     \
      hipLaunchKernelGGL((k_dct_stats<BF, GG, false, kWavesStats>), grid,                    \
                         dim3(64 * kWavesStats), 0, s, kv, gauges, C128, C16, rtab, part,    \
                         gpart, a);                                                          \
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
