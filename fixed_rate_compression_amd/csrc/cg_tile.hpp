// Device building blocks shared by the Codec-Gauge kernels: the LDS token
// tile, storage-format conversion, and the fmaf-chain gauge (matrix cores for
// g = 16, 32 and, with fp32 storage, 128; VALU for g = 8).
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

constexpr int D = 128;        // head_dim the kernels are specialized for
constexpr int PITCH = D + 4;  // LDS row pitch in floats
constexpr int NT = 256;       // threads per workgroup (4 waves)

// field of launch field i when a launch covers runs of `sel` consecutive
// fields every `step` fields, starting at field `base`
__device__ __forceinline__ int64_t launch_field(int64_t i, int64_t sel, int64_t step, int64_t base) {
  return (i / sel) * step + base + i % sel;
}

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

// Marks registers that global loads fill as read at this point (an empty
// asm statement, no instruction), so the wait for those loads is placed
// here.  The wait counter of vector memory operations drains in issue order
// and also counts stores; where a prefetch is followed by a run of predicated
// row stores, the compiler's wait at the data's first real use is counted
// from the path without the stores and so also waits for the stores to be
// acknowledged.  Calling this after the work that hides the loads and before
// the stores puts the wait where only the loads are outstanding.
__device__ __forceinline__ void loads_done(uint32_t x) { asm volatile("" ::"v"(x)); }
__device__ __forceinline__ void loads_done(float x) { asm volatile("" ::"v"(x)); }
__device__ __forceinline__ void loads_done(const uint4 &x) {
  asm volatile("" ::"v"(x.x), "v"(x.y), "v"(x.z), "v"(x.w));
}
template <typename T, int N>
__device__ __forceinline__ void loads_done(const T (&x)[N]) {
#pragma unroll
  for (int i = 0; i < N; i++) loads_done(x[i]);
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

// Cache-side error of decoded values against the reference, on the values as
// stored (after rounding to the storage format): sum of squared errors and of
// squared reference values, and the largest absolute error, all in fp64 (the
// difference of two storage values is exact in fp64).
struct ErrAcc {
  double sse = 0.0, ssr = 0.0, mx = 0.0;
  __device__ __forceinline__ void add(float xhat, float x) {
    const double e = (double)xhat - (double)x;
    sse += e * e;
    ssr += (double)x * (double)x;
    mx = fmax(mx, fabs(e));
  }
};

// store_tile that also accumulates the error against `ref` (same layout as dst)
template <bool BF16>
__device__ __forceinline__ void store_tile_err(void *__restrict__ dst, int nrows, const float *xs,
                                               const void *__restrict__ ref, ErrAcc &e) {
  if (BF16) {
    uint4 *d = (uint4 *)dst;
    const uint4 *r = (const uint4 *)ref;
    for (int i = threadIdx.x; i < nrows * 16; i += NT) {
      const float *s = xs + (i >> 4) * PITCH + (i & 15) * 8;
      const float4 a = *(const float4 *)s, b = *(const float4 *)(s + 4);
      const uint4 w = make_uint4(pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w), pack_bf16x2(b.x, b.y),
                                 pack_bf16x2(b.z, b.w));
      d[i] = w;
      const uint4 q = r[i];
      e.add(bf16lo(w.x), bf16lo(q.x)); e.add(bf16hi(w.x), bf16hi(q.x));
      e.add(bf16lo(w.y), bf16lo(q.y)); e.add(bf16hi(w.y), bf16hi(q.y));
      e.add(bf16lo(w.z), bf16lo(q.z)); e.add(bf16hi(w.z), bf16hi(q.z));
      e.add(bf16lo(w.w), bf16lo(q.w)); e.add(bf16hi(w.w), bf16hi(q.w));
    }
  } else {
    float4 *d = (float4 *)dst;
    const float4 *r = (const float4 *)ref;
    for (int i = threadIdx.x; i < nrows * 32; i += NT) {
      const float4 v = *(const float4 *)(xs + (i >> 5) * PITCH + (i & 31) * 4);
      d[i] = v;
      const float4 q = r[i];
      e.add(v.x, q.x); e.add(v.y, q.y); e.add(v.z, q.z); e.add(v.w, q.w);
    }
  }
}

// workgroup total of the error sums in a fixed order -> epart[blockIdx.x][3]
// (contains a workgroup barrier)
__device__ __forceinline__ void write_err(ErrAcc e, double *__restrict__ epart) {
  __shared__ double red[NT / 64][3];
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    e.sse += __shfl_xor(e.sse, m);
    e.ssr += __shfl_xor(e.ssr, m);
    e.mx = fmax(e.mx, __shfl_xor(e.mx, m));
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    red[w][0] = e.sse;
    red[w][1] = e.ssr;
    red[w][2] = e.mx;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double a = red[0][0], b = red[0][1], c = red[0][2];
    for (int k = 1; k < NT / 64; k++) {
      a += red[k][0];
      b += red[k][1];
      c = fmax(c, red[k][2]);
    }
    double *o = epart + (size_t)blockIdx.x * 3;
    o[0] = a;
    o[1] = b;
    o[2] = c;
  }
}

typedef float cg_f32x4_t __attribute__((ext_vector_type(4)));

// Matrix-core form of the gauge for g = 16, 32 and 128, in place on the
// tile.  v_mfma_f32_16x16x4f32 adds its four products to the accumulator as
// a chain of fused multiply-adds in k order (checked bit for bit on gfx950
// against fmaf chains, over normal, wide-exponent, cancelling and subnormal
// operands), so g/4 of them in k order give exactly the fmaf chain over the
// group's inputs in index order from +0 that the VALU form computes.
// Operand layout: A[m][k] in lane m + 16k, B[k][n] in lane n + 16k, D[m][n]
// in lane n + 16 (m / 4), element m % 4.  Wave w owns channels
// [32w, 32w + 32) (two groups of 16, one of 32, or a quarter of the full-head
// group) for all rows; one 16-row x 16-channel output block takes g/4
// instructions.  The B operands of a wave depend only on the field, so they
// are loaded once per workgroup (g = 128: 64 floats per lane).
template <int G>
struct MfmaGaugeFrags {
  static constexpr int KS = G / 4;  // instructions per output block
  float b[2][KS];                   // output block nb, step s: M[4s + kr][n]
};

// M[k][c] = G[c][k] (forward) or G[k][c] (inverse) of the output block's group
template <int G, bool INV>
__device__ __forceinline__ void load_mfma_gauge(const float *__restrict__ Gf, MfmaGaugeFrags<G> &f) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, kr = lane >> 4, n = lane & 15;
#pragma unroll
  for (int nb = 0; nb < 2; nb++) {
    const int col = 32 * wave + 16 * nb + n;     // output channel
    const float *Gr = Gf + (col / G) * G * G;
    const int c = col % G;
#pragma unroll
    for (int s = 0; s < MfmaGaugeFrags<G>::KS; s++) {
      const int k = 4 * s + kr;
      f.b[nb][s] = INV ? Gr[k * G + c] : Gr[c * G + k];
    }
  }
}

// Rows past nrows (up to the next 32-row boundary) are computed from
// whatever the tile holds there and are never stored by the callers.
// g = 128: every wave reads all 128 channels of the rows it updates, so the
// waves meet at a workgroup barrier between reading a row pair's operands and
// writing its results (the trip count depends on nrows only: uniform).
template <int G>
__device__ __forceinline__ void gauge_tile_mfma(float *xs, int nrows, const MfmaGaugeFrags<G> &f) {
  static_assert(G == 16 || G == 32 || G == 128, "matrix-core gauge handles g = 16, 32 and 128");
  constexpr int KS = G / 4;
  constexpr int TP = 2;  // 16-row blocks per pass: independent accumulation chains interleave
  constexpr int NA = G == 16 ? 2 : 1;  // A operand sets per row block (g >= 32: shared by both blocks)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, kr = lane >> 4, n = lane & 15;
  for (int tb0 = 0; tb0 < TILE_T / 16 && 16 * tb0 < nrows; tb0 += TP) {
    float a[TP][NA][KS];  // A[m = n][k = 4s + kr] of row block tb0 + p (g = 16: output block nb)
#pragma unroll
    for (int p = 0; p < TP; p++) {
      const float *arow = xs + (16 * (tb0 + p) + n) * PITCH + (G == 128 ? 0 : 32 * wave) + kr;
#pragma unroll
      for (int nb = 0; nb < NA; nb++)
#pragma unroll
        for (int s = 0; s < KS; s++) a[p][nb][s] = arow[16 * nb + 4 * s];
    }
    if constexpr (G == 128) __syncthreads();  // all waves hold the rows' operands
    cg_f32x4_t acc[TP][2];
#pragma unroll
    for (int p = 0; p < TP; p++)
#pragma unroll
      for (int nb = 0; nb < 2; nb++) acc[p][nb] = cg_f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < KS; s++)
#pragma unroll
      for (int p = 0; p < TP; p++)
#pragma unroll
        for (int nb = 0; nb < 2; nb++)
          acc[p][nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[p][NA == 2 ? nb : 0][s], f.b[nb][s],
                                                             acc[p][nb], 0, 0, 0);
#pragma unroll
    for (int p = 0; p < TP; p++)
#pragma unroll
      for (int nb = 0; nb < 2; nb++)
#pragma unroll
        for (int j = 0; j < 4; j++)
          xs[(16 * (tb0 + p) + 4 * kr + j) * PITCH + 32 * wave + 16 * nb + n] = acc[p][nb][j];
  }
}

// Gauge (INV = false: y = G x) or inverse gauge (INV = true: y = G^T x) of
// every token row of the tile, in place, for group size G = 8 on the VALU.
// Each output is an fmaf chain over the group's inputs in index order from
// +0.  A wave owns whole groups (the group index is wave-uniform), so the
// g x g matrix is read through the scalar cache and every FMA takes its
// matrix operand from an SGPR; lane = token row.
template <int G, bool INV>
__device__ __forceinline__ void gauge_tile(float *xs, int nrows, const float *__restrict__ Gf) {
  static_assert(G == 8 || G == 16 || G == 32, "gauge_tile handles g = 8, 16 and 32");
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

// The gauge of one field for every tile a workgroup processes: g = 16, 32
// and 128 on the matrix cores (operands loaded once), g = 8 on the VALU,
// g = 0 (identity) nothing.  Same results in every case: fmaf chains in index
// order from +0.
template <int G, bool INV>
struct TileGauge {
  static constexpr bool kMfma = G == 16 || G == 32 || G == 128;
  MfmaGaugeFrags<kMfma ? G : 16> f;
  const float *Gf;
  __device__ __forceinline__ void load(const float *__restrict__ gf) {
    Gf = gf;
    if constexpr (kMfma) load_mfma_gauge<G, INV>(gf, f);
  }
  __device__ __forceinline__ void apply(float *xs, int nrows) const {
    if constexpr (kMfma)
      gauge_tile_mfma<G>(xs, nrows, f);
    else if constexpr (G == 8)
      gauge_tile<G, INV>(xs, nrows, Gf);
  }
};

}  // namespace cgk
