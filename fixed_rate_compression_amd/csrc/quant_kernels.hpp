// Fused gauge + block-uniform / KIVI-style quantizers, and their decoders
// ("Codec-Gauge", arXiv HTML, evaluation-protocol paragraph: block-uniform
// uses one range per T_b x d_l block; the KIVI-style path uses per-channel
// key and per-token value ranges; both run on the gauged cache with the same
// bit settings, and decoding applies the inverse gauge).
//
// Quantizer (one range [mn, mx] per group, L = 2^bits - 1):
//   scale = (mx - mn) / L, inv = L / (mx - mn)    (correctly rounded fp32)
//   q     = clamp(rint((x - mn) * inv), 0, L)     (ties to even, no FMA)
//   x_hat = mn + q * scale                        (multiply, then add)
//   mx == mn, or inv not finite: scale = 0, every q = 0.
// Codes are packed LSB first in token-major value order (value (t, c) of a
// field at bit (t * 128 + c) * bits of its code region).
//
// Work layout: a workgroup (256 threads) processes 64-token tiles of one
// field (a chunk of consecutive tiles when the full-head gauge is used, so
// its 64 KB matrix is loaded once).  With bf16 storage the full-head gauge
// runs on the matrix cores in reduced precision (kDense: one bf16 pass
// forward, one fp16 pass inverse, gauge128.hpp); with fp32 storage as fp32
// matrix-core fmaf chains (TileGauge, the reading order of the smaller
// groups).  After the gauge, thread i owns the 32 values (row i/4, channels
// 32 (i%4) .. +31): exactly `bits` 32-bit words of codes, stored with one
// vector store, so a wave writes a contiguous span.
#pragma once

#include <float.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cg_quant.hpp"
#include "cg_tile.hpp"
#include "gauge128.hpp"
#include "split_gauge.hpp"

namespace cgq {

using namespace cgk;

// full-head gauge with bf16 storage: reduced-precision matrix-core path
template <int G, bool BF16>
constexpr bool kDense = G == 128 && BF16;

// decoders with bf16 storage and g = 16 / 32: inverse gauge as
// split-precision bf16 matrix-core products (split_gauge.hpp)
template <int G, bool BF16>
constexpr bool kSplitInv = BF16 && (G == 16 || G == 32);

// the fp32 fmaf-chain inverse gauge a decoder keeps (none where another
// path applies it)
template <int G, bool BF16>
constexpr int kChainInv = (kDense<G, BF16> || kSplitInv<G, BF16>) ? 0 : G;

struct QK {
  int64_t tcap, tokens, t0, nt;
  int64_t chunks;           // workgroups per field
  int32_t tiles_per_chunk;  // 64-token tiles per workgroup
  int32_t batch, heads, kv;
  int32_t block;            // block-uniform: tokens per range block
  int32_t residual;         // KIVI: tail rows kept in the storage format
  const void *ref;          // decode: reference rows for the error sums (or null)
  double *epart;            // decode: per-workgroup error partials [grid][3]
  int64_t fsel, fstep, fbase;  // decode: fields covered (launch_field)
};

// valid rows of tile `tile` of the call's row range
__device__ __forceinline__ int tile_rows(const QK &a, int64_t tile) {
  return (int)min((int64_t)TILE_T, a.nt - tile * TILE_T);
}

struct Range {
  float mn, scale, inv;
  bool zero;
};

__device__ __forceinline__ Range make_range(float mn, float mx, int L) {
  Range r;
  r.mn = mn;
  const float diff = mx - mn;
  r.inv = diff > 0.0f ? (float)L / diff : 0.0f;
  r.zero = (mx == mn) || !(r.inv <= FLT_MAX);
  r.scale = r.zero ? 0.0f : diff / (float)L;
  return r;
}

__device__ __forceinline__ uint32_t quant1(float x, const Range &r, int L) {
  if (r.zero) return 0u;
  const float s = x - r.mn;
  const float p = s * r.inv;
  int q = (int)rintf(p);
  q = q < 0 ? 0 : (q > L ? L : q);
  return (uint32_t)q;
}

__device__ __forceinline__ float dequant1(uint32_t q, float mn, float scale) {
  const float p = (float)q * scale;
  return mn + p;
}

template <int BITS>
__device__ __forceinline__ void pack32(const uint32_t (&q)[32], uint32_t (&w)[BITS]) {
#pragma unroll
  for (int d = 0; d < BITS; d++) w[d] = 0;
#pragma unroll
  for (int k = 0; k < 32; k++) {
    const int pos = k * BITS;
    w[pos >> 5] |= q[k] << (pos & 31);
    if ((pos & 31) + BITS > 32) w[(pos >> 5) + 1] |= q[k] >> (32 - (pos & 31));
  }
}

template <int BITS>
__device__ __forceinline__ void unpack32(const uint32_t (&w)[BITS], uint32_t (&q)[32]) {
  constexpr uint32_t M = (1u << BITS) - 1u;
#pragma unroll
  for (int k = 0; k < 32; k++) {
    const int pos = k * BITS;
    uint32_t v = w[pos >> 5] >> (pos & 31);
    if ((pos & 31) + BITS > 32) v |= w[(pos >> 5) + 1] << (32 - (pos & 31));
    q[k] = v & M;
  }
}

template <int BITS>
__device__ __forceinline__ void store_words(uint8_t *p, const uint32_t (&w)[BITS]) {
  if constexpr (BITS == 4) {
    *(uint4 *)p = make_uint4(w[0], w[1], w[2], w[3]);
  } else if constexpr (BITS == 8) {
    ((uint4 *)p)[0] = make_uint4(w[0], w[1], w[2], w[3]);
    ((uint4 *)p)[1] = make_uint4(w[4], w[5], w[6], w[7]);
  } else if constexpr (BITS == 2) {
    *(uint2 *)p = make_uint2(w[0], w[1]);
  } else {
#pragma unroll
    for (int d = 0; d < BITS; d++) ((uint32_t *)p)[d] = w[d];
  }
}

template <int BITS>
__device__ __forceinline__ void load_words(const uint8_t *p, uint32_t (&w)[BITS]) {
  if constexpr (BITS == 4) {
    const uint4 u = *(const uint4 *)p;
    w[0] = u.x; w[1] = u.y; w[2] = u.z; w[3] = u.w;
  } else if constexpr (BITS == 8) {
    const uint4 u = ((const uint4 *)p)[0], v = ((const uint4 *)p)[1];
    w[0] = u.x; w[1] = u.y; w[2] = u.z; w[3] = u.w;
    w[4] = v.x; w[5] = v.y; w[6] = v.z; w[7] = v.w;
  } else if constexpr (BITS == 2) {
    const uint2 u = *(const uint2 *)p;
    w[0] = u.x; w[1] = u.y;
  } else {
#pragma unroll
    for (int d = 0; d < BITS; d++) w[d] = ((const uint32_t *)p)[d];
  }
}

__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fminf(v, __shfl_xor(v, m));
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}

// the 32 tile values owned by this thread (row t, channels 32 j .. 32 j + 31)
__device__ __forceinline__ void read32(const float *xs, int t, int j, float (&v)[32]) {
  const float *s = xs + t * PITCH + 32 * j;
#pragma unroll
  for (int k = 0; k < 32; k += 4) {
    const float4 q = *(const float4 *)(s + k);
    v[k] = q.x; v[k + 1] = q.y; v[k + 2] = q.z; v[k + 3] = q.w;
  }
}

__device__ __forceinline__ void write32(float *xs, int t, int j, const float (&v)[32]) {
  float *d = xs + t * PITCH + 32 * j;
#pragma unroll
  for (int k = 0; k < 32; k += 4) *(float4 *)(d + k) = make_float4(v[k], v[k + 1], v[k + 2], v[k + 3]);
}

// Forward-gauged tiles of one workgroup's chunk.  next() stores the fetched
// tile (rows [0, nrows); rows past nrows are zero) and applies the forward
// gauge; the fp32 result is in the tile view of `lds` (PITCH floats per row).
// The global loads of the following tile are issued before the gauge, so
// they are in flight during the gauge and the quantizer work.  Full-head
// gauge: `lds` holds kEncLds<G, BF16> bytes, the fp32 tile apart from the
// bf16 operand tile, so next() needs no barrier between the products and
// their results, and the caller none after its reads of the fp32 tile (the
// next call's barrier after the operand writes orders them).  Otherwise the
// caller synchronizes after its reads of the fp32 tile before calling next()
// again.
// LDS bytes of the encoders' tile
template <int G, bool BF16>
constexpr int kEncLds = kDense<G, BF16> ? APART_TILE_BYTES : LDS_TILE_BYTES;

template <int G, bool BF16>
struct GaugedTiles {
  TileFetch<BF16> pre;

  __device__ __forceinline__ void prefetch(const void *__restrict__ src, int nrows) {
    pre.fetch(src, nrows);
  }

  // the wait for the prefetched tile, placed by the caller after the work
  // that hides it and before the tile's stores (see loads_done)
  __device__ __forceinline__ void arrived() const { loads_done(pre.r); }

  // next_src/next_rows: the tile after this one (next_rows = 0: none)
  __device__ __forceinline__ void next(const void *__restrict__ src, int nrows,
                                       const void *__restrict__ next_src, int next_rows,
                                       unsigned char *lds, const TileGauge<G, false> &tg,
                                       const G128Frags &fr) {
    float *xs = (float *)lds;
    if constexpr (kDense<G, BF16>) {
      uint16_t *sh = (uint16_t *)(lds + TILE_BYTES);
      pre.put(sh, sh);
      __syncthreads();
      if (next_rows > 0) pre.fetch(next_src, next_rows);
      gauge128_tile<true, true, true>(sh, sh, xs, fr);
    } else {
      (void)src;
      pre.put_f32(xs);
      __syncthreads();
      if (next_rows > 0) pre.fetch(next_src, next_rows);
      if constexpr (G != 0) {
        tg.apply(xs, nrows);
        __syncthreads();
      }
    }
  }
};

// Every thread hands over its 32 decoded values (row t, channels 32 j ..);
// apply the inverse gauge to the whole tile, result in the tile view of lds
// (every path but the full-head gauge with bf16 storage, which the decoders
// run on fp16 operands with direct row stores).
template <int G, bool BF16>
__device__ __forceinline__ void inverse_gauged_tile(unsigned char *lds, int t, int j,
                                                    const float (&v)[32], int nrows,
                                                    const TileGauge<kChainInv<G, BF16>, true> &tg,
                                                    const SplitGaugeFrags<kSplitInv<G, BF16> ? G : 16> &sg) {
  static_assert(!kDense<G, BF16>, "full-head bf16 decoders use gauge128_f16_rows");
  float *xs = (float *)lds;
  if constexpr (kSplitInv<G, BF16>) {
    split_store32(lds, t, j, v);
    __syncthreads();
    gauge_tile_split<G>(lds, nrows, sg);
    __syncthreads();
  } else {
    write32(xs, t, j, v);
    __syncthreads();
    if constexpr (G != 0) {
      tg.apply(xs, nrows);
      __syncthreads();
    }
  }
}

// Full-head decoders: the product leaves each lane 16 B of one row (8
// channels), so a wave could store only 64 B of each of 16 rows per
// instruction, and such stores, with two waves completing each 128-byte
// line, stream markedly slower than whole rows.  The bf16 results are
// therefore staged in LDS as the tile's 64 rows x 256 B and stored as whole
// rows, 4 rows per wave instruction (wave w: rows 16 w .. + 15).  The
// 16-byte pieces of a staged row are swizzled, piece ^ (row % 16), so that
// the writes (16 rows, one piece each) and the row reads both hit 64
// distinct banks.
constexpr int STAGE_BYTES = TILE_T * D * 2;

__device__ __forceinline__ int stage_off(int r, int piece) { return r * 256 + 16 * (piece ^ (r & 15)); }

// row blocks MT0 .. MT0 + NMT - 1 of the accumulators of gauge128_f16_rows
// as bf16 into the staged tile.  AFFINE: value = scale_r acc + min_r cs[c]
// with (min_r, scale_r) = rowp[r]; otherwise acc rsc[r].
template <bool AFFINE, int MT0, int NMT>
__device__ __forceinline__ void stage_rows(unsigned char *stage, const f32x4_t (&acc)[NMT][2],
                                           const float *rsc, const float2 *rowp, const float *cs) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, g = lane >> 4;
  const int c0 = 32 * wave + 8 * g;
  float c[8];
  if constexpr (AFFINE) {
    const float4 ca = *(const float4 *)(cs + c0), cb = *(const float4 *)(cs + c0 + 4);
    c[0] = ca.x; c[1] = ca.y; c[2] = ca.z; c[3] = ca.w;
    c[4] = cb.x; c[5] = cb.y; c[6] = cb.z; c[7] = cb.w;
  }
#pragma unroll
  for (int m = 0; m < NMT; m++) {
    const int r = 16 * (MT0 + m) + (lane & 15);
    float v[8];
    if constexpr (AFFINE) {
      const float2 pr = rowp[r];
#pragma unroll
      for (int q = 0; q < 4; q++) {
        v[q] = fmaf(pr.y, acc[m][0][q], pr.x * c[q]);
        v[4 + q] = fmaf(pr.y, acc[m][1][q], pr.x * c[4 + q]);
      }
    } else {
      const float sr = rsc[r];
#pragma unroll
      for (int q = 0; q < 4; q++) {
        v[q] = acc[m][0][q] * sr;
        v[4 + q] = acc[m][1][q] * sr;
      }
    }
    *(uint4 *)(stage + stage_off(r, 4 * wave + g)) =
        make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
  }
}

// the inverse gauge of the fp16 tile into the staged tile, in two halves of
// 32 rows (fewer live accumulators)
template <bool AFFINE>
__device__ __forceinline__ void gauge_stage_tile(const uint16_t *sh, unsigned char *stage, const G128Frags &fr,
                                                 const float *rsc, const float2 *rowp, const float *cs) {
  {
    f32x4_t acc[2][2];
    gauge128_f16_rows<0, 2>(sh, fr, acc);
    stage_rows<AFFINE, 0, 2>(stage, acc, rsc, rowp, cs);
  }
  {
    f32x4_t acc[2][2];
    gauge128_f16_rows<2, 2>(sh, fr, acc);
    stage_rows<AFFINE, 2, 2>(stage, acc, rsc, rowp, cs);
  }
}

// the reference rows the lanes store in store_staged (zeros past nrows)
__device__ __forceinline__ void load_ref_rows(const uint8_t *__restrict__ ref, int nrows, uint4 (&rq)[4]) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int k = 0; k < 4; k++) {
    const int r = 16 * wave + 4 * k + (lane >> 4);
    rq[k] = r < nrows ? *(const uint4 *)(ref + (size_t)r * D * 2 + 16 * (lane & 15)) : make_uint4(0u, 0u, 0u, 0u);
  }
}

// the staged tile's rows [0, nrows) -> bf16 rows at dst (the tile's first
// row); with_ref: also the error sums against the rows rq of load_ref_rows
__device__ __forceinline__ void store_staged(uint8_t *__restrict__ dst, int nrows, const unsigned char *stage,
                                             bool with_ref, const uint4 (&rq)[4], ErrAcc &e) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int k = 0; k < 4; k++) {
    const int r = 16 * wave + 4 * k + (lane >> 4);
    const uint4 w = *(const uint4 *)(stage + stage_off(r, lane & 15));
    if (r < nrows) {
      *(uint4 *)(dst + (size_t)r * D * 2 + 16 * (lane & 15)) = w;
      if (with_ref) {
        const uint4 q = rq[k];
        e.add(bf16lo(w.x), bf16lo(q.x)); e.add(bf16hi(w.x), bf16hi(q.x));
        e.add(bf16lo(w.y), bf16lo(q.y)); e.add(bf16hi(w.y), bf16hi(q.y));
        e.add(bf16lo(w.z), bf16lo(q.z)); e.add(bf16hi(w.z), bf16hi(q.z));
        e.add(bf16lo(w.w), bf16lo(q.w)); e.add(bf16hi(w.w), bf16hi(q.w));
      }
    }
  }
}

// Full-head decoders, after every thread has written its part of the fp16
// tile (the start of lds, row pitch HP): the inverse gauge, the bf16 rows
// staged beside the tile (stage_rows) and stored whole.  arrived() places
// the wait for the prefetched next tile before the stores (see loads_done).
// Two barriers; the second also orders this tile's reads of the fp16 tile,
// of rsc / rowp and of the key ranges before the next tile's writes.  The
// block-uniform decoder (AFFINE) loads the reference rows after the product
// (it fits four waves' registers that way), the KIVI-style one before it.
template <bool AFFINE, typename Arrived>
__device__ __forceinline__ void decode_tile_dense(unsigned char *lds, const G128Frags &fr, const float *rsc,
                                                  const float2 *rowp, const float *cs, int nrows,
                                                  uint8_t *__restrict__ dst, const uint8_t *__restrict__ ref,
                                                  ErrAcc &err, Arrived arrived) {
  const uint16_t *sh = (const uint16_t *)lds;
  unsigned char *stage = lds + TILE_T * HP * 2;
  __syncthreads();
  uint4 rq[4];
  if (!AFFINE && ref) load_ref_rows(ref, nrows, rq);
  gauge_stage_tile<AFFINE>(sh, stage, fr, rsc, rowp, cs);
  if (AFFINE && ref) load_ref_rows(ref, nrows, rq);
  arrived();
  if (ref) loads_done(rq);
  __syncthreads();
  store_staged(dst, nrows, stage, ref != nullptr, rq, err);
}

// storage-format row segment of 32 values <-> fp32
template <bool BF16>
__device__ __forceinline__ void store32_storage(uint8_t *p, const float (&v)[32]) {
  if (BF16) {
    uint4 *d = (uint4 *)p;
#pragma unroll
    for (int k = 0; k < 4; k++)
      d[k] = make_uint4(pack_bf16x2(v[8 * k], v[8 * k + 1]), pack_bf16x2(v[8 * k + 2], v[8 * k + 3]),
                        pack_bf16x2(v[8 * k + 4], v[8 * k + 5]), pack_bf16x2(v[8 * k + 6], v[8 * k + 7]));
  } else {
    float4 *d = (float4 *)p;
#pragma unroll
    for (int k = 0; k < 8; k++) d[k] = make_float4(v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]);
  }
}

template <bool BF16>
__device__ __forceinline__ void load32_storage(const uint8_t *p, float (&v)[32]) {
  if (BF16) {
    const uint4 *s = (const uint4 *)p;
#pragma unroll
    for (int k = 0; k < 4; k++) {
      const uint4 r = s[k];
      v[8 * k] = bf16lo(r.x); v[8 * k + 1] = bf16hi(r.x);
      v[8 * k + 2] = bf16lo(r.y); v[8 * k + 3] = bf16hi(r.y);
      v[8 * k + 4] = bf16lo(r.z); v[8 * k + 5] = bf16hi(r.z);
      v[8 * k + 6] = bf16lo(r.w); v[8 * k + 7] = bf16hi(r.w);
    }
  } else {
    const float4 *s = (const float4 *)p;
#pragma unroll
    for (int k = 0; k < 8; k++) {
      const float4 r = s[k];
      v[4 * k] = r.x; v[4 * k + 1] = r.y; v[4 * k + 2] = r.z; v[4 * k + 3] = r.w;
    }
  }
}

// ---------------------------------------------------------------------------
// block-uniform
// ---------------------------------------------------------------------------

template <int BITS, bool BF16, int G>
__device__ __forceinline__ void bu_encode_body(const void *__restrict__ kv,
                                                  const float *__restrict__ gauges,
                                                  uint8_t *__restrict__ payload,
                                                  float *__restrict__ meta, QK a) {
  __shared__ __align__(16) unsigned char lds[kEncLds<G, BF16>];
  float *xs = (float *)lds;
  __shared__ float red[8];
  constexpr int L = (1 << BITS) - 1;
  const int64_t f = (int64_t)blockIdx.x / a.chunks;
  const int64_t chunk = (int64_t)blockIdx.x % a.chunks;
  const int64_t ntiles = (a.nt + TILE_T - 1) / TILE_T;
  const float *Gf = G ? gauges + gauge_index(f, a.batch, a.heads) * D * (G ? G : 1) : nullptr;
  G128Frags fr;
  if constexpr (kDense<G, BF16>) load_g128<false>(Gf, fr);
  TileGauge<G, false> tg;
  if constexpr (G != 0 && !kDense<G, BF16>) tg.load(Gf);
  const int BT = a.block;
  const int64_t nblk_f = a.tcap / BT;
  const int t = threadIdx.x >> 2, j = threadIdx.x & 3, w = threadIdx.x >> 6;
  constexpr size_t ESZ = BF16 ? 2 : 4;
  const uint8_t *src_f = (const uint8_t *)kv + (size_t)f * a.tcap * D * ESZ;
  const int64_t tile0 = chunk * a.tiles_per_chunk;
  const int64_t tend = min(ntiles, (chunk + 1) * a.tiles_per_chunk);
  GaugedTiles<G, BF16> tiles;
  if (tile0 < tend) tiles.prefetch(src_f + (size_t)(a.t0 + tile0 * TILE_T) * D * ESZ, tile_rows(a, tile0));
  tiles.arrived();
  for (int64_t tile = tile0; tile < tend; tile++) {
    const int64_t tb = a.t0 + tile * TILE_T;
    const int nrows = tile_rows(a, tile);
    tiles.next(src_f + (size_t)tb * D * ESZ, nrows, src_f + (size_t)(tb + TILE_T) * D * ESZ,
               tile + 1 < tend ? tile_rows(a, tile + 1) : 0, lds, tg, fr);
    const bool active = t < nrows;
    float v[32];
    float mn = INFINITY, mx = -INFINITY;
    if (active) {
      read32(xs, t, j, v);
#pragma unroll
      for (int k = 0; k < 32; k++) {
        mn = fminf(mn, v[k]);
        mx = fmaxf(mx, v[k]);
      }
    }
    mn = wave_min(mn);
    mx = wave_max(mx);
    if ((threadIdx.x & 63) == 0) {
      red[2 * w] = mn;
      red[2 * w + 1] = mx;
    }
    __syncthreads();
    tiles.arrived();
    if (active) {
      const int wpb = BT / 16, w0 = (t / BT) * wpb;
      mn = red[2 * w0];
      mx = red[2 * w0 + 1];
      for (int k = 1; k < wpb; k++) {
        mn = fminf(mn, red[2 * (w0 + k)]);
        mx = fmaxf(mx, red[2 * (w0 + k) + 1]);
      }
      const Range r = make_range(mn, mx, L);
      uint32_t q[32], wd[BITS];
#pragma unroll
      for (int k = 0; k < 32; k++) q[k] = quant1(v[k], r, L);
      pack32<BITS>(q, wd);
      store_words<BITS>(payload + (size_t)(f * a.tcap + tb) * 16 * BITS + threadIdx.x * 4 * BITS, wd);
      if (j == 0 && (t % BT) == 0) {
        float *m = meta + 2 * (f * nblk_f + (tb + t) / BT);
        m[0] = r.mn;
        m[1] = r.scale;
      }
    }
    if constexpr (!kDense<G, BF16>) __syncthreads();  // see GaugedTiles
  }
}

template <int BITS, bool BF16, int G>
__global__ __launch_bounds__(NT) void k_bu_encode(const void *__restrict__ kv,
                                                  const float *__restrict__ gauges,
                                                  uint8_t *__restrict__ payload,
                                                  float *__restrict__ meta, QK a) {
  bu_encode_body<BITS, BF16, G>(kv, gauges, payload, meta, a);
}

// the same with three waves per SIMD (launched for the full-head gauge with
// bf16 storage below 8-bit codes, which fits in 168 VGPRs; other instances
// would spill)
template <int BITS, bool BF16, int G>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(3))) void k_bu_encode_w3(const void *__restrict__ kv,
                                                  const float *__restrict__ gauges,
                                                  uint8_t *__restrict__ payload,
                                                  float *__restrict__ meta, QK a) {
  bu_encode_body<BITS, BF16, G>(kv, gauges, payload, meta, a);
}

template <int BITS, bool BF16, int G>
__device__ __forceinline__ void bu_decode_body(const uint8_t *__restrict__ payload,
                                                  const float *__restrict__ meta,
                                                  const float *__restrict__ gauges,
                                                  void *__restrict__ out, QK a) {
  __shared__ __align__(16) unsigned char lds[LDS_TILE_BYTES];
  // dense gauge: (min, step) of each tile row and the column sums of the
  // inverse matrix, for the range applied after the product
  __shared__ __align__(16) float2 rowp[kDense<G, BF16> ? TILE_T : 1];
  __shared__ __align__(16) float csum[kDense<G, BF16> ? D : 1];
  float *xs = (float *)lds;
  const int64_t f = launch_field((int64_t)blockIdx.x / a.chunks, a.fsel, a.fstep, a.fbase);
  const int64_t chunk = (int64_t)blockIdx.x % a.chunks;
  const int64_t ntiles = (a.nt + TILE_T - 1) / TILE_T;
  const float *Gf = G ? gauges + gauge_index(f, a.batch, a.heads) * D * (G ? G : 1) : nullptr;
  G128Frags fr;
  if constexpr (kDense<G, BF16>) {
    load_g128_f16(Gf, fr);
    // inverse matrix B[k][n] = G[k][n]: column sums in a fixed order
    if (threadIdx.x < D) {
      float c = 0.0f;
      for (int k = 0; k < D; k++) c += Gf[k * D + threadIdx.x];
      csum[threadIdx.x] = c;
    }
  }
  TileGauge<kChainInv<G, BF16>, true> tg;
  SplitGaugeFrags<kSplitInv<G, BF16> ? G : 16> sg;
  if constexpr (kSplitInv<G, BF16>)
    load_split_gauge<G>(Gf, sg);
  else if constexpr (kChainInv<G, BF16> != 0)
    tg.load(Gf);
  const int BT = a.block;
  const int64_t nblk_f = a.tcap / BT;
  const int t = threadIdx.x >> 2, j = threadIdx.x & 3;
  const int64_t tile0 = chunk * a.tiles_per_chunk;
  const int64_t tend = min(ntiles, (chunk + 1) * a.tiles_per_chunk);
  // this thread's codes and range of a tile, loaded one tile ahead
  uint32_t wd[BITS];
  float mn = 0.0f, sc = 0.0f;
  auto fetch = [&](int64_t tile) {
    const int64_t tb = a.t0 + tile * TILE_T;
    if (t < tile_rows(a, tile)) {
      load_words<BITS>(payload + (size_t)(f * a.tcap + tb) * 16 * BITS + threadIdx.x * 4 * BITS, wd);
      const float *m = meta + 2 * (f * nblk_f + (tb + t) / BT);
      mn = m[0];
      sc = m[1];
    }
  };
  if (tile0 < tend) fetch(tile0);
  if constexpr (kDense<G, BF16>) {
    loads_done(wd);
    loads_done(mn);
    loads_done(sc);
  }
  ErrAcc err;
  for (int64_t tile = tile0; tile < tend; tile++) {
    const int64_t tb = a.t0 + tile * TILE_T;
    const int nrows = tile_rows(a, tile);
    const size_t off = (size_t)(f * a.tcap + tb) * D * (BF16 ? 2 : 4);
    if constexpr (kDense<G, BF16>) {
      // block-uniform ranges are one per block: (min + q step) G = step (q G) + min colsum(G),
      // and the codes (at most 8 bits) are exact fp16 values: one fp16 pass
      // (decode_tile_dense)
      uint32_t q[32];
      if (t < nrows) {
        unpack32<BITS>(wd, q);
      } else {
#pragma unroll
        for (int k = 0; k < 32; k++) q[k] = 0u;
      }
      uint16_t *sh = (uint16_t *)lds;
#pragma unroll
      for (int k4 = 0; k4 < 4; k4++) {
        uint32_t h[4];
#pragma unroll
        for (int e = 0; e < 4; e++)
          h[e] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(uint16_t)q[8 * k4 + 2 * e]) |
                 ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(uint16_t)q[8 * k4 + 2 * e + 1]) << 16);
        *(uint4 *)(sh + t * HP + 32 * j + 8 * k4) = make_uint4(h[0], h[1], h[2], h[3]);
      }
      if (j == 0) rowp[t] = t < nrows ? make_float2(mn, sc) : make_float2(0.0f, 0.0f);
      if (tile + 1 < tend) fetch(tile + 1);
      decode_tile_dense<true>(lds, fr, nullptr, rowp, csum, nrows, (uint8_t *)out + off,
                              a.ref ? (const uint8_t *)a.ref + off : nullptr, err,
                              [&] { loads_done(wd); loads_done(mn); loads_done(sc); });
    } else {
      float v[32];
      if (t < nrows) {
        uint32_t q[32];
        unpack32<BITS>(wd, q);
#pragma unroll
        for (int k = 0; k < 32; k++) v[k] = dequant1(q[k], mn, sc);
      } else {
#pragma unroll
        for (int k = 0; k < 32; k++) v[k] = 0.0f;
      }
      if (tile + 1 < tend) fetch(tile + 1);
      inverse_gauged_tile<G, BF16>(lds, t, j, v, nrows, tg, sg);
      if (a.ref)
        store_tile_err<BF16>((uint8_t *)out + off, nrows, xs, (const uint8_t *)a.ref + off, err);
      else
        store_tile<BF16>((uint8_t *)out + off, nrows, xs);
      __syncthreads();
    }
  }
  if (a.ref) write_err(err, a.epart);
}

template <int BITS, bool BF16, int G>
__global__ __launch_bounds__(NT) void k_bu_decode(const uint8_t *__restrict__ payload,
                                                  const float *__restrict__ meta,
                                                  const float *__restrict__ gauges,
                                                  void *__restrict__ out, QK a) {
  bu_decode_body<BITS, BF16, G>(payload, meta, gauges, out, a);
}

// the same with four waves per SIMD (launched for the full-head gauge with
// bf16 storage below 8-bit codes, which fits in 128 VGPRs)
template <int BITS, bool BF16, int G>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(4))) void k_bu_decode_w4(const uint8_t *__restrict__ payload,
                                                  const float *__restrict__ meta,
                                                  const float *__restrict__ gauges,
                                                  void *__restrict__ out, QK a) {
  bu_decode_body<BITS, BF16, G>(payload, meta, gauges, out, a);
}

// ---------------------------------------------------------------------------
// KIVI-style: keys one range per channel per 32 tokens, values one range per
// token per 32 channels; the last `residual` rows stay in the storage format.
// Field payload: codes of rows [0, Tcap - residual), then the tail rows.
// Metadata: 4 * (Tcap - residual) (mn, scale) pairs per field, keys indexed
// (row / 32) * 128 + channel, values row * 4 + channel / 32.
// ---------------------------------------------------------------------------

template <int BITS, bool BF16, int G>
__device__ __forceinline__ void kivi_encode_body(const void *__restrict__ kv,
                                                    const float *__restrict__ gauges,
                                                    uint8_t *__restrict__ payload,
                                                    float *__restrict__ meta, QK a) {
  __shared__ __align__(16) unsigned char lds[kEncLds<G, BF16>];
  float *xs = (float *)lds;
  // key column ranges of the tile's two 32-row groups (index 128 group +
  // channel): the minimum in pmn; the inverse step in the fp32 tile's row
  // padding (4 unused floats per row, exactly 256: kinv), 0 for a range that
  // quantizes everything to code 0 (then clamp(rint((x - min) * 0), 0, L) =
  // 0, as quant1 returns for it).  No flag array and no separate inverse
  // array: the full-head encoder keeps three workgroups per CU.
  __shared__ float pmn[2 * D];
  auto kinv = [&](int i) -> float & { return xs[(i >> 2) * PITCH + D + (i & 3)]; };
  constexpr int L = (1 << BITS) - 1;
  constexpr size_t ESZ = BF16 ? 2 : 4;
  const int64_t f = (int64_t)blockIdx.x / a.chunks;
  const int64_t chunk = (int64_t)blockIdx.x % a.chunks;
  const int64_t ntiles = (a.nt + TILE_T - 1) / TILE_T;
  const float *Gf = G ? gauges + gauge_index(f, a.batch, a.heads) * D * (G ? G : 1) : nullptr;
  G128Frags fr;
  if constexpr (kDense<G, BF16>) load_g128<false>(Gf, fr);
  TileGauge<G, false> tg;
  if constexpr (G != 0 && !kDense<G, BF16>) tg.load(Gf);
  const int64_t Tq = a.tokens - a.residual, Tcq = a.tcap - a.residual;
  const size_t Pf = (size_t)Tcq * 16 * BITS + (size_t)a.residual * D * ESZ;
  uint8_t *pf = payload + (size_t)f * Pf;
  float *mf = meta + 2 * (size_t)f * 4 * Tcq;
  const bool keys = ((f / ((int64_t)a.batch * a.heads)) % a.kv) == 0;
  const int t = threadIdx.x >> 2, j = threadIdx.x & 3;
  const uint8_t *src_f = (const uint8_t *)kv + (size_t)f * a.tcap * D * ESZ;
  const int64_t tile0 = chunk * a.tiles_per_chunk;
  const int64_t tend = min(ntiles, (chunk + 1) * a.tiles_per_chunk);
  GaugedTiles<G, BF16> tiles;
  if (tile0 < tend) tiles.prefetch(src_f + (size_t)(a.t0 + tile0 * TILE_T) * D * ESZ, tile_rows(a, tile0));
  tiles.arrived();
  for (int64_t tile = tile0; tile < tend; tile++) {
    const int64_t tb = a.t0 + tile * TILE_T;
    const int nrows = tile_rows(a, tile);
    tiles.next(src_f + (size_t)tb * D * ESZ, nrows, src_f + (size_t)(tb + TILE_T) * D * ESZ,
               tile + 1 < tend ? tile_rows(a, tile + 1) : 0, lds, tg, fr);
    // keys: this thread's column range (stored after the codes, so that no
    // store precedes the wait for the prefetched tile)
    const int gi = threadIdx.x >> 7, c = threadIdx.x & 127, r0 = 32 * gi;
    const bool kcol = keys && r0 < nrows && tb + r0 < Tq;
    Range krg{};
    if (keys) {
      if (kcol) {
        float mn = INFINITY, mx = -INFINITY;
        for (int r = 0; r < 32; r++) {
          const float x = xs[(r0 + r) * PITCH + c];
          mn = fminf(mn, x);
          mx = fmaxf(mx, x);
        }
        krg = make_range(mn, mx, L);
        pmn[threadIdx.x] = krg.mn;
        kinv(threadIdx.x) = krg.zero ? 0.0f : krg.inv;
      }
      __syncthreads();
    }
    tiles.arrived();
    if (t < nrows) {
      const int64_t row = tb + t;
      float v[32];
      read32(xs, t, j, v);
      if (row < Tq) {
        uint32_t q[32], wd[BITS];
        if (keys) {
          const int base = (t >> 5) * D + 32 * j;
#pragma unroll
          for (int k = 0; k < 32; k++) {
            Range rg;
            rg.mn = pmn[base + k];
            rg.inv = kinv(base + k);
            rg.zero = false;
            q[k] = quant1(v[k], rg, L);
          }
        } else {
          float mn = v[0], mx = v[0];
#pragma unroll
          for (int k = 1; k < 32; k++) {
            mn = fminf(mn, v[k]);
            mx = fmaxf(mx, v[k]);
          }
          const Range rg = make_range(mn, mx, L);
#pragma unroll
          for (int k = 0; k < 32; k++) q[k] = quant1(v[k], rg, L);
          float *m = mf + 2 * (row * 4 + j);
          m[0] = rg.mn;
          m[1] = rg.scale;
        }
        pack32<BITS>(q, wd);
        store_words<BITS>(pf + (size_t)row * 16 * BITS + j * 4 * BITS, wd);
      } else {
        store32_storage<BF16>(pf + (size_t)Tcq * 16 * BITS + ((size_t)(row - Tq) * D + 32 * j) * ESZ, v);
      }
    }
    if (kcol) {
      float *m = mf + 2 * (((tb + r0) / 32) * D + c);
      m[0] = krg.mn;
      m[1] = krg.scale;
    }
    if constexpr (!kDense<G, BF16>) __syncthreads();  // see GaugedTiles
  }
}

template <int BITS, bool BF16, int G>
__global__ __launch_bounds__(NT) void k_kivi_encode(const void *__restrict__ kv,
                                                    const float *__restrict__ gauges,
                                                    uint8_t *__restrict__ payload,
                                                    float *__restrict__ meta, QK a) {
  kivi_encode_body<BITS, BF16, G>(kv, gauges, payload, meta, a);
}

// the same with three waves per SIMD (launched for the full-head gauge with
// bf16 storage below 8-bit codes, which fits in 168 VGPRs; other instances
// would spill)
template <int BITS, bool BF16, int G>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(3))) void k_kivi_encode_w3(const void *__restrict__ kv,
                                                    const float *__restrict__ gauges,
                                                    uint8_t *__restrict__ payload,
                                                    float *__restrict__ meta, QK a) {
  kivi_encode_body<BITS, BF16, G>(kv, gauges, payload, meta, a);
}

template <int BITS, bool BF16, int G>
__device__ __forceinline__ void kivi_decode_body(const uint8_t *__restrict__ payload,
                                                    const float *__restrict__ meta,
                                                    const float *__restrict__ gauges,
                                                    void *__restrict__ out, QK a) {
  __shared__ __align__(16) unsigned char lds[LDS_TILE_BYTES];
  float *xs = (float *)lds;
  __shared__ float pmn[2 * D], psc[2 * D];
  constexpr size_t ESZ = BF16 ? 2 : 4;
  const int64_t f = launch_field((int64_t)blockIdx.x / a.chunks, a.fsel, a.fstep, a.fbase);
  const int64_t chunk = (int64_t)blockIdx.x % a.chunks;
  const int64_t ntiles = (a.nt + TILE_T - 1) / TILE_T;
  const float *Gf = G ? gauges + gauge_index(f, a.batch, a.heads) * D * (G ? G : 1) : nullptr;
  G128Frags fr;
  if constexpr (kDense<G, BF16>) load_g128_f16(Gf, fr);
  // dense gauge: the power-of-two row scales of the fp16 tile
  __shared__ __align__(16) float rsc[kDense<G, BF16> ? TILE_T : 1];
  TileGauge<kChainInv<G, BF16>, true> tg;
  SplitGaugeFrags<kSplitInv<G, BF16> ? G : 16> sg;
  if constexpr (kSplitInv<G, BF16>)
    load_split_gauge<G>(Gf, sg);
  else if constexpr (kChainInv<G, BF16> != 0)
    tg.load(Gf);
  const int64_t Tq = a.tokens - a.residual, Tcq = a.tcap - a.residual;
  const size_t Pf = (size_t)Tcq * 16 * BITS + (size_t)a.residual * D * ESZ;
  const uint8_t *pf = payload + (size_t)f * Pf;
  const float *mf = meta + 2 * (size_t)f * 4 * Tcq;
  const bool keys = ((f / ((int64_t)a.batch * a.heads)) % a.kv) == 0;
  const int t = threadIdx.x >> 2, j = threadIdx.x & 3;
  const int gi = threadIdx.x >> 7, c = threadIdx.x & 127, r0 = 32 * gi;
  const int64_t tile0 = chunk * a.tiles_per_chunk;
  const int64_t tend = min(ntiles, (chunk + 1) * a.tiles_per_chunk);
  // this thread's codes, its row's value range and (keys) one column range of
  // a tile, loaded one tile ahead; tail rows are read when they are used
  uint32_t wd[BITS];
  float mn = 0.0f, sc = 0.0f, kmn = 0.0f, ksc = 0.0f;
  auto fetch = [&](int64_t tile) {
    const int64_t tb = a.t0 + tile * TILE_T;
    const int nrows = tile_rows(a, tile);
    if (keys && r0 < nrows && tb + r0 < Tq) {
      const float *m = mf + 2 * (((tb + r0) / 32) * D + c);
      kmn = m[0];
      ksc = m[1];
    }
    const int64_t row = tb + t;
    if (t < nrows && row < Tq) {
      load_words<BITS>(pf + (size_t)row * 16 * BITS + j * 4 * BITS, wd);
      if (!keys) {
        const float *m = mf + 2 * (row * 4 + j);
        mn = m[0];
        sc = m[1];
      }
    }
  };
  if (tile0 < tend) fetch(tile0);
  if constexpr (kDense<G, BF16>) {
    loads_done(wd);
    loads_done(mn);
    loads_done(sc);
    loads_done(kmn);
    loads_done(ksc);
  }
  ErrAcc err;
  for (int64_t tile = tile0; tile < tend; tile++) {
    const int64_t tb = a.t0 + tile * TILE_T;
    const int nrows = tile_rows(a, tile);
    if (keys) {
      if (r0 < nrows && tb + r0 < Tq) {
        pmn[threadIdx.x] = kmn;
        psc[threadIdx.x] = ksc;
      }
      __syncthreads();
    }
    const size_t off = (size_t)(f * a.tcap + tb) * D * ESZ;
    float v[32];
    if (t < nrows) {
      const int64_t row = tb + t;
      if (row < Tq) {
        uint32_t q[32];
        unpack32<BITS>(wd, q);
        if (keys) {
          const int base = (t >> 5) * D + 32 * j;
#pragma unroll
          for (int k = 0; k < 32; k++) v[k] = dequant1(q[k], pmn[base + k], psc[base + k]);
        } else {
#pragma unroll
          for (int k = 0; k < 32; k++) v[k] = dequant1(q[k], mn, sc);
        }
      } else {
        load32_storage<BF16>(pf + (size_t)Tcq * 16 * BITS + ((size_t)(row - Tq) * D + 32 * j) * ESZ, v);
      }
    } else {
#pragma unroll
      for (int k = 0; k < 32; k++) v[k] = 0.0f;
    }
    if (tile + 1 < tend) fetch(tile + 1);
    if constexpr (kDense<G, BF16>) {
      // rows scaled into fp16 from their largest magnitude
      scaled_f16_32((uint16_t *)lds, rsc, t, j, v);
      decode_tile_dense<false>(lds, fr, rsc, nullptr, nullptr, nrows, (uint8_t *)out + off,
                               a.ref ? (const uint8_t *)a.ref + off : nullptr, err, [&] {
                                 loads_done(wd);
                                 loads_done(mn);
                                 loads_done(sc);
                                 loads_done(kmn);
                                 loads_done(ksc);
                               });
    } else {
      inverse_gauged_tile<G, BF16>(lds, t, j, v, nrows, tg, sg);
      if (a.ref)
        store_tile_err<BF16>((uint8_t *)out + off, nrows, xs, (const uint8_t *)a.ref + off, err);
      else
        store_tile<BF16>((uint8_t *)out + off, nrows, xs);
      __syncthreads();
    }
  }
  if (a.ref) write_err(err, a.epart);
}

template <int BITS, bool BF16, int G>
__global__ __launch_bounds__(NT) void k_kivi_decode(const uint8_t *__restrict__ payload,
                                                    const float *__restrict__ meta,
                                                    const float *__restrict__ gauges,
                                                    void *__restrict__ out, QK a) {
  kivi_decode_body<BITS, BF16, G>(payload, meta, gauges, out, a);
}

// the same with three waves per SIMD (launched for the full-head gauge with
// bf16 storage below 8-bit codes, which fits in 168 VGPRs; other instances
// would spill)
template <int BITS, bool BF16, int G>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(3))) void k_kivi_decode_w3(const uint8_t *__restrict__ payload,
                                                    const float *__restrict__ meta,
                                                    const float *__restrict__ gauges,
                                                    void *__restrict__ out, QK a) {
  kivi_decode_body<BITS, BF16, G>(payload, meta, gauges, out, a);
}

// dense-gauge rows kernel behind cg_gauge_apply(g = 128) with bf16 storage:
// same tiles, same fragments, same MFMA sequence as the fused quantizer
// kernels (fp32 storage uses the fmaf-chain rows kernel of the smaller groups)
template <bool BF16, bool INV>
__global__ __launch_bounds__(NT) void k_gauge128_rows(const void *__restrict__ src,
                                                      const float *__restrict__ gauges,
                                                      float *__restrict__ out, QK a) {
  __shared__ __align__(16) unsigned char lds[LDS_TILE_BYTES];
  float *xs = (float *)lds;
  uint16_t *sh = (uint16_t *)lds, *sl = sh + TILE_T * HP;
  constexpr size_t ESZ = BF16 ? 2 : 4;
  const int64_t f = (int64_t)blockIdx.x / a.chunks;
  const int64_t chunk = (int64_t)blockIdx.x % a.chunks;
  const int64_t ntiles = (a.nt + TILE_T - 1) / TILE_T;
  const float *Gf = gauges + gauge_index(f, a.batch, a.heads) * D * 128;
  G128Frags fr;
  load_g128<INV>(Gf, fr);
  const uint8_t *src_f = (const uint8_t *)src + (size_t)f * a.tcap * D * ESZ;
  const int64_t tile0 = chunk * a.tiles_per_chunk;
  const int64_t tend = min(ntiles, (chunk + 1) * a.tiles_per_chunk);
  TileFetch<BF16> pre;
  if (tile0 < tend) pre.fetch(src_f + (size_t)(a.t0 + tile0 * TILE_T) * D * ESZ, tile_rows(a, tile0));
  for (int64_t tile = tile0; tile < tend; tile++) {
    const int64_t tb = a.t0 + tile * TILE_T;
    const int nrows = tile_rows(a, tile);
    pre.put(sh, sl);
    __syncthreads();
    if (tile + 1 < tend) pre.fetch(src_f + (size_t)(tb + TILE_T) * D * ESZ, tile_rows(a, tile + 1));
    gauge128_tile<BF16, BF16 && !INV>(sh, sl, xs, fr);
    store_tile<false>(out + (size_t)(f * a.tcap + tb) * D, nrows, xs);
    __syncthreads();
  }
}

}  // namespace cgq
