// Fused gauge + zfp-style fixed-rate encode, and fused decode + inverse gauge
// ("Codec-Gauge", arXiv HTML, evaluation-protocol paragraph: the gauged FP32
// tensor is zfp-encoded at a fixed rate as a 2D field with n_x = d_l, decoded,
// and the inverse gauge restores the cache before attention).
//
// A tile is 64 tokens x 128 channels of one field: 16 block rows x 32 blocks =
// 512 blocks, whose 16R-bit codes are one contiguous 1024R-byte span of the
// stream.  A workgroup (256 threads) walks a chunk of consecutive tiles of one
// field, loading tile i+1 into registers while it works on tile i:
//   encode: coalesced tile load -> LDS (fp32) -> gauge in place (TileGauge:
//           matrix-core fmaf chains for g = 16/32 and, with fp32 storage,
//           g = 128; VALU for g = 8; the split-precision bf16 MFMA routine
//           for g = 128 with bf16 storage)
//           -> one block per thread-iteration (zfp_block.hpp, all in VGPRs)
//           -> codes staged in LDS -> coalesced 16-byte stores of the span.
//   decode: the mirror image; with a reference pointer the store also
//           accumulates the cache-side error sums.
// Stream layout: field f, block (bx, by) (bx = channel block, fastest) sits at
// bits [((f * Tcap/4 + by) * 32 + bx) * 16R, +16R), stream bit p = bit p%8 of
// byte p/8 -- the pages' whole-tensor 2D field with the fields in order,
// since no 4x4 block straddles two fields (Tcap % 4 == 0).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cg_launch.hpp"
#include "cg_tile.hpp"
#include "gauge128.hpp"
#include "split_gauge.hpp"
#include "zfp_block.hpp"

namespace cgk {

// write the 16R bits of block b into the LDS stream image (halfword granular)
template <int R>
__device__ __forceinline__ void stage_block(uint32_t *os, int b, const uint64_t (&acc)[cgz::Rate<R>::kAcc]) {
  if constexpr (R % 2 == 0) {
    uint32_t *d = os + b * (R / 2);
#pragma unroll
    for (int h = 0; h < R / 2; h++) d[h] = (uint32_t)(acc[h / 2] >> (32 * (h % 2)));
  } else {
    uint16_t *d = (uint16_t *)os + b * R;
#pragma unroll
    for (int h = 0; h < R; h++) d[h] = (uint16_t)(acc[h / 4] >> (16 * (h % 4)));
  }
}

template <int R>
__device__ __forceinline__ void unstage_block(const uint32_t *os, int b, uint64_t (&acc)[cgz::Rate<R>::kAcc]) {
#pragma unroll
  for (int a = 0; a < cgz::Rate<R>::kAcc; a++) acc[a] = 0;
  if constexpr (R % 2 == 0) {
    const uint32_t *s = os + b * (R / 2);
#pragma unroll
    for (int h = 0; h < R / 2; h++) acc[h / 2] |= (uint64_t)s[h] << (32 * (h % 2));
  } else {
    const uint16_t *s = (const uint16_t *)os + b * R;
#pragma unroll
    for (int h = 0; h < R; h++) acc[h / 4] |= (uint64_t)s[h] << (16 * (h % 4));
  }
}

// Even rates: a block's 16R bits are R/2 aligned 32-bit words, so a lane
// loads or stores its own block's code directly (the 64 lanes of a wave touch
// 64 consecutive blocks: one contiguous span).  Odd rates stage through LDS.
template <int R>
struct BlockCode {
  static constexpr bool kDirect = R % 2 == 0 && R <= 8;
  static constexpr int NW = kDirect ? R / 2 : 1;
  uint32_t w[NW];
  __device__ __forceinline__ void load(const uint8_t *__restrict__ p) {
    const uint32_t *q = (const uint32_t *)p;
    if constexpr (NW == 1) {
      w[0] = q[0];
    } else if constexpr (NW == 2) {
      const uint2 t = *(const uint2 *)q;
      w[0] = t.x; w[1] = t.y;
    } else if constexpr (NW == 3) {
      const uint3 t = *(const uint3 *)q;
      w[0] = t.x; w[1] = t.y; w[2] = t.z;
    } else {
      const uint4 t = *(const uint4 *)q;
      w[0] = t.x; w[1] = t.y; w[2] = t.z; w[3] = t.w;
    }
  }
  __device__ __forceinline__ void to_acc(uint64_t (&acc)[cgz::Rate<R>::kAcc]) const {
#pragma unroll
    for (int a = 0; a < cgz::Rate<R>::kAcc; a++) acc[a] = 0;
#pragma unroll
    for (int h = 0; h < NW; h++) acc[h / 2] |= (uint64_t)w[h] << (32 * (h % 2));
  }
};

template <int R>
__device__ __forceinline__ void store_block_code(uint8_t *__restrict__ p,
                                                 const uint64_t (&acc)[cgz::Rate<R>::kAcc]) {
  constexpr int NW = R / 2;
  uint32_t w[NW];
#pragma unroll
  for (int h = 0; h < NW; h++) w[h] = (uint32_t)(acc[h / 2] >> (32 * (h % 2)));
  uint32_t *q = (uint32_t *)p;
  if constexpr (NW == 1) q[0] = w[0];
  else if constexpr (NW == 2) *(uint2 *)q = make_uint2(w[0], w[1]);
  else if constexpr (NW == 3) *(uint3 *)q = make_uint3(w[0], w[1], w[2]);
  else *(uint4 *)q = make_uint4(w[0], w[1], w[2], w[3]);
}

// Lifted reconstruction on the matrix cores (zfp_block.hpp, "Lifted
// reconstruction"): one v_mfma_i32_32x32x32_i8 per wave computes A d for the
// wave's 64 blocks.  B operand: lane l = (n = l % 32, g = l / 32) gives its
// own block's 16 digit bytes as k-group g.  Result D[m][n] lands in lane
// n + 32 ((m >> 2) & 1), register (m >> 3) * 4 + (m & 3); rows m with
// ((m >> 2) & 1) == g take block (n, g)'s coefficients, as output
// p = ((m >> 3) << 2) | (m & 3), so each lane receives its own block's 16
// values with register r = output position r.  A operand: lane l holds row
// m = l % 32, k-group l / 32.
typedef int cg_v4i __attribute__((ext_vector_type(4)));
typedef int cg_v16i __attribute__((ext_vector_type(16)));

struct LiftRows {
  uint32_t w[16][4];  // row p of A as 16 int8, k = 4 * word + byte
};

__host__ __device__ constexpr LiftRows make_lift_rows() {
  LiftRows t{};
  for (int p = 0; p < 16; p++)
    for (int k = 0; k < 16; k++)
      t.w[p][k >> 2] |= (uint32_t)(uint8_t)cgz::kLift.a[p][k] << (8 * (k & 3));
  return t;
}

__constant__ LiftRows kLiftRows = make_lift_rows();

__device__ __forceinline__ cg_v4i lift_operand() {
  const int l = threadIdx.x & 63, m = l & 31;
  const bool mine = (l >> 5) == ((m >> 2) & 1);
  const int p = ((m >> 3) << 2) | (m & 3);
  cg_v4i a;
#pragma unroll
  for (int j = 0; j < 4; j++) a[j] = mine ? (int)kLiftRows.w[p][j] : 0;
  return a;
}

// Wave-uniform: false unless every lane's block takes the lifted
// reconstruction; then v holds the block's 16 values (v[4j + i]: token row
// j, channel i).  Called with all 64 lanes active.
template <int R>
__device__ __forceinline__ bool lifted_tail(const cg_v4i &liftA, const cgz::BlockParse<R> &st,
                                            float (&v)[16]) {
  const cgz::LiftScale ls = cgz::lift_scale<R>(st);
  if (cgz::wave_any(!ls.ok)) return false;
  uint32_t T[4];
  cgz::plane_bytes(st.Z, st.s, T);
  cg_v4i B;
#pragma unroll
  for (int j = 0; j < 4; j++) B[j] = (int)(T[j] ^ 0x80808080u);
  cg_v16i C;
#pragma unroll
  for (int r = 0; r < 16; r++) C[r] = cgz::kLiftMagic + ls.beta * cgz::kLift.rowsum[r];
  const cg_v16i D = __builtin_amdgcn_mfma_i32_32x32x32_i8(liftA, B, C, 0, 0, 0);
  float mx = 0.f;
#pragma unroll
  for (int r = 0; r < 16; r++) {
    v[r] = fmaf(__int_as_float(D[r]), ls.scale, ls.offset);
    mx = fmaxf(mx, fabsf(v[r]));
  }
  return !cgz::wave_any(!(mx < ls.limit));
}

// Gauges g <= 32: a workgroup walks a.chunk_tiles consecutive tiles of
// one field and loads tile i+1 (KV rows, or code words) into registers while
// it codes tile i.
// A partial last block row (nrows % 4 != 0, only at the end of a field's
// valid tokens) is completed by repeating the tile's last valid row.  The
// gauge acts on each row alone, so padding the gauged rows equals padding
// the inputs.  The decoder stores the valid rows only.
__device__ __forceinline__ void pad_block_row(float *xs, int nrows) {
  const int pad = (4 - (nrows & 3)) & 3;
  for (int i = threadIdx.x; i < pad * 32; i += NT)
    *(float4 *)(xs + (nrows + (i >> 5)) * PITCH + (i & 31) * 4) =
        *(const float4 *)(xs + (nrows - 1) * PITCH + (i & 31) * 4);
}

template <int R, bool BF16, int G>
__global__ __launch_bounds__(NT) void k_zfp_encode(const void *__restrict__ kv,
                                                   const float *__restrict__ gauges,
                                                   uint8_t *__restrict__ payload, TileArgs a) {
  __shared__ float xs[TILE_T * PITCH];
  __shared__ uint32_t os[TILE_T / 4 * 32 * R / 2];
  __shared__ cgz::PlaneTables tab;
  const int64_t field = (int64_t)blockIdx.x / a.chunks;
  const int tile0 = (int)((int64_t)blockIdx.x % a.chunks) * a.chunk_tiles;
  const int tend = min(a.tiles, tile0 + a.chunk_tiles);
  const size_t esz = BF16 ? 2 : 4;
  TileGauge<G, false> tg;
  if constexpr (G != 0) tg.load(gauges + gauge_index(field, a.batch, a.heads) * D * G);
  cgz::plane_tables_entry(tab, threadIdx.x);
  const uint8_t *src_f = (const uint8_t *)kv + (size_t)field * a.tcap * D * esz;
  auto rows = [&](int tile) { return (int)min((int64_t)TILE_T, a.nt - (int64_t)tile * TILE_T); };
  TileFetch<BF16> pre;
  if (tile0 < tend) pre.fetch(src_f + (size_t)(a.t0 + (int64_t)tile0 * TILE_T) * D * esz, rows(tile0));
  for (int tile = tile0; tile < tend; tile++) {
    const int64_t tb = a.t0 + (int64_t)tile * TILE_T;
    const int nrows = rows(tile);
    pre.put_f32(xs);
    __syncthreads();
    if (tile + 1 < tend) pre.fetch(src_f + (size_t)(tb + TILE_T) * D * esz, rows(tile + 1));
    if constexpr (G != 0) {
      tg.apply(xs, nrows);
      __syncthreads();
    }
    if (nrows & 3) {
      pad_block_row(xs, nrows);
      __syncthreads();
    }
    const int nblk = ((nrows + 3) / 4) * 32;
    uint8_t *dst = payload + (size_t)(field * (a.tcap / 4) + tb / 4) * 32 * 2 * R;
    for (int b = threadIdx.x; b < nblk; b += NT) {
      const float *src = xs + (b >> 5) * 4 * PITCH + (b & 31) * 4;
      float v[16];
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const float4 t = *(const float4 *)(src + j * PITCH);
        v[4 * j] = t.x; v[4 * j + 1] = t.y; v[4 * j + 2] = t.z; v[4 * j + 3] = t.w;
      }
      uint64_t acc[cgz::Rate<R>::kAcc];
      cgz::encode_block<R>(v, acc, tab);
      if constexpr (BlockCode<R>::kDirect)
        store_block_code<R>(dst + (size_t)b * 2 * R, acc);
      else
        stage_block<R>(os, b, acc);
    }
    __syncthreads();  // every thread is done with xs (and the codes are staged)
    if constexpr (!BlockCode<R>::kDirect) {
      const int n16 = nblk * 2 * R / 16;
      for (int i = threadIdx.x; i < n16; i += NT) ((uint4 *)dst)[i] = ((const uint4 *)os)[i];
    }
  }
}

// the code words of one tile held in registers between their global load
// and their LDS store (16-B pieces i, i + NT, ...)
template <int R>
struct CodeFetch {
  static constexpr int NC = (TILE_T / 4 * 32 * 2 * R / 16 + NT - 1) / NT;
  uint4 r[NC];
  __device__ __forceinline__ void fetch(const uint4 *__restrict__ src, int n16) {
#pragma unroll
    for (int k = 0; k < NC; k++) {
      const int i = threadIdx.x + NT * k;
      if (i < n16) r[k] = src[i];
    }
  }
  __device__ __forceinline__ void put(uint32_t *os, int n16) const {
#pragma unroll
    for (int k = 0; k < NC; k++) {
      const int i = threadIdx.x + NT * k;
      if (i < n16) ((uint4 *)os)[i] = r[k];
    }
  }
};

template <int R, bool BF16, int G>
__global__ __launch_bounds__(NT) void k_zfp_decode(const uint8_t *__restrict__ payload,
                                                   const float *__restrict__ gauges,
                                                   void *__restrict__ out, TileArgs a) {
  __shared__ float xs[TILE_T * PITCH];
  __shared__ uint32_t os[TILE_T / 4 * 32 * R / 2];
  const int64_t field = launch_field((int64_t)blockIdx.x / a.chunks, a.fsel, a.fstep, a.fbase);
  const int tile0 = (int)((int64_t)blockIdx.x % a.chunks) * a.chunk_tiles;
  const int tend = min(a.tiles, tile0 + a.chunk_tiles);
  const size_t esz = BF16 ? 2 : 4;
  // bf16 storage, g = 16 / 32: split-precision bf16 matrix cores; otherwise
  // the fp32 fmaf-chain form (or nothing, g = 0)
  constexpr bool kSplit = BF16 && (G == 16 || G == 32);
  TileGauge<kSplit ? 0 : G, true> tg;
  SplitGaugeFrags<kSplit ? G : 16> sg;
  if constexpr (kSplit)
    load_split_gauge<G>(gauges + gauge_index(field, a.batch, a.heads) * D * G, sg);
  else if constexpr (G != 0)
    tg.load(gauges + gauge_index(field, a.batch, a.heads) * D * G);
  auto rows = [&](int tile) { return (int)min((int64_t)TILE_T, a.nt - (int64_t)tile * TILE_T); };
  auto codes = [&](int tile) {
    return (const uint4 *)(payload + (size_t)(field * (a.tcap / 4) + (a.t0 + (int64_t)tile * TILE_T) / 4) * 32 * 2 * R);
  };
  auto n16 = [&](int tile) { return ((rows(tile) + 3) / 4) * 32 * 2 * R / 16; };
  auto nblocks = [&](int tile) { return ((rows(tile) + 3) / 4) * 32; };
  constexpr bool kDirect = BlockCode<R>::kDirect;
  constexpr int BPT = TILE_T / 4 * 32 / NT;   // blocks per thread and tile
  CodeFetch<R> pre;                            // odd rates: the tile's code words
  BlockCode<R> pc[BPT];                        // even rates: this thread's blocks
  auto fetch = [&](int tile) {
    if constexpr (kDirect) {
      const uint8_t *c = (const uint8_t *)codes(tile);
      const int nb = nblocks(tile);
#pragma unroll
      for (int i = 0; i < BPT; i++) {
        const int b = threadIdx.x + NT * i;
        if (b < nb) pc[i].load(c + (size_t)b * 2 * R);
      }
    } else {
      pre.fetch(codes(tile), n16(tile));
    }
  };
  if (tile0 < tend) fetch(tile0);
  const cg_v4i liftA = lift_operand();
  const cgz::ParseConsts kc = cgz::parse_consts();
  ErrAcc err;
  for (int tile = tile0; tile < tend; tile++) {
    const int64_t tb = a.t0 + (int64_t)tile * TILE_T;
    const int nrows = rows(tile);
    const int nblk = ((nrows + 3) / 4) * 32;
    BlockCode<R> cur[BPT];
    if constexpr (kDirect) {
#pragma unroll
      for (int i = 0; i < BPT; i++) cur[i] = pc[i];
    } else {
      pre.put(os, n16(tile));
      __syncthreads();
    }
    if (tile + 1 < tend) fetch(tile + 1);
    // every lane takes part (the lifted reconstruction is a wave-wide
    // product): lanes past the tile's blocks decode an empty block into
    // rows the gauge and the store do not read
#pragma unroll
    for (int i = 0; i < BPT; i++) {
      const int b = threadIdx.x + NT * i;
      uint64_t acc[cgz::Rate<R>::kAcc];
      if constexpr (kDirect)
        cur[i].to_acc(acc);
      else
        unstage_block<R>(os, b, acc);
      if (b >= nblk) {
#pragma unroll
        for (int a2 = 0; a2 < cgz::Rate<R>::kAcc; a2++) acc[a2] = 0;
      }
      cgz::BlockParse<R> st;
      cgz::decode_planes8<R>(acc, st, kc);
      float v[16];
      if (!lifted_tail<R>(liftA, st, v)) cgz::decode_finish<R>(acc, st, v, kc);
      if constexpr (kSplit) {
#pragma unroll
        for (int j = 0; j < 4; j++)
          split_store4((unsigned char *)xs, (b >> 5) * 4 + j, (b & 31) * 4, v[4 * j], v[4 * j + 1],
                       v[4 * j + 2], v[4 * j + 3]);
      } else {
        float *dst = xs + (b >> 5) * 4 * PITCH + (b & 31) * 4;
#pragma unroll
        for (int j = 0; j < 4; j++)
          *(float4 *)(dst + j * PITCH) = make_float4(v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]);
      }
    }
    __syncthreads();
    if constexpr (kSplit) {
      gauge_tile_split<G>((unsigned char *)xs, nrows, sg);
      __syncthreads();
    } else if constexpr (G != 0) {
      tg.apply(xs, nrows);
      __syncthreads();
    }
    const size_t off = (size_t)(field * a.tcap + tb) * D * esz;
    if (a.ref)
      store_tile_err<BF16>((uint8_t *)out + off, nrows, xs, (const uint8_t *)a.ref + off, err);
    else
      store_tile<BF16>((uint8_t *)out + off, nrows, xs);
    __syncthreads();  // xs (and os) are rewritten by the next tile
  }
  if (a.ref) write_err(err, a.epart);
}

// Dense (g = 128) gauge with bf16 storage on the bf16 matrix cores
// (gauge128.hpp, split precision): a workgroup walks ZFP128_CHUNK
// consecutive tiles of one field so the 64 KB gauge is turned into VGPR
// fragments once, and loads tile i+1 (KV rows, or code words) while it works
// on tile i.  (fp32 storage takes the fp32 fmaf-chain gauge of k_zfp_encode /
// k_zfp_decode instead.)
template <int R, bool BF16>
__global__ __launch_bounds__(NT) void k_zfp_encode128(const void *__restrict__ kv,
                                                      const float *__restrict__ gauges,
                                                      uint8_t *__restrict__ payload, TileArgs a) {
  __shared__ __align__(16) unsigned char lds[LDS_TILE_BYTES];
  __shared__ uint32_t os[TILE_T / 4 * 32 * R / 2];
  __shared__ cgz::PlaneTables tab;
  float *xs = (float *)lds;
  uint16_t *sh = (uint16_t *)lds, *sl = sh + TILE_T * HP;
  const int64_t field = (int64_t)blockIdx.x / a.chunks;
  const int tile0 = (int)((int64_t)blockIdx.x % a.chunks) * ZFP128_CHUNK;
  const int tend = min(a.tiles, tile0 + ZFP128_CHUNK);
  const size_t esz = BF16 ? 2 : 4;
  cgz::plane_tables_entry(tab, threadIdx.x);
  G128Frags fr;
  load_g128<false>(gauges + gauge_index(field, a.batch, a.heads) * D * 128, fr);
  const uint8_t *src_f = (const uint8_t *)kv + (size_t)field * a.tcap * D * esz;
  auto rows = [&](int tile) { return (int)min((int64_t)TILE_T, a.nt - (int64_t)tile * TILE_T); };
  TileFetch<BF16> pre;
  if (tile0 < tend) pre.fetch(src_f + (size_t)(a.t0 + (int64_t)tile0 * TILE_T) * D * esz, rows(tile0));
  for (int tile = tile0; tile < tend; tile++) {
    const int64_t tb = a.t0 + (int64_t)tile * TILE_T;
    const int nrows = rows(tile);
    pre.put(sh, sl);
    __syncthreads();
    if (tile + 1 < tend) pre.fetch(src_f + (size_t)(tb + TILE_T) * D * esz, rows(tile + 1));
    gauge128_tile<BF16, BF16>(sh, sl, xs, fr);
    if (nrows & 3) {
      pad_block_row(xs, nrows);
      __syncthreads();
    }
    const int nblk = ((nrows + 3) / 4) * 32;
    uint8_t *dst = payload + (size_t)(field * (a.tcap / 4) + tb / 4) * 32 * 2 * R;
    for (int b = threadIdx.x; b < nblk; b += NT) {
      const float *src = xs + (b >> 5) * 4 * PITCH + (b & 31) * 4;
      float v[16];
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const float4 t = *(const float4 *)(src + j * PITCH);
        v[4 * j] = t.x; v[4 * j + 1] = t.y; v[4 * j + 2] = t.z; v[4 * j + 3] = t.w;
      }
      uint64_t acc[cgz::Rate<R>::kAcc];
      cgz::encode_block<R>(v, acc, tab);
      if constexpr (BlockCode<R>::kDirect)
        store_block_code<R>(dst + (size_t)b * 2 * R, acc);
      else
        stage_block<R>(os, b, acc);
    }
    __syncthreads();  // every thread is done with xs (and the codes are staged)
    if constexpr (!BlockCode<R>::kDirect) {
      const int n16 = nblk * 2 * R / 16;
      for (int i = threadIdx.x; i < n16; i += NT) ((uint4 *)dst)[i] = ((const uint4 *)os)[i];
    }
  }
}

template <int R, bool BF16>
__global__ __launch_bounds__(NT) void k_zfp_decode128(const uint8_t *__restrict__ payload,
                                                      const float *__restrict__ gauges,
                                                      void *__restrict__ out, TileArgs a) {
  __shared__ __align__(16) unsigned char lds[LDS_TILE_BYTES];
  __shared__ uint32_t os[TILE_T / 4 * 32 * R / 2];
  constexpr int NC = (TILE_T / 4 * 32 * 2 * R / 16 + NT - 1) / NT;  // 16-B code pieces per thread
  float *xs = (float *)lds;
  uint16_t *sh = (uint16_t *)lds, *sl = sh + TILE_T * HP;
  const int64_t field = launch_field((int64_t)blockIdx.x / a.chunks, a.fsel, a.fstep, a.fbase);
  const int tile0 = (int)((int64_t)blockIdx.x % a.chunks) * ZFP128_CHUNK;
  const int tend = min(a.tiles, tile0 + ZFP128_CHUNK);
  const size_t esz = BF16 ? 2 : 4;
  G128Frags fr;
  load_g128<true>(gauges + gauge_index(field, a.batch, a.heads) * D * 128, fr);
  auto rows = [&](int tile) { return (int)min((int64_t)TILE_T, a.nt - (int64_t)tile * TILE_T); };
  auto codes = [&](int tile) {
    return (const uint4 *)(payload + (size_t)(field * (a.tcap / 4) + (a.t0 + (int64_t)tile * TILE_T) / 4) * 32 * 2 * R);
  };
  uint4 pre[NC];
  auto fetch = [&](int tile) {
    const uint4 *src = codes(tile);
    const int n16 = ((rows(tile) + 3) / 4) * 32 * 2 * R / 16;
#pragma unroll
    for (int k = 0; k < NC; k++) {
      const int i = threadIdx.x + NT * k;
      if (i < n16) pre[k] = src[i];
    }
  };
  if (tile0 < tend) fetch(tile0);
  const cg_v4i liftA = lift_operand();
  const cgz::ParseConsts kc = cgz::parse_consts();
  ErrAcc err;
  for (int tile = tile0; tile < tend; tile++) {
    const int64_t tb = a.t0 + (int64_t)tile * TILE_T;
    const int nrows = rows(tile);
    const int nblk = ((nrows + 3) / 4) * 32;
    const int n16 = nblk * 2 * R / 16;
#pragma unroll
    for (int k = 0; k < NC; k++) {
      const int i = threadIdx.x + NT * k;
      if (i < n16) ((uint4 *)os)[i] = pre[k];
    }
    __syncthreads();
    if (tile + 1 < tend) fetch(tile + 1);
    // decoded blocks go straight into the split operand tiles; every lane
    // takes part (the lifted reconstruction is a wave-wide product), lanes
    // past the tile's blocks decode an empty block into rows that are not
    // stored (output rows depend on their own row only)
#pragma unroll
    for (int i = 0; i < TILE_T / 4 * 32 / NT; i++) {
      const int b = threadIdx.x + NT * i;
      uint64_t acc[cgz::Rate<R>::kAcc];
      unstage_block<R>(os, b, acc);
      if (b >= nblk) {
#pragma unroll
        for (int a2 = 0; a2 < cgz::Rate<R>::kAcc; a2++) acc[a2] = 0;
      }
      cgz::BlockParse<R> st;
      cgz::decode_planes8<R>(acc, st, kc);
      float v[16];
      if (!lifted_tail<R>(liftA, st, v)) cgz::decode_finish<R>(acc, st, v, kc);
      const int off = (b >> 5) * 4 * HP + (b & 31) * 4;
#pragma unroll
      for (int j = 0; j < 4; j++) {
        uint2 h, l;
        split_pair(v[4 * j], v[4 * j + 1], h.x, l.x);
        split_pair(v[4 * j + 2], v[4 * j + 3], h.y, l.y);
        *(uint2 *)(sh + off + j * HP) = h;
        *(uint2 *)(sl + off + j * HP) = l;
      }
    }
    __syncthreads();
    gauge128_tile<false>(sh, sl, xs, fr);
    const size_t off = (size_t)(field * a.tcap + tb) * D * esz;
    if (a.ref)
      store_tile_err<BF16>((uint8_t *)out + off, nrows, xs, (const uint8_t *)a.ref + off, err);
    else
      store_tile<BF16>((uint8_t *)out + off, nrows, xs);
    __syncthreads();
  }
  if (a.ref) write_err(err, a.epart);
}

// all launches of one rate R (encode or decode, storage format, group size)
template <int R>
hipError_t zfp_launch_rate(bool encode, bool bf16, int g, const void *src, const float *gauges,
                           void *dst, const TileArgs &a, hipStream_t s) {
  const dim3 block(NT);
  const int64_t fields = a.grid / a.tiles;
  TileArgs v = a;
  v.chunk_tiles = zfp_chunk_tiles(fields, a.tiles);
  v.chunks = (a.tiles + v.chunk_tiles - 1) / v.chunk_tiles;
  const dim3 grid((unsigned)(fields * v.chunks));
#define CG_L(BF, GG)                                                                             \
  if (bf16 == BF && g == GG) {                                                                   \
    if (encode)                                                                                  \
      hipLaunchKernelGGL((k_zfp_encode<R, BF, GG>), grid, block, 0, s, src, gauges,             \
                         (uint8_t *)dst, v);                                                     \
    else                                                                                         \
      hipLaunchKernelGGL((k_zfp_decode<R, BF, GG>), grid, block, 0, s, (const uint8_t *)src,    \
                         gauges, dst, v);                                                        \
    return hipGetLastError();                                                                    \
  }
  CG_L(true, 0) CG_L(true, 8) CG_L(true, 16) CG_L(true, 32)
  CG_L(false, 0) CG_L(false, 8) CG_L(false, 16) CG_L(false, 32)
  // fp32 storage, full-head gauge: fp32 matrix-core fmaf chains (exact
  // reading order), in the same kernels as the grouped gauges
  CG_L(false, 128)
#undef CG_L
  if (g == 128 && bf16) {
    TileArgs c = a;
    c.chunks = (a.tiles + ZFP128_CHUNK - 1) / ZFP128_CHUNK;
    c.chunk_tiles = ZFP128_CHUNK;
    const dim3 grid128((unsigned)(fields * c.chunks));
#define CG_L128(BF)                                                                              \
  if (bf16 == BF) {                                                                              \
    if (encode)                                                                                  \
      hipLaunchKernelGGL((k_zfp_encode128<R, BF>), grid128, block, 0, s, src, gauges,           \
                         (uint8_t *)dst, c);                                                     \
    else                                                                                         \
      hipLaunchKernelGGL((k_zfp_decode128<R, BF>), grid128, block, 0, s, (const uint8_t *)src,  \
                         gauges, dst, c);                                                        \
    return hipGetLastError();                                                                    \
  }
    CG_L128(true)
#undef CG_L128
  }
  return hipErrorInvalidValue;
}

}  // namespace cgk
