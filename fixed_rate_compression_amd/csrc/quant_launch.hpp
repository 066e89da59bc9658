// Per-bit-width launcher of the quantizer kernels (included by quant_b<bits>.hip).
#pragma once

#include "quant_kernels.hpp"

namespace cgq {

inline QK make_qk(const QuantArgs &q, int tiles_per_chunk) {
  QK a{};
  a.tcap = q.tcap;
  a.tokens = q.tokens;
  a.t0 = q.t0;
  a.nt = q.nt;
  const int64_t ntiles = (q.nt + TILE_T - 1) / TILE_T;
  a.tiles_per_chunk = tiles_per_chunk;
  a.chunks = (ntiles + tiles_per_chunk - 1) / tiles_per_chunk;
  a.batch = q.batch;
  a.heads = q.heads;
  a.kv = q.kv;
  a.block = q.block;
  a.residual = q.residual;
  a.ref = q.ref;
  a.epart = q.epart;
  a.fsel = q.fsel;
  a.fstep = q.fstep;
  a.fbase = q.fbase;
  return a;
}



template <int BITS>
hipError_t quant_launch_bits(bool encode, bool bf16, int g, int backend, const void *src,
                             const float *gauges, void *dst, const void *meta_in, float *meta_out,
                             const QuantArgs &q, hipStream_t s) {
  const QK a = make_qk(q, quant_chunk_tiles(g, q.fields, (q.nt + TILE_T - 1) / TILE_T));
  const dim3 grid((unsigned)(q.fields * a.chunks)), block(NT);
  const bool bu = backend == 2;
  // BE, BD, KE, KD: the instance suffixes of the block-uniform encoder and
  // decoder and the KIVI-style encoder and decoder (_w3 / _w4: three / four
  // waves per SIMD)
#define CG_Q(BF, GG, BE, BD, KE, KD)                                                                 \
  if (bf16 == BF && g == GG) {                                                                       \
    if (bu && encode)                                                                                \
      hipLaunchKernelGGL((k_bu_encode##BE<BITS, BF, GG>), grid, block, 0, s, src, gauges,           \
                         (uint8_t *)dst, meta_out, a);                                               \
    else if (bu)                                                                                     \
      hipLaunchKernelGGL((k_bu_decode##BD<BITS, BF, GG>), grid, block, 0, s, (const uint8_t *)src,  \
                         (const float *)meta_in, gauges, dst, a);                                    \
    else if (encode)                                                                                 \
      hipLaunchKernelGGL((k_kivi_encode##KE<BITS, BF, GG>), grid, block, 0, s, src, gauges,         \
                         (uint8_t *)dst, meta_out, a);                                               \
    else                                                                                             \
      hipLaunchKernelGGL((k_kivi_decode##KD<BITS, BF, GG>), grid, block, 0, s, (const uint8_t *)src,\
                         (const float *)meta_in, gauges, dst, a);                                    \
    return hipGetLastError();                                                                        \
  }
  CG_Q(true, 0, , , , ) CG_Q(true, 8, , , , ) CG_Q(true, 16, , , , ) CG_Q(true, 32, , , , )
  // full-head gauge with bf16 storage: the instances with more waves per SIMD
  // fit their registers below 8-bit codes
  if constexpr (BITS < 8) {
    CG_Q(true, 128, _w3, _w4, _w3, _w3)
  } else {
    CG_Q(true, 128, , , , )
  }
  CG_Q(false, 0, , , , ) CG_Q(false, 8, , , , ) CG_Q(false, 16, , , , ) CG_Q(false, 32, , , , )
  CG_Q(false, 128, , , , )
#undef CG_Q
  return hipErrorInvalidValue;
}

}  // namespace cgq
