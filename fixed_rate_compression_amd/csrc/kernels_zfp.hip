// Dispatch of the fused zfp-style kernels (zfp_kernels.hpp) and of the
// gauge-only rows kernel.  Each rate's kernels are instantiated in their own
// translation unit (zfp_r<R>.hip) so the library builds in parallel.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cg_launch.hpp"
#include "cg_tile.hpp"

namespace cgk {

template <int R>
hipError_t zfp_launch_rate(bool encode, bool bf16, int g, const void *src, const float *gauges,
                           void *dst, const TileArgs &a, hipStream_t s);

#define CG_ZFP_RATES(X) X(2) X(3) X(4) X(6) X(8)

bool zfp_rate_built(int R) {
  switch (R) {
#define CASE(r) case r: return true;
    CG_ZFP_RATES(CASE)
#undef CASE
  }
  return false;
}

static hipError_t zfp_launch(int R, bool encode, bool bf16, int g, const void *src,
                             const float *gauges, void *dst, const TileArgs &a, hipStream_t s) {
  if (g != 0 && g != 8 && g != 16 && g != 32 && g != 128) return hipErrorInvalidValue;
  switch (R) {
#define CASE(r) case r: return zfp_launch_rate<r>(encode, bf16, g, src, gauges, dst, a, s);
    CG_ZFP_RATES(CASE)
#undef CASE
  }
  return hipErrorInvalidValue;
}

hipError_t zfp_encode_launch(int R, bool bf16, int g, const void *kv, const float *gauges,
                             uint8_t *payload, const TileArgs &a, hipStream_t s) {
  return zfp_launch(R, true, bf16, g, kv, gauges, payload, a, s);
}

hipError_t zfp_decode_launch(int R, bool bf16, int g, const uint8_t *payload, const float *gauges,
                             void *out, const TileArgs &a, hipStream_t s) {
  return zfp_launch(R, false, bf16, g, payload, gauges, out, a, s);
}

// Gauge-only rows kernel: storage (or fp32) rows -> gauge / inverse gauge ->
// storage (or fp32) rows.  Backs the NONE backend and cg_gauge_apply.
template <bool SRC_BF16, bool DST_BF16, int G, bool INV>
__global__ __launch_bounds__(NT) void k_gauge_rows(const void *__restrict__ src,
                                                   const float *__restrict__ gauges,
                                                   void *__restrict__ dst, TileArgs a) {
  __shared__ float xs[TILE_T * PITCH];
  const int64_t field = launch_field((int64_t)blockIdx.x / a.tiles, a.fsel, a.fstep, a.fbase);
  const int tile = (int)((int64_t)blockIdx.x % a.tiles);
  const int64_t tb = a.t0 + (int64_t)tile * TILE_T;
  const int nrows = (int)min((int64_t)TILE_T, a.t0 + a.nt - tb);
  const int64_t row0 = field * a.tcap + tb;
  load_tile<SRC_BF16>((const uint8_t *)src + (size_t)row0 * D * (SRC_BF16 ? 2 : 4), nrows, xs);
  __syncthreads();
  if constexpr (G != 0) {
    TileGauge<G, INV> tg;
    tg.load(gauges + gauge_index(field, a.batch, a.heads) * D * G);
    tg.apply(xs, nrows);
    __syncthreads();
  }
  const size_t off = (size_t)row0 * D * (DST_BF16 ? 2 : 4);
  if (a.ref) {
    ErrAcc e;
    store_tile_err<DST_BF16>((uint8_t *)dst + off, nrows, xs, (const uint8_t *)a.ref + off, e);
    write_err(e, a.epart);
  } else {
    store_tile<DST_BF16>((uint8_t *)dst + off, nrows, xs);
  }
}

template <bool SB, bool DB, bool INV>
static hipError_t gauge_rows_g(int g, const void *src, const float *gauges, void *dst,
                               const TileArgs &a, hipStream_t s) {
  const dim3 grid((unsigned)a.grid), block(NT);
  switch (g) {
    case 0:
      hipLaunchKernelGGL((k_gauge_rows<SB, DB, 0, INV>), grid, block, 0, s, src, gauges, dst, a);
      return hipGetLastError();
    case 8:
      hipLaunchKernelGGL((k_gauge_rows<SB, DB, 8, INV>), grid, block, 0, s, src, gauges, dst, a);
      return hipGetLastError();
    case 16:
      hipLaunchKernelGGL((k_gauge_rows<SB, DB, 16, INV>), grid, block, 0, s, src, gauges, dst, a);
      return hipGetLastError();
    case 32:
      hipLaunchKernelGGL((k_gauge_rows<SB, DB, 32, INV>), grid, block, 0, s, src, gauges, dst, a);
      return hipGetLastError();
    case 128:  // fp32 storage only (bf16 takes the split bf16 rows kernel)
      if constexpr (!SB) {
        hipLaunchKernelGGL((k_gauge_rows<SB, DB, 128, INV>), grid, block, 0, s, src, gauges, dst, a);
        return hipGetLastError();
      }
      break;
  }
  return hipErrorInvalidValue;
}

hipError_t gauge_rows_launch(bool src_bf16, bool dst_bf16, bool inverse, int g, const void *src,
                             const float *gauges, void *dst, const TileArgs &a, hipStream_t s) {
  if (inverse) {
    if (src_bf16) return dst_bf16 ? gauge_rows_g<true, true, true>(g, src, gauges, dst, a, s)
                                  : gauge_rows_g<true, false, true>(g, src, gauges, dst, a, s);
    return dst_bf16 ? gauge_rows_g<false, true, true>(g, src, gauges, dst, a, s)
                    : gauge_rows_g<false, false, true>(g, src, gauges, dst, a, s);
  }
  if (src_bf16) return dst_bf16 ? gauge_rows_g<true, true, false>(g, src, gauges, dst, a, s)
                                : gauge_rows_g<true, false, false>(g, src, gauges, dst, a, s);
  return dst_bf16 ? gauge_rows_g<false, true, false>(g, src, gauges, dst, a, s)
                  : gauge_rows_g<false, false, false>(g, src, gauges, dst, a, s);
}

__global__ __launch_bounds__(64) void k_error_reduce(const double *__restrict__ epart,
                                                      int64_t per_field, double values,
                                                      double *__restrict__ out) {
  if (threadIdx.x != 0) return;
  const int64_t f = blockIdx.x;
  const double *p = epart + (size_t)f * per_field * 3;
  double a = 0.0, b = 0.0, c = 0.0;
  for (int64_t j = 0; j < per_field; j++) {
    a += p[3 * j];
    b += p[3 * j + 1];
    c = fmax(c, p[3 * j + 2]);
  }
  double *o = out + (size_t)f * 4;
  o[0] = a;
  o[1] = b;
  o[2] = c;
  o[3] = values;
}

hipError_t error_reduce_launch(const double *epart, int64_t fields, int64_t per_field,
                               double values_per_field, double *out, hipStream_t s) {
  hipLaunchKernelGGL(k_error_reduce, dim3((unsigned)fields), dim3(64), 0, s, epart, per_field,
                     values_per_field, out);
  return hipGetLastError();
}

}  // namespace cgk
