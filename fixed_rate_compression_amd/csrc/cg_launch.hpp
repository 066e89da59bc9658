// Internal launch interface between the C ABI (codec_gauge_api.cpp) and the
// kernel translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cgk {

constexpr int TILE_T = 64;  // tokens per workgroup tile of the rows kernels
constexpr int ZFP128_CHUNK = 16;  // tiles per workgroup with the dense (g = 128) gauge
constexpr int ZFP_CHUNK = 4;      // tiles per workgroup with the g <= 32 gauges, given enough work

// tiles per workgroup of the VALU-gauge zfp kernels: ZFP_CHUNK when the call
// still gives at least 8192 workgroups (8 per CU-slot), else 1
inline int zfp_chunk_tiles(int64_t fields, int64_t tiles) {
  return fields * ((tiles + ZFP_CHUNK - 1) / ZFP_CHUNK) >= 8192 ? ZFP_CHUNK : 1;
}

// geometry of a rows launch over every field: one workgroup per
// (field, 64-token tile) of rows [t0, t0 + nt)
struct TileArgs {
  int64_t tcap;   // token_capacity (row stride of a field)
  int64_t t0;     // first row
  int64_t nt;     // number of rows
  int64_t grid;   // fields * tiles
  int32_t tiles;  // tiles per field = ceil(nt / 64)
  int32_t batch;  // B (gauges are shared across the batch)
  int32_t heads;  // H
  int32_t chunks;       // zfp kernels: workgroups per field = ceil(tiles / chunk_tiles)
  int32_t chunk_tiles;  // zfp kernels: tiles per workgroup (set by the launcher)
  // decode only: reference rows in the output layout (or null) and the
  // per-workgroup error partials [grid][3] they produce
  const void *ref;
  double *epart;
  // decode only: the fields a launch covers, runs of fsel consecutive fields
  // every fstep fields from field fbase (all fields: fsel = fstep = count)
  int64_t fsel, fstep, fbase;
};

bool zfp_rate_built(int R);
hipError_t zfp_encode_launch(int R, bool bf16, int g, const void *kv, const float *gauges,
                             uint8_t *payload, const TileArgs &a, hipStream_t s);
hipError_t zfp_decode_launch(int R, bool bf16, int g, const uint8_t *payload, const float *gauges,
                             void *out, const TileArgs &a, hipStream_t s);
// forward gauge of (layer, kind) on head_dim segments of rows x, y
// [rows][q_heads * 128] (query head h uses gauge head h / group_ratio); gk
// points at the (layer, kind) gauges
hipError_t gauge_heads_launch(int g, bool bf16, const void *x, const float *gk, void *y,
                              int64_t rows, int q_heads, int group_ratio, hipStream_t s);
hipError_t gauge_rows_launch(bool src_bf16, bool dst_bf16, bool inverse, int g, const void *src,
                             const float *gauges, void *dst, const TileArgs &a, hipStream_t s);
// per-group second moments: part[field][moment_chunks(tokens)][D * g] (fp64)
int64_t moment_chunks(int64_t tokens);
hipError_t second_moment_launch(bool bf16, int g, const void *kv, int64_t tcap, int64_t tokens,
                                int64_t fields, double *part, hipStream_t s);
// per field: sum its `per_field` consecutive error partials in order ->
// out[field][4] = {sum e^2, sum x^2, max |e|, values}
hipError_t error_reduce_launch(const double *epart, int64_t fields, int64_t per_field,
                               double values_per_field, double *out, hipStream_t s);

}  // namespace cgk
