// Per-group uncentered second moments of a KV cache, the input of the PCA/KLT
// coordinate control ("Codec-Gauge", arXiv HTML, coordinate-control
// paragraph: the KLT basis is the eigenbasis of the uncentered second moment
// at layer, K/V, head and group granularity).
//   M_r = sum_t x_t[r] x_t[r]^T      (g x g per group r of every field)
// One workgroup per (field, chunk of 64 tiles = 4096 rows): the tile is staged
// in LDS as fp32, each thread owns the entries e = tid + 256 j of the field's
// D * g moment entries and accumulates them in fp64 (the products of two
// storage values are exact in fp64), then writes its chunk partial.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cg_launch.hpp"
#include "cg_tile.hpp"

namespace cgk {

constexpr int MOMENT_CHUNK = 64;  // tiles per workgroup

template <bool BF16, int G>
__global__ __launch_bounds__(NT) void k_second_moment(const void *__restrict__ kv, int64_t tcap,
                                                      int64_t tokens, int64_t chunks,
                                                      double *__restrict__ part) {
  __shared__ float xs[TILE_T * PITCH];
  constexpr int E = D * G;            // entries per field
  constexpr int PER = E / NT;         // entries per thread
  const int64_t f = (int64_t)blockIdx.x / chunks;
  const int64_t chunk = (int64_t)blockIdx.x % chunks;
  const int64_t ntiles = (tokens + TILE_T - 1) / TILE_T;
  int ci[PER], ck[PER];
#pragma unroll
  for (int j = 0; j < PER; j++) {
    const int e = threadIdx.x + NT * j;
    const int r = e / (G * G), i = (e / G) % G, k = e % G;
    ci[j] = r * G + i;
    ck[j] = r * G + k;
  }
  double acc[PER];
#pragma unroll
  for (int j = 0; j < PER; j++) acc[j] = 0.0;
  for (int64_t tile = chunk * MOMENT_CHUNK; tile < min(ntiles, (chunk + 1) * MOMENT_CHUNK); tile++) {
    const int64_t tb = tile * TILE_T;
    const int nrows = (int)min((int64_t)TILE_T, tokens - tb);
    load_tile<BF16>((const uint8_t *)kv + (size_t)(f * tcap + tb) * D * (BF16 ? 2 : 4), nrows, xs);
    __syncthreads();
    for (int t = 0; t < nrows; t++) {
      const float *row = xs + t * PITCH;
#pragma unroll
      for (int j = 0; j < PER; j++) acc[j] += (double)row[ci[j]] * (double)row[ck[j]];
    }
    __syncthreads();
  }
  double *o = part + ((size_t)f * chunks + chunk) * E;
#pragma unroll
  for (int j = 0; j < PER; j++) o[threadIdx.x + NT * j] = acc[j];
}

int64_t moment_chunks(int64_t tokens) {
  const int64_t ntiles = (tokens + TILE_T - 1) / TILE_T;
  const int64_t c = (ntiles + MOMENT_CHUNK - 1) / MOMENT_CHUNK;
  return c < 1 ? 1 : c;
}

hipError_t second_moment_launch(bool bf16, int g, const void *kv, int64_t tcap, int64_t tokens,
                                int64_t fields, double *part, hipStream_t s) {
  const int64_t chunks = moment_chunks(tokens);
  const dim3 grid((unsigned)(fields * chunks)), block(NT);
#define CG_M(BF, GG)                                                                          \
  if (bf16 == BF && g == GG) {                                                                \
    hipLaunchKernelGGL((k_second_moment<BF, GG>), grid, block, 0, s, kv, tcap, tokens, chunks, \
                       part);                                                                 \
    return hipGetLastError();                                                                 \
  }
  CG_M(true, 8) CG_M(true, 16) CG_M(true, 32) CG_M(true, 128)
  CG_M(false, 8) CG_M(false, 16) CG_M(false, 32) CG_M(false, 128)
#undef CG_M
  return hipErrorInvalidValue;
}

}  // namespace cgk
