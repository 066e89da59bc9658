// Gauge applied to head segments of consumer-side rows, for folding the
// cache recovery into the consumer ("Codec-Gauge", arXiv HTML, gauge
// parameterization: recovery can move into downstream projections, and on
// the key side that depends on the positional encoding).  With the cache
// kept in gauged coordinates (x' = G x per group):
//   keys    q . (G^T k') = (G q) . k'    -- gauge the query after its RoPE
//   values  W_o (G^T u) = (W_o G^T) u    -- row r of W_o G^T is G (row r)
// so both consumers need the forward gauge on head_dim segments of rows.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cg_launch.hpp"
#include "cg_tile.hpp"

namespace cgk {

constexpr int FOLD_ROWS = 64;  // rows per workgroup

// Workgroup (row chunk, head h): 128 threads, one per output channel c.
// Thread c keeps its gauge row G[c/g][c%g][0..g) in registers and walks the
// chunk's rows; the row segment is staged in LDS (double buffered).  The sum
// is the fmaf chain k = 0..g-1 from +0, as in the fused gauge.
template <int G, bool BF16>
__global__ __launch_bounds__(D) void k_gauge_heads(const void *__restrict__ x,
                                                   const float *__restrict__ gk, void *__restrict__ y,
                                                   int64_t rows, int q_heads, int group_ratio) {
  __shared__ float xs[2][D];
  const int c = threadIdx.x, h = blockIdx.y;
  const int64_t r0 = (int64_t)blockIdx.x * FOLD_ROWS;
  const int r1 = (int)min((int64_t)FOLD_ROWS, rows - r0);
  const int64_t ld = (int64_t)q_heads * D;
  float gr[G ? G : 1];
  if constexpr (G != 0) {
    const float *row = gk + (int64_t)(h / group_ratio) * D * G + (int64_t)c * G;  // [d/g][g][g]: row c
#pragma unroll
    for (int k = 0; k < G; k++) gr[k] = row[k];
  }
  const int base = G ? (c / (G ? G : 1)) * G : 0;
  for (int r = 0; r < r1; r++) {
    const int64_t off = (r0 + r) * ld + (int64_t)h * D + c;
    float v;
    if (BF16) v = __uint_as_float((uint32_t)((const uint16_t *)x)[off] << 16);
    else v = ((const float *)x)[off];
    float *b = xs[r & 1];
    b[c] = v;
    __syncthreads();
    float acc = 0.0f;
    if constexpr (G == 0) {
      acc = b[c];
    } else {
#pragma unroll
      for (int k = 0; k < G; k++) acc = __builtin_fmaf(gr[k], b[base + k], acc);
    }
    if (BF16) ((uint16_t *)y)[off] = (uint16_t)bf16_rne(acc);
    else ((float *)y)[off] = acc;
    // the next row writes the other buffer; the one after that waits for this
    // row's barrier, by which every thread has read b
  }
}

hipError_t gauge_heads_launch(int g, bool bf16, const void *x, const float *gk, void *y,
                              int64_t rows, int q_heads, int group_ratio, hipStream_t s) {
  const dim3 grid((unsigned)((rows + FOLD_ROWS - 1) / FOLD_ROWS), (unsigned)q_heads), block(D);
#define CG_F(GG, BF)                                                                              \
  if (g == GG && bf16 == BF) {                                                                    \
    hipLaunchKernelGGL((k_gauge_heads<GG, BF>), grid, block, 0, s, x, gk, y, rows, q_heads,      \
                       group_ratio);                                                              \
    return hipGetLastError();                                                                     \
  }
  CG_F(0, true) CG_F(8, true) CG_F(16, true) CG_F(32, true) CG_F(128, true)
  CG_F(0, false) CG_F(8, false) CG_F(16, false) CG_F(32, false) CG_F(128, false)
#undef CG_F
  return hipErrorInvalidValue;
}

}  // namespace cgk
