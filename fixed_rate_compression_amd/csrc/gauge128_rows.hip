// cg_gauge_apply for the dense (g = 128) gauge with bf16 storage: the
// quantizers' split bf16 MFMA routine on the same 64-token tiles and 16-tile
// workgroup chunks.
#include "quant_launch.hpp"

namespace cgq {

hipError_t gauge128_rows_launch(bool bf16, bool inverse, const void *kv, const float *gauges,
                                float *out, int64_t tcap, int64_t tokens, int64_t fields, int batch,
                                int heads, hipStream_t s) {
  QuantArgs q = make_args(tcap, tokens, 0, tokens, fields, batch, heads, 0, 0, 0, 0, 1);
  const QK a = make_qk(q, quant_chunk_tiles(128, fields, (tokens + TILE_T - 1) / TILE_T));
  const dim3 grid((unsigned)(fields * a.chunks)), block(NT);
  if (!bf16) return hipErrorInvalidValue;  // fp32 storage: the fmaf-chain rows kernel
  if (inverse) hipLaunchKernelGGL((k_gauge128_rows<true, true>), grid, block, 0, s, kv, gauges, out, a);
  else hipLaunchKernelGGL((k_gauge128_rows<true, false>), grid, block, 0, s, kv, gauges, out, a);
  return hipGetLastError();
}

}  // namespace cgq
