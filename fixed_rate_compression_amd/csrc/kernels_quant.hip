// Dispatch of the block-uniform / KIVI-style kernels (quant_kernels.hpp) and
// of the dense-gauge rows kernel.  Bit widths are instantiated in their own
// translation units (quant_b<bits>.hip).
#include "cg_quant.hpp"
#include "cg_tile.hpp"

namespace cgq {

template <int BITS>
hipError_t quant_launch_bits(bool encode, bool bf16, int g, int backend, const void *src,
                             const float *gauges, void *dst, const void *meta_in, float *meta_out,
                             const QuantArgs &q, hipStream_t s);

bool bits_built(int bits) { return bits == 2 || bits == 3 || bits == 4 || bits == 6 || bits == 8; }
bool bu_block_built(int bt) { return bt == 16 || bt == 32 || bt == 64; }

static hipError_t launch(bool encode, bool bf16, int g, const void *src, const float *gauges,
                         void *dst, const void *meta_in, float *meta_out, const QuantArgs &q,
                         hipStream_t s) {
  if (g != 0 && g != 8 && g != 16 && g != 32 && g != 128) return hipErrorInvalidValue;
  switch (q.bits) {
    case 2: return quant_launch_bits<2>(encode, bf16, g, q.backend, src, gauges, dst, meta_in, meta_out, q, s);
    case 3: return quant_launch_bits<3>(encode, bf16, g, q.backend, src, gauges, dst, meta_in, meta_out, q, s);
    case 4: return quant_launch_bits<4>(encode, bf16, g, q.backend, src, gauges, dst, meta_in, meta_out, q, s);
    case 6: return quant_launch_bits<6>(encode, bf16, g, q.backend, src, gauges, dst, meta_in, meta_out, q, s);
    case 8: return quant_launch_bits<8>(encode, bf16, g, q.backend, src, gauges, dst, meta_in, meta_out, q, s);
  }
  return hipErrorInvalidValue;
}

hipError_t encode_launch(const QuantArgs &q, bool bf16, int g, const void *kv, const float *gauges,
                         uint8_t *payload, float *meta, hipStream_t s) {
  return launch(true, bf16, g, kv, gauges, payload, nullptr, meta, q, s);
}

hipError_t decode_launch(const QuantArgs &q, bool bf16, int g, const uint8_t *payload,
                         const float *meta, const float *gauges, void *out, hipStream_t s) {
  return launch(false, bf16, g, payload, gauges, out, meta, nullptr, q, s);
}

}  // namespace cgq
