// Internal launch interface of the block-uniform / KIVI-style quantizer
// kernels and the dense (g = 128) MFMA gauge.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cgq {

struct QuantArgs {
  int64_t tcap;      // token_capacity
  int64_t tokens;    // valid rows
  int64_t t0, nt;    // rows to process
  int64_t fields;    // number of fields
  int32_t batch, heads, kv;
  int32_t backend;   // CG_BACKEND_BLOCK_UNIFORM or CG_BACKEND_KIVI
  int32_t bits;
  int32_t block;     // BU: tokens per block; KIVI: group (32)
  int32_t residual;  // KIVI tail rows
  const void *ref;   // decode: reference rows for the error sums (or null)
  double *epart;     // decode: per-workgroup error partials [grid][3]
  // decode: fields covered, runs of fsel fields every fstep from fbase
  // (`fields` is then the number covered)
  int64_t fsel, fstep, fbase;
};

// tiles per workgroup: the dense gauge walks 16 tiles (1024 tokens) so each
// workgroup turns its 64 KB gauge into fragments once; the others walk 4 when
// the call still gives at least 8192 workgroups, else 1.  Every workgroup
// fetches tile i+1 while it works on tile i.
inline int quant_chunk_tiles(int g, int64_t fields, int64_t ntiles) {
  if (g == 128) return 16;
  return fields * ((ntiles + 3) / 4) >= 8192 ? 4 : 1;
}

bool bits_built(int bits);
bool bu_block_built(int bt);

inline QuantArgs make_args(int64_t tcap, int64_t tokens, int64_t t0, int64_t nt, int64_t fields,
                           int batch, int heads, int backend, int bits, int block, int residual,
                           int kv) {
  QuantArgs q{};
  q.tcap = tcap; q.tokens = tokens; q.t0 = t0; q.nt = nt; q.fields = fields;
  q.batch = batch; q.heads = heads; q.kv = kv; q.backend = backend; q.bits = bits;
  q.block = block; q.residual = residual;
  q.fsel = q.fstep = fields; q.fbase = 0;
  return q;
}

hipError_t encode_launch(const QuantArgs &q, bool bf16, int g, const void *kv, const float *gauges,
                         uint8_t *payload, float *meta, hipStream_t s);
hipError_t decode_launch(const QuantArgs &q, bool bf16, int g, const uint8_t *payload,
                         const float *meta, const float *gauges, void *out, hipStream_t s);
hipError_t gauge128_rows_launch(bool bf16, bool inverse, const void *kv, const float *gauges,
                                float *out, int64_t tcap, int64_t tokens, int64_t fields,
                                int batch, int heads, hipStream_t s);

}  // namespace cgq
