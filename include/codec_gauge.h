/*
 * codec_gauge.h -- C ABI of libcodecgauge.so, the MI355X (gfx950) Codec-Gauge
 * KV-cache round trip.
 *
 * Method: "Codec-Gauge: Learning Compression-Friendly Gauges for Transformer
 * KV Caches" (arXiv 2607.20538; HTML page and its Chinese translation).
 *  - Problem statement (Chinese page): per layer l the cache holds
 *    K_l, V_l in R^{B x H_l x T x d_l}; for each layer, cache type s in
 *    {K, V}, head h and channel group r (g channels, R_l = d_l / g groups,
 *    g = d_l is a full-head gauge) a gauge G_{l,s,h,r} acts on
 *    X_{l,s}[b,h,t,r] in R^g.  It mixes channels within a group only, never
 *    tokens, heads or layers.
 *  - Gauge parameterization (arXiv page): G = exp(A - A^T), orthogonal; the
 *    gauge is a fixed model-side object, not per-token payload; explicit
 *    application costs O(N_KV g) multiply-adds and is charged in timing.
 *  - Evaluation protocol (arXiv page): the cache goes through the gauge, a
 *    fixed backend (fixed-rate zfp on the FP32-transformed tensor as a 2D
 *    field n_x = d_l, n_y = numel/d_l; block-uniform ranges per T_b x d_l
 *    block; KIVI-style per-channel key / per-token value ranges), decode and
 *    the inverse gauge; actual compressed bytes are recorded (payload plus a
 *    fixed shape header).
 *  - Frequency objective (arXiv page): orthonormal 2D DCT of T_b x d_l
 *    token-channel blocks of X' = G X, spectral-centroid loss L_freq and
 *    smooth log-amplitude rate proxy L_rate (tau = 0.04), combined with
 *    lambda_f, lambda_r; the gauge is trained on it with AdamW.
 *
 * Conventions for every entry point:
 *  - Device pointers point to memory the caller allocated on the current HIP
 *    device (hipMalloc or torch); host pointers are ordinary host memory.
 *    The library never allocates or frees caller-visible memory and keeps no
 *    state between calls (except the thread-local error string).
 *  - Device buffers of KV rows, payloads, metadata, outputs, references and
 *    workspaces must be 16-byte aligned (the kernels use 16-byte vector
 *    accesses; torch allocations are); gauge matrices 4-byte aligned.
 *    Otherwise CG_E_INVAL, before anything is enqueued.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Device work is
 *    enqueued asynchronously unless stated otherwise.
 *  - Every argument is validated on the host before anything is enqueued; on
 *    error nothing is written and a negative CG_E_* code is returned, with a
 *    message available from cg_last_error().  No C++ exception crosses the
 *    ABI.
 *  - KV layout: data[layers][kv][batch][heads][token_capacity][head_dim],
 *    row-major, rows [0, tokens) valid.  A "field" is one
 *    (layer, kv, batch, head) slab [token_capacity][head_dim]; fields are
 *    numbered in that row-major order.
 *  - Gauge layout: G[layers][kv][heads][head_dim/g][g][g] fp32 row-major,
 *    shared by every sequence of the batch; x'[r*g+i] = sum_k G[r][i][k]
 *    x[r*g+k] per token, evaluated (for g <= 32) as an fmaf chain over
 *    k = 0..g-1 from +0; the inverse applies G^T the same way.
 *  - Non-finite KV values are not supported (no check is made).
 */
#ifndef CODEC_GAUGE_H
#define CODEC_GAUGE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* return codes */
#define CG_OK 0
#define CG_E_INVAL (-1)       /* NULL or misaligned pointer, bad enum, negative size */
#define CG_E_SHAPE (-2)       /* sizes not divisible / out of range */
#define CG_E_UNSUPPORTED (-3) /* valid but not built (dtype/backend/bits/g combination) */
#define CG_E_SIZE (-4)        /* a caller buffer or workspace is too small */
#define CG_E_HIP (-5)         /* HIP runtime / launch error (message from HIP) */
#define CG_E_INTERNAL (-6)

/* storage formats */
#define CG_DTYPE_F32 0
#define CG_DTYPE_BF16 1

/* backends */
#define CG_BACKEND_NONE 0          /* gauge only: payload = gauged fp32 values */
#define CG_BACKEND_ZFP 1           /* zfp-style fixed rate, 4x4 blocks */
#define CG_BACKEND_BLOCK_UNIFORM 2 /* one min/max range per block_tokens x head_dim */
#define CG_BACKEND_KIVI 3          /* keys per-channel, values per-token ranges */

/* size of the fixed per-tensor shape header (one per (layer, kv) tensor) */
#define CG_HEADER_BYTES 64

typedef struct cg_shape {
  int32_t layers;         /* L >= 1 */
  int32_t kv;             /* 1 or 2 (index 0 = K, 1 = V) */
  int32_t batch;          /* B >= 1 */
  int32_t heads;          /* KV heads H >= 1 */
  int64_t tokens;         /* valid rows T, 0 <= T <= token_capacity */
  int64_t token_capacity; /* allocated rows per field */
  int32_t head_dim;       /* d_l; the library supports 128 */
  int32_t dtype;          /* CG_DTYPE_* storage format of the KV tensors */
} cg_shape;

typedef struct cg_gauge {
  int32_t group;   /* g: 0 = identity (no arithmetic), else divides head_dim;
                      built: 8, 16 and 32 for every backend, 128 (dense
                      full-head gauge, matrix cores) for ZFP,
                      BLOCK_UNIFORM and KIVI */
  const float *G;  /* device, fp32 [layers][kv][heads][head_dim/g][g][g];
                      ignored when group == 0 */
} cg_gauge;

typedef struct cg_codec {
  int32_t backend;         /* CG_BACKEND_* */
  int32_t bits;            /* ZFP: bits per value R in {2,3,4,6,8};
                              quantizers: code bits in {2,3,4,6,8} */
  int32_t block_tokens;    /* BLOCK_UNIFORM: tokens per range block (T_b);
                              KIVI: group size (tokens per key range, channels
                              per value range) */
  int32_t residual_tokens; /* KIVI: trailing tokens kept in the storage
                              format (after the gauge); else 0 */
} cg_codec;

typedef struct cg_stats {
  double L_freq; /* mean over blocks of sum(r E) / sum(E) */
  double L_rate; /* mean over coefficients of log(1 + U^2 / tau^2) */
  double L;      /* lambda_f L_freq + lambda_r L_rate */
  double sum_E;  /* total DCT energy (equals the field energy, Parseval) */
} cg_stats;

/*
 * Exact byte counts of an encoded cache (host only, no device work).
 * Evaluation protocol (arXiv page): reported bytes are the zfp payload plus a
 * fixed shape header.  Per field of token_capacity rows:
 *   ZFP            payload token_capacity*d*R/8, no metadata
 *   BLOCK_UNIFORM  payload token_capacity*d*bits/8, metadata 8 B per block
 *                  (fp32 min, fp32 step)
 *   KIVI           payload (token_capacity-residual)*d*bits/8 + residual*d*
 *                  sizeof(storage), metadata 8 B per group of block_tokens
 *   NONE           payload token_capacity*d*4 (gauged fp32), no metadata
 * header = CG_HEADER_BYTES * layers * kv.  Any output pointer may be NULL.
 */
int cg_encoded_bytes(const cg_shape *shape, const cg_codec *codec, uint64_t *payload_bytes,
                     uint64_t *meta_bytes, uint64_t *header_bytes);

/*
 * Gauge + encode rows [t0, t0+nt) of every field (evaluation protocol: every
 * new KV token passes through gauge -> backend; rolling compressed history).
 *   kv       device, storage format, KV layout above (read only)
 *   payload  device, >= payload_bytes of cg_encoded_bytes; block rows of a
 *            field sit at fixed offsets, so appends (t0 > 0) only write the
 *            rows they encode
 *   meta     device metadata buffer (quantizers), or NULL when meta_cap == 0
 * ZFP: t0 a multiple of 4 and nt too, except where t0 + nt == tokens: a
 * partial last block row is completed by repeating the last token (gauged)
 * row, and decoding it returns the valid rows only.  BLOCK_UNIFORM:
 * multiples of block_tokens.
 * KIVI: t0 == 0 and nt == tokens (whole fields).  t0 + nt <= tokens.
 */
int cg_encode(const cg_shape *shape, const void *kv, const cg_gauge *gauge,
              const cg_codec *codec, int64_t t0, int64_t nt, void *payload,
              uint64_t payload_cap, void *meta, uint64_t meta_cap, void *stream);

/*
 * Decode + inverse gauge rows [t0, t0+nt) of every field into kv_out
 * (storage format, KV layout; only those rows are written).  Decoding reads
 * exactly the bits each block owns, so any payload content decodes without
 * out-of-bounds access.  Same alignment rules as cg_encode.
 */
int cg_decode(const cg_shape *shape, const void *payload, uint64_t payload_cap,
              const void *meta, uint64_t meta_cap, const cg_gauge *gauge,
              const cg_codec *codec, int64_t t0, int64_t nt, void *kv_out, void *stream);

/*
 * Recovery folded into the consumer (gauge-parameterization paragraph, arXiv
 * page: some recovery operations can move into the downstream projections;
 * on the key side that depends on the positional encoding).  cg_decode_gauged
 * is cg_decode, except that fields whose K/V index s has bit s set in `keep`
 * are written in gauged coordinates, x' = G x: their inverse gauge is
 * skipped.  The consumer then applies G on its side with cg_gauge_heads:
 *   keys    q . (G^T k') = (G q) . k'    gauge each query after its RoPE
 *   values  W_o (G^T u) = (W_o G^T) u    gauge the rows of W_o once
 * keep: 0 (same as cg_decode), CG_KEEP_KEYS, CG_KEEP_VALUES (shape kv = 2)
 * or both; other values give CG_E_INVAL.  Same layout, alignment and error
 * behaviour as cg_decode; one launch per kind that differs in treatment.
 */
#define CG_KEEP_KEYS 1   /* K/V index 0 */
#define CG_KEEP_VALUES 2 /* K/V index 1 */
int cg_decode_gauged(const cg_shape *shape, const void *payload, uint64_t payload_cap,
                     const void *meta, uint64_t meta_cap, const cg_gauge *gauge,
                     const cg_codec *codec, int64_t t0, int64_t nt, int32_t keep, void *kv_out,
                     void *stream);

/*
 * Cache-side error (evaluation protocol, arXiv page: compressed bytes, actual
 * bits/value, KV MSE, KV NRMSE, key/value NRMSE and maximum absolute error;
 * the evaluator keeps raw sums and counts).  Per field, over the decoded rows
 * as stored (after rounding to the storage format), against a reference in
 * the same layout:
 *   sse     = sum (x_hat - x)^2      ref_ss = sum x^2
 *   max_abs = max |x_hat - x|        values = rows * head_dim
 * Sums are fp64, reduced in a fixed order (deterministic).
 */
typedef struct cg_field_error {
  double sse;
  double ref_ss;
  double max_abs;
  double values;
} cg_field_error;

/* Whole-cache figures from the per-field sums: mse = sse / values,
   nrmse = sqrt(sse / ref_ss) (over all, key and value fields), max_abs. */
typedef struct cg_cache_error {
  double mse;
  double nrmse;
  double key_nrmse;
  double value_nrmse; /* 0 when kv == 1 */
  double max_abs;
  double values;
} cg_cache_error;

/* Device scratch needed by cg_decode_error for these rows (host only). */
int cg_decode_error_workspace_bytes(const cg_shape *shape, const cg_gauge *gauge,
                                    const cg_codec *codec, int64_t t0, int64_t nt, size_t *bytes);

/*
 * cg_decode that also accumulates the error of every decoded value against
 * kv_ref (device, storage format, KV layout; rows [t0, t0+nt) are read) in the
 * kernels that store it.  err: device cg_field_error[n_fields], overwritten
 * (values = nt * head_dim).  Same validation and errors as cg_decode, plus
 * CG_E_SIZE for a missing or small workspace.
 */
int cg_decode_error(const cg_shape *shape, const void *payload, uint64_t payload_cap,
                    const void *meta, uint64_t meta_cap, const cg_gauge *gauge,
                    const cg_codec *codec, int64_t t0, int64_t nt, void *kv_out,
                    const void *kv_ref, void *workspace, size_t ws_bytes, cg_field_error *err,
                    void *stream);

/*
 * cg_decode_error for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same arguments, validation, results and errors as cg_decode_error, minus
 * the workspace: the per-workgroup error partials go to a device array of
 * CG_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends.  Its device address is looked up on the first
 * call on a device (that device must be current, and `stream` must belong
 * to it).  The call allocates nothing (no hipMalloc, hipFree or allocating
 * library routine).  Calls whose partials need more than
 * CG_NOALLOC_SCRATCH_BYTES (see cg_decode_error_workspace_bytes) return
 * CG_E_SIZE before anything is enqueued.  Every call on a GPU shares that
 * GPU's array and nothing in it needs to start at zero (each launch
 * overwrites the partials it reads), but calls that overlap on one GPU
 * (concurrent streams or threads) race on it: serialize them.
 */
#define CG_NOALLOC_SCRATCH_BYTES (16u << 20)
int cg_decode_error_noalloc(const cg_shape *shape, const void *payload, uint64_t payload_cap,
                            const void *meta, uint64_t meta_cap, const cg_gauge *gauge,
                            const cg_codec *codec, int64_t t0, int64_t nt, void *kv_out,
                            const void *kv_ref, cg_field_error *err, void *stream);

/* Host: per-field sums (host array of n_fields) -> whole-cache figures. */
int cg_cache_error_summary(const cg_shape *shape, const cg_field_error *err, cg_cache_error *out);

/* cg_encode of rows [0, tokens) followed by cg_decode of the same rows. */
int cg_roundtrip(const cg_shape *shape, const void *kv_in, const cg_gauge *gauge,
                 const cg_codec *codec, void *payload, uint64_t payload_cap, void *meta,
                 uint64_t meta_cap, void *kv_out, void *stream);

/*
 * Gauge-fit statistics (frequency objective, arXiv page) of every field over
 * rows [0, tokens): X' = G X with G = exp(A - A^T) per group (built here in
 * fp64 and rounded to fp32), orthonormal 2D DCT-II U of each T_b x head_dim
 * block, E = U^2, r_uv = sqrt((u/(T_b-1))^2 + (v/(d-1))^2)/sqrt(2),
 * L_freq = mean over blocks of sum(r E)/sum(E) (0 for an all-zero block),
 * L_rate = mean over coefficients of log(1 + U^2/tau^2) (smooth in U,
 * concave in the energy U^2),
 * L = lambda_f L_freq + lambda_r L_rate, per field.
 *   kv         device, storage format, KV layout (tokens % T_b == 0)
 *   g          0 (identity), 8, 16 or 32 (built); A_host fp64
 *              [layers][kv][heads][d/g][g][g] (ignored when g == 0)
 *   T_b        16 (built)
 *   workspace  device scratch of >= cg_stats_workspace_bytes() bytes
 *   out_host   host cg_stats[n_fields]
 *   dA_host    host fp64 [n_fields][d/g][g][g] gradient of each field's L
 *              with respect to its A (through the Frechet derivative of exp),
 *              or NULL to skip the gradient
 * Synchronous: returns after the results are in host memory.
 */
int cg_gauge_fit_stats(const cg_shape *shape, const void *kv, int32_t g, const double *A_host,
                       int32_t T_b, float tau, float lambda_f, float lambda_r, void *workspace,
                       size_t ws_bytes, cg_stats *out_host, double *dA_host, void *stream);

/*
 * cg_gauge_fit_stats with the gradient of the training objective per gauge
 * (gauge-training paragraph, arXiv page: one gauge per layer, K/V, head and
 * group, shared by every sequence of the batch and trained with AdamW on the
 * frequency objective of the cached windows): dA_gauge_host fp64
 * [layers][kv][heads][d/g][g][g] = sum over b = 0..batch-1 of the gradient of
 * field (l, s, b, h)'s L with respect to A[l][s][h], i.e. the gradient of
 * sum_b L(l, s, b, h).  The batch sum is taken on dL/dG before the Frechet
 * adjoint (a linear map), in b order.  dA_gauge_host must not be NULL when
 * g != 0 (CG_E_INVAL); everything else as cg_gauge_fit_stats.  Synchronous.
 */
int cg_gauge_fit_grad(const cg_shape *shape, const void *kv, int32_t g, const double *A_host,
                      int32_t T_b, float tau, float lambda_f, float lambda_r, void *workspace,
                      size_t ws_bytes, cg_stats *out_host, double *dA_gauge_host, void *stream);

/* Device scratch needed by cg_gauge_fit_stats and cg_gauge_fit_grad (host only). */
int cg_stats_workspace_bytes(const cg_shape *shape, int32_t g, int32_t T_b, size_t *bytes);

/*
 * Chain rule through the gauge parameterization (gauge-training paragraph,
 * arXiv page): for G = exp(S), S = A - A^T, and a gradient dL/dG,
 *   dL/dA = Psi - Psi^T,  Psi = L_exp(S^T, dL/dG)
 * (the Frechet derivative of exp at S^T in the direction dL/dG), evaluated
 * in fp64 with one [13/13] Pade pass with scaling and squaring.  A_host,
 * dG_host, dA_host: host fp64 [n][g][g].  cg_gauge_fit_stats applies the
 * same map to its device-side dL/dG.
 */
int cg_gauge_grad(int64_t n, int32_t g, const double *A_host, const double *dG_host, double *dA_host);

/*
 * G = exp(A - A^T) for n matrices of size g x g (gauge parameterization,
 * arXiv page): host fp64 scaling and squaring with a [13/13] Pade
 * approximant, rounded to fp32.  A_host fp64 [n][g][g], G_host fp32
 * [n][g][g] (both host).  Synchronous.
 */
int cg_gauge_from_skew(int64_t n, int32_t g, const double *A_host, float *G_host);

/*
 * Apply the gauge (direction 0: G, 1: G^T) to rows [0, tokens) of every
 * field with the same device routine the fused kernels use, writing fp32
 * [fields][token_capacity][head_dim] to `out` (device).  Exported so the
 * gauge stage can be checked on its own.
 */
int cg_gauge_apply(const cg_shape *shape, const void *kv, const cg_gauge *gauge,
                   int32_t direction, float *out, void *stream);

/*
 * Consumer side of the folded recovery (see cg_decode_gauged): the forward
 * gauge of cache layer `layer`, K/V index `kind`, on the head_dim segments
 * of `rows` rows,
 *   y[r][h d + c] = sum_k G[h / (q_heads / heads)][c / g][c % g][k] * x[r][h d + (c / g) g + k]
 * as an fp32 fmaf chain over k = 0..g-1 from +0 (the fused gauge's order);
 * group 0 copies.  Query head h uses the gauge of KV head h / (q_heads /
 * heads) (grouped-query attention).
 *   shape    the cache shape the gauges belong to (layers, kv, heads, head_dim)
 *   x, y     device [rows][q_heads * head_dim], both CG_DTYPE_F32 or both
 *            CG_DTYPE_BF16 (`dtype`; bf16 output rounded to nearest even);
 *            they must not overlap (CG_E_INVAL)
 *   q_heads  a positive multiple of shape->heads (CG_E_SHAPE otherwise)
 * Queries: x = post-RoPE queries, kind 0.  Output projection: x = W_o
 * ([d_model][q_heads * head_dim], row-major), kind 1.  Asynchronous on stream.
 */
int cg_gauge_heads(const cg_shape *shape, const cg_gauge *gauge, int32_t layer, int32_t kind,
                   int32_t q_heads, int64_t rows, int32_t dtype, const void *x, void *y,
                   void *stream);

/*
 * Gauge training and coordinate controls.
 *
 * One AdamW step (gauge-training paragraph, arXiv page: the gauge parameters
 * are optimized with AdamW; decoupled weight decay, Loshchilov and Hutter):
 *   p <- p (1 - lr wd);  m <- b1 m + (1 - b1) grad;  v <- b2 v + (1 - b2) grad^2
 *   p <- p - lr (m / (1 - b1^step)) / (sqrt(v / (1 - b2^step)) + eps)
 * param, grad, m, v: host fp64 arrays of n values (m, v start at 0); step >= 1.
 */
int cg_adamw_update(int64_t n, double *param, const double *grad, double *m, double *v,
                    int64_t step, double lr, double beta1, double beta2, double eps,
                    double weight_decay);

/* control gauges (main-grid and coordinate-control paragraphs, arXiv page) */
#define CG_CONTROL_IDENTITY 0
#define CG_CONTROL_HADAMARD 1       /* Sylvester order, scaled 1/sqrt(g); g a power of two */
#define CG_CONTROL_DCT 2            /* orthonormal DCT-II, rows = frequencies */
#define CG_CONTROL_ORTHONORMALIZE 3 /* Q of M = Q R with diag(R) > 0 (Haar for Gaussian M) */
#define CG_CONTROL_KLT 4            /* rows = eigenvectors of the symmetric M, decreasing
                                       eigenvalue, largest-magnitude component positive */

/*
 * n control gauges of size g x g, computed in fp64 and rounded to fp32:
 * G_host fp32 [n][g][g]; M_host fp64 [n][g][g] for ORTHONORMALIZE and KLT
 * (a random matrix drawn by the caller; a second moment from
 * cg_second_moment), else ignored (may be NULL).  Host only.
 */
int cg_gauge_control(int32_t kind, int64_t n, int32_t g, const double *M_host, float *G_host);

/* Device scratch needed by cg_second_moment (host only). */
int cg_second_moment_workspace_bytes(const cg_shape *shape, int32_t g, size_t *bytes);

/*
 * Uncentered second moments per gauge group (input of the KLT control):
 *   M[l][s][h][r] = sum over the batch and rows [0, tokens) of x_t[r] x_t[r]^T
 * kv: device, storage format, KV layout; g in {8, 16, 32, 128}; M_host fp64
 * [layers][kv][heads][d/g][g][g] (host, overwritten).  Products and sums in
 * fp64, reduced in a fixed order.  Synchronous.
 */
int cg_second_moment(const cg_shape *shape, const void *kv, int32_t g, void *workspace,
                     size_t ws_bytes, double *M_host, void *stream);

/* Write the fixed-size shape header of one (layer, kv) tensor into a host
   buffer of >= CG_HEADER_BYTES bytes. */
int cg_write_header(const cg_shape *shape, const cg_codec *codec, int32_t layer, int32_t kv,
                    void *header_host, uint64_t cap);

/* Message of the last error on the calling thread ("" if none). */
const char *cg_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* CODEC_GAUGE_H */
