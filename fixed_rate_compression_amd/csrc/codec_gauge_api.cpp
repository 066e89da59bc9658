// C ABI of libcodecgauge.so (declared in include/codec_gauge.h): argument
// validation, byte accounting, dispatch to the HIP kernels, and the host fp64
// matrix exponential used to build gauges.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "../../include/codec_gauge.h"
#include "cg_launch.hpp"
#include "cg_quant.hpp"
#include "cg_stats.hpp"

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_fail(hipError_t e, const char *what) {
  return fail(CG_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

int64_t n_fields(const cg_shape *s) {
  return (int64_t)s->layers * s->kv * s->batch * s->heads;
}

// device buffers are read and written with 16-byte vector accesses
bool misaligned(const void *p) { return ((uintptr_t)p & 15u) != 0; }

int check_shape(const cg_shape *s) {
  if (!s) return fail(CG_E_INVAL, "shape is NULL");
  if (s->layers < 1 || s->batch < 1 || s->heads < 1 || (s->kv != 1 && s->kv != 2))
    return fail(CG_E_SHAPE, "layers, batch, heads must be >= 1 and kv 1 or 2");
  if (s->dtype != CG_DTYPE_F32 && s->dtype != CG_DTYPE_BF16)
    return fail(CG_E_INVAL, "dtype %d is not CG_DTYPE_F32 or CG_DTYPE_BF16", s->dtype);
  if (s->head_dim != 128)
    return fail(CG_E_UNSUPPORTED, "head_dim %d: the kernels are specialized for head_dim 128", s->head_dim);
  if (s->tokens < 0 || s->token_capacity < s->tokens)
    return fail(CG_E_SHAPE, "need 0 <= tokens (%lld) <= token_capacity (%lld)",
                (long long)s->tokens, (long long)s->token_capacity);
  if (n_fields(s) > (int64_t)1 << 31) return fail(CG_E_SHAPE, "too many fields");
  return CG_OK;
}

int check_gauge(const cg_gauge *g, const cg_shape *s, const cg_codec *c) {
  if (!g) return fail(CG_E_INVAL, "gauge is NULL");
  if (g->group == 0) return CG_OK;
  if (g->group < 0 || s->head_dim % g->group)
    return fail(CG_E_SHAPE, "gauge group %d must divide head_dim %d", g->group, s->head_dim);
  if (!g->G) return fail(CG_E_INVAL, "gauge matrices are NULL");
  if ((uintptr_t)g->G & 3u) return fail(CG_E_INVAL, "gauge matrices must be 4-byte aligned");
  const bool dense_ok = !c || c->backend == CG_BACKEND_ZFP || c->backend == CG_BACKEND_BLOCK_UNIFORM ||
                        c->backend == CG_BACKEND_KIVI;
  if (g->group == 8 || g->group == 16 || g->group == 32) return CG_OK;
  if (g->group == 128 && dense_ok) return CG_OK;
  return fail(CG_E_UNSUPPORTED, "gauge group %d is not built for this backend", g->group);
}

int check_codec(const cg_codec *c, const cg_shape *s) {
  if (!c) return fail(CG_E_INVAL, "codec is NULL");
  switch (c->backend) {
    case CG_BACKEND_NONE:
      return CG_OK;
    case CG_BACKEND_ZFP:
      if (!cgk::zfp_rate_built(c->bits))
        return fail(CG_E_UNSUPPORTED, "zfp rate %d bits/value is not built (2,3,4,6,8)", c->bits);
      if (s->token_capacity % 4) return fail(CG_E_SHAPE, "zfp needs token_capacity % 4 == 0");
      return CG_OK;
    case CG_BACKEND_BLOCK_UNIFORM:
      if (!cgq::bits_built(c->bits))
        return fail(CG_E_UNSUPPORTED, "block-uniform bits %d not built (2,3,4,6,8)", c->bits);
      if (!cgq::bu_block_built(c->block_tokens))
        return fail(CG_E_UNSUPPORTED, "block-uniform block_tokens %d not built (16,32,64)",
                    c->block_tokens);
      if (s->token_capacity % c->block_tokens)
        return fail(CG_E_SHAPE, "token_capacity must be a multiple of block_tokens");
      return CG_OK;
    case CG_BACKEND_KIVI:
      if (!cgq::bits_built(c->bits))
        return fail(CG_E_UNSUPPORTED, "KIVI bits %d not built (2,3,4,6,8)", c->bits);
      if (c->block_tokens != 32) return fail(CG_E_UNSUPPORTED, "KIVI group must be 32");
      if (c->residual_tokens < 0 || c->residual_tokens > s->tokens ||
          (s->tokens - c->residual_tokens) % 32 || c->residual_tokens % 4)
        return fail(CG_E_SHAPE, "KIVI needs 0 <= residual <= tokens, residual % 4 == 0 and "
                                "(tokens - residual) % 32 == 0");
      if (s->token_capacity - s->tokens < 0) return fail(CG_E_SHAPE, "bad capacity");
      return CG_OK;
  }
  return fail(CG_E_INVAL, "unknown backend %d", c->backend);
}

uint64_t storage_size(const cg_shape *s) { return s->dtype == CG_DTYPE_BF16 ? 2 : 4; }

void byte_counts(const cg_shape *s, const cg_codec *c, uint64_t *pay, uint64_t *meta) {
  const uint64_t F = (uint64_t)n_fields(s), cap = (uint64_t)s->token_capacity,
                 d = (uint64_t)s->head_dim;
  switch (c->backend) {
    case CG_BACKEND_NONE:
      *pay = F * cap * d * 4;
      *meta = 0;
      return;
    case CG_BACKEND_ZFP:
      *pay = F * cap * d * (uint64_t)c->bits / 8;
      *meta = 0;
      return;
    case CG_BACKEND_BLOCK_UNIFORM:
      *pay = F * cap * d * (uint64_t)c->bits / 8;
      *meta = F * (cap / (uint64_t)c->block_tokens) * 8;
      return;
    case CG_BACKEND_KIVI: {
      const uint64_t res = (uint64_t)c->residual_tokens, tq = cap - res;
      *pay = F * (tq * d * (uint64_t)c->bits / 8 + res * d * storage_size(s));
      *meta = F * (tq * d / 32) * 8;
      return;
    }
  }
  *pay = *meta = 0;
}

cgk::TileArgs tile_args(const cg_shape *s, int64_t t0, int64_t nt) {
  cgk::TileArgs a{};
  a.tcap = s->token_capacity;
  a.t0 = t0;
  a.nt = nt;
  a.tiles = (int32_t)((nt + cgk::TILE_T - 1) / cgk::TILE_T);
  a.grid = n_fields(s) * a.tiles;
  a.batch = s->batch;
  a.heads = s->heads;
  a.fsel = a.fstep = n_fields(s);
  a.fbase = 0;
  return a;
}

int check_rows(const cg_shape *s, const cg_codec *c, int64_t t0, int64_t nt) {
  if (t0 < 0 || nt < 0 || t0 + nt > s->tokens)
    return fail(CG_E_SHAPE, "rows [%lld, %lld) outside [0, tokens=%lld)", (long long)t0,
                (long long)(t0 + nt), (long long)s->tokens);
  // zfp: 4-token block rows; a partial last block row only where the valid
  // tokens end (it is padded by repeating the last token)
  if (c->backend == CG_BACKEND_ZFP && (t0 % 4 || (nt % 4 && t0 + nt != s->tokens)))
    return fail(CG_E_SHAPE, "zfp rows must start on a multiple of 4 and end on one or at tokens");
  if (c->backend == CG_BACKEND_BLOCK_UNIFORM && ((t0 % c->block_tokens) || (nt % c->block_tokens)))
    return fail(CG_E_SHAPE, "block-uniform rows must be multiples of block_tokens");
  if (c->backend == CG_BACKEND_KIVI && (t0 != 0 || nt != s->tokens))
    return fail(CG_E_SHAPE, "KIVI encodes and decodes whole fields (t0 = 0, nt = tokens)");
  const int64_t tiles = (nt + cgk::TILE_T - 1) / cgk::TILE_T;
  if (n_fields(s) * tiles >= ((int64_t)1 << 31)) return fail(CG_E_SHAPE, "grid too large");
  return CG_OK;
}

// ---------------------------------------------------------------------------
// host fp64 matrix exponential: scaling and squaring with the diagonal
// [13/13] Pade approximant (Higham, "The scaling and squaring method for the
// matrix exponential revisited", SIAM J. Matrix Anal. Appl. 2005).
// ---------------------------------------------------------------------------

void matmul(int n, const double *A, const double *B, double *C) {
  for (int i = 0; i < n; i++) {
    double *c = C + (size_t)i * n;
    for (int j = 0; j < n; j++) c[j] = 0.0;
    for (int k = 0; k < n; k++) {
      const double a = A[(size_t)i * n + k];
      const double *b = B + (size_t)k * n;
      for (int j = 0; j < n; j++) c[j] += a * b[j];
    }
  }
}

// solve P X = Q for X (n x n), Gaussian elimination with partial pivoting
bool solve(int n, std::vector<double> P, std::vector<double> &Q) {
  for (int col = 0; col < n; col++) {
    int piv = col;
    for (int r = col + 1; r < n; r++)
      if (fabs(P[(size_t)r * n + col]) > fabs(P[(size_t)piv * n + col])) piv = r;
    if (P[(size_t)piv * n + col] == 0.0) return false;
    if (piv != col)
      for (int j = 0; j < n; j++) {
        std::swap(P[(size_t)piv * n + j], P[(size_t)col * n + j]);
        std::swap(Q[(size_t)piv * n + j], Q[(size_t)col * n + j]);
      }
    const double inv = 1.0 / P[(size_t)col * n + col];
    for (int r = col + 1; r < n; r++) {
      const double f = P[(size_t)r * n + col] * inv;
      if (f == 0.0) continue;
      for (int j = col; j < n; j++) P[(size_t)r * n + j] -= f * P[(size_t)col * n + j];
      for (int j = 0; j < n; j++) Q[(size_t)r * n + j] -= f * Q[(size_t)col * n + j];
    }
  }
  for (int col = n - 1; col >= 0; col--) {
    const double inv = 1.0 / P[(size_t)col * n + col];
    for (int j = 0; j < n; j++) Q[(size_t)col * n + j] *= inv;
    for (int r = 0; r < col; r++) {
      const double f = P[(size_t)r * n + col];
      if (f == 0.0) continue;
      for (int j = 0; j < n; j++) Q[(size_t)r * n + j] -= f * Q[(size_t)col * n + j];
    }
  }
  return true;
}

// E = exp(M), n x n, fp64
bool expm_pade13(int n, const double *M, double *E) {
  // Pade [13/13] numerator coefficients p_j = (26-j)! 13! / (26! j! (13-j)!),
  // scaled so that b_13 = 1; consecutive ratio b_j / b_{j+1} = (j+1)(26-j)/(13-j)
  double b[14];
  b[13] = 1.0;
  for (int j = 12; j >= 0; j--) b[j] = b[j + 1] * (double)(j + 1) * (double)(26 - j) / (double)(13 - j);
  const size_t nn = (size_t)n * n;
  double norm1 = 0.0;
  for (int j = 0; j < n; j++) {
    double cs = 0.0;
    for (int i = 0; i < n; i++) cs += fabs(M[(size_t)i * n + j]);
    norm1 = cs > norm1 ? cs : norm1;
  }
  const double theta13 = 5.371920351148152;
  int s = 0;
  if (norm1 > theta13) s = (int)ceil(log2(norm1 / theta13));
  const double scale = ldexp(1.0, -s);
  std::vector<double> A(nn), A2(nn), A4(nn), A6(nn), T1(nn), T2(nn), U(nn), V(nn);
  for (size_t k = 0; k < nn; k++) A[k] = M[k] * scale;
  matmul(n, A.data(), A.data(), A2.data());
  matmul(n, A2.data(), A2.data(), A4.data());
  matmul(n, A4.data(), A2.data(), A6.data());
  // U = A [A6 (b13 A6 + b11 A4 + b9 A2) + b7 A6 + b5 A4 + b3 A2 + b1 I]
  for (size_t k = 0; k < nn; k++) T1[k] = b[13] * A6[k] + b[11] * A4[k] + b[9] * A2[k];
  matmul(n, A6.data(), T1.data(), T2.data());
  for (size_t k = 0; k < nn; k++) T2[k] += b[7] * A6[k] + b[5] * A4[k] + b[3] * A2[k];
  for (int i = 0; i < n; i++) T2[(size_t)i * n + i] += b[1];
  matmul(n, A.data(), T2.data(), U.data());
  // V = A6 (b12 A6 + b10 A4 + b8 A2) + b6 A6 + b4 A4 + b2 A2 + b0 I
  for (size_t k = 0; k < nn; k++) T1[k] = b[12] * A6[k] + b[10] * A4[k] + b[8] * A2[k];
  matmul(n, A6.data(), T1.data(), V.data());
  for (size_t k = 0; k < nn; k++) V[k] += b[6] * A6[k] + b[4] * A4[k] + b[2] * A2[k];
  for (int i = 0; i < n; i++) V[(size_t)i * n + i] += b[0];
  // (V - U) X = (V + U)
  std::vector<double> P(nn), Q(nn);
  for (size_t k = 0; k < nn; k++) {
    P[k] = V[k] - U[k];
    Q[k] = V[k] + U[k];
  }
  if (!solve(n, P, Q)) return false;
  for (int k = 0; k < s; k++) {
    matmul(n, Q.data(), Q.data(), T1.data());
    Q.swap(T1);
  }
  memcpy(E, Q.data(), nn * sizeof(double));
  return true;
}

// R = exp(M) and L = L_exp(M, D), the Frechet derivative of exp at M in the
// direction D, n x n fp64, from one [13/13] Pade evaluation with scaling and
// squaring (Al-Mohy and Higham 2009, "Computing the Frechet derivative of the
// matrix exponential": the Pade numerator/denominator parts U, V and their
// directional derivatives Lu, Lv are built from the same powers of M; then
// (V - U) R = V + U, (V - U) L = Lu + Lv + (Lu - Lv) R, and each squaring
// R <- R R takes L <- R L + L R).
bool expm_frechet_pade13(int n, const double *M, const double *D, double *Rout, double *Lout) {
  double b[14];
  b[13] = 1.0;
  for (int j = 12; j >= 0; j--) b[j] = b[j + 1] * (double)(j + 1) * (double)(26 - j) / (double)(13 - j);
  const size_t nn = (size_t)n * n;
  double norm1 = 0.0;
  for (int j = 0; j < n; j++) {
    double cs = 0.0;
    for (int i = 0; i < n; i++) cs += fabs(M[(size_t)i * n + j]);
    norm1 = cs > norm1 ? cs : norm1;
  }
  const double theta13 = 5.371920351148152;
  int s = 0;
  if (norm1 > theta13) s = (int)ceil(log2(norm1 / theta13));
  const double scale = ldexp(1.0, -s);
  std::vector<double> A(nn), E(nn), A2(nn), A4(nn), A6(nn), M2(nn), M4(nn), M6(nn), T1(nn), T2(nn);
  for (size_t k = 0; k < nn; k++) {
    A[k] = M[k] * scale;
    E[k] = D[k] * scale;
  }
  matmul(n, A.data(), A.data(), A2.data());
  matmul(n, A2.data(), A2.data(), A4.data());
  matmul(n, A4.data(), A2.data(), A6.data());
  // M2 = A E + E A, M4 = A2 M2 + M2 A2, M6 = A4 M2 + M4 A2 (derivatives of A2, A4, A6)
  matmul(n, A.data(), E.data(), M2.data());
  matmul(n, E.data(), A.data(), T1.data());
  for (size_t k = 0; k < nn; k++) M2[k] += T1[k];
  matmul(n, A2.data(), M2.data(), M4.data());
  matmul(n, M2.data(), A2.data(), T1.data());
  for (size_t k = 0; k < nn; k++) M4[k] += T1[k];
  matmul(n, A4.data(), M2.data(), M6.data());
  matmul(n, M4.data(), A2.data(), T1.data());
  for (size_t k = 0; k < nn; k++) M6[k] += T1[k];
  std::vector<double> W1(nn), Z1(nn), W(nn), U(nn), V(nn), Lw(nn), Lu(nn), Lv(nn);
  // W = A6 W1 + W2 (U = A W); V = A6 Z1 + Z2
  for (size_t k = 0; k < nn; k++) {
    W1[k] = b[13] * A6[k] + b[11] * A4[k] + b[9] * A2[k];
    Z1[k] = b[12] * A6[k] + b[10] * A4[k] + b[8] * A2[k];
  }
  matmul(n, A6.data(), W1.data(), W.data());
  for (size_t k = 0; k < nn; k++) W[k] += b[7] * A6[k] + b[5] * A4[k] + b[3] * A2[k];
  for (int i = 0; i < n; i++) W[(size_t)i * n + i] += b[1];
  matmul(n, A.data(), W.data(), U.data());
  matmul(n, A6.data(), Z1.data(), V.data());
  for (size_t k = 0; k < nn; k++) V[k] += b[6] * A6[k] + b[4] * A4[k] + b[2] * A2[k];
  for (int i = 0; i < n; i++) V[(size_t)i * n + i] += b[0];
  // Lw = A6 Lw1 + M6 W1 + Lw2;  Lu = A Lw + E W;  Lv = A6 Lz1 + M6 Z1 + Lz2
  for (size_t k = 0; k < nn; k++) T1[k] = b[13] * M6[k] + b[11] * M4[k] + b[9] * M2[k];
  matmul(n, A6.data(), T1.data(), Lw.data());
  matmul(n, M6.data(), W1.data(), T2.data());
  for (size_t k = 0; k < nn; k++) Lw[k] += T2[k] + b[7] * M6[k] + b[5] * M4[k] + b[3] * M2[k];
  matmul(n, A.data(), Lw.data(), Lu.data());
  matmul(n, E.data(), W.data(), T2.data());
  for (size_t k = 0; k < nn; k++) Lu[k] += T2[k];
  for (size_t k = 0; k < nn; k++) T1[k] = b[12] * M6[k] + b[10] * M4[k] + b[8] * M2[k];
  matmul(n, A6.data(), T1.data(), Lv.data());
  matmul(n, M6.data(), Z1.data(), T2.data());
  for (size_t k = 0; k < nn; k++) Lv[k] += T2[k] + b[6] * M6[k] + b[4] * M4[k] + b[2] * M2[k];
  std::vector<double> P(nn), R(nn), L(nn);
  for (size_t k = 0; k < nn; k++) {
    P[k] = V[k] - U[k];
    R[k] = V[k] + U[k];
  }
  if (!solve(n, P, R)) return false;
  matmul(n, Lu.data(), R.data(), T1.data());   // (Lu - Lv) R
  matmul(n, Lv.data(), R.data(), T2.data());
  for (size_t k = 0; k < nn; k++) L[k] = Lu[k] + Lv[k] + T1[k] - T2[k];
  if (!solve(n, P, L)) return false;
  for (int k = 0; k < s; k++) {
    matmul(n, R.data(), L.data(), T1.data());
    matmul(n, L.data(), R.data(), T2.data());
    for (size_t i = 0; i < nn; i++) L[i] = T1[i] + T2[i];
    matmul(n, R.data(), R.data(), T1.data());
    R.swap(T1);
  }
  if (Rout) memcpy(Rout, R.data(), nn * sizeof(double));
  memcpy(Lout, L.data(), nn * sizeof(double));
  return true;
}

}  // namespace

// exported for the statistics path (cg_stats.cpp)
namespace cgh {
bool expm(int n, const double *M, double *E) { return expm_pade13(n, M, E); }
bool expm_frechet(int n, const double *M, const double *D, double *R, double *L) {
  return expm_frechet_pade13(n, M, D, R, L);
}
void set_error(const char *msg) { g_err = msg; }
}  // namespace cgh

extern "C" {

const char *cg_last_error(void) { return g_err.c_str(); }

int cg_encoded_bytes(const cg_shape *shape, const cg_codec *codec, uint64_t *payload_bytes,
                     uint64_t *meta_bytes, uint64_t *header_bytes) {
  g_err.clear();
  int rc = check_shape(shape);
  if (rc) return rc;
  if ((rc = check_codec(codec, shape))) return rc;
  uint64_t p, m;
  byte_counts(shape, codec, &p, &m);
  if (payload_bytes) *payload_bytes = p;
  if (meta_bytes) *meta_bytes = m;
  if (header_bytes) *header_bytes = (uint64_t)CG_HEADER_BYTES * shape->layers * shape->kv;
  return CG_OK;
}

int cg_write_header(const cg_shape *shape, const cg_codec *codec, int32_t layer, int32_t kv,
                    void *header_host, uint64_t cap) {
  g_err.clear();
  int rc = check_shape(shape);
  if (rc) return rc;
  if ((rc = check_codec(codec, shape))) return rc;
  if (!header_host) return fail(CG_E_INVAL, "header buffer is NULL");
  if (cap < CG_HEADER_BYTES) return fail(CG_E_SIZE, "header buffer smaller than CG_HEADER_BYTES");
  if (layer < 0 || layer >= shape->layers || kv < 0 || kv >= shape->kv)
    return fail(CG_E_SHAPE, "layer/kv index out of range");
  uint8_t h[CG_HEADER_BYTES];
  memset(h, 0, sizeof h);
  memcpy(h, "CGKV", 4);
  // magic "CGKV", 11 int32 (version, backend, bits, block_tokens, residual,
  // dtype, layer, kv, batch, heads, head_dim), 2 int64 (tokens, capacity)
  int32_t i32[11] = {1, codec->backend, codec->bits, codec->block_tokens, codec->residual_tokens,
                     shape->dtype, layer, kv, shape->batch, shape->heads, shape->head_dim};
  memcpy(h + 4, i32, sizeof i32);
  int64_t i64[2] = {shape->tokens, shape->token_capacity};
  memcpy(h + 4 + sizeof i32, i64, sizeof i64);
  memcpy(header_host, h, CG_HEADER_BYTES);
  return CG_OK;
}

int cg_encode(const cg_shape *shape, const void *kv, const cg_gauge *gauge, const cg_codec *codec,
              int64_t t0, int64_t nt, void *payload, uint64_t payload_cap, void *meta,
              uint64_t meta_cap, void *stream) {
  g_err.clear();
  int rc;
  if ((rc = check_shape(shape))) return rc;
  if ((rc = check_codec(codec, shape))) return rc;
  if ((rc = check_gauge(gauge, shape, codec))) return rc;
  if ((rc = check_rows(shape, codec, t0, nt))) return rc;
  if (!kv || !payload) return fail(CG_E_INVAL, "kv or payload is NULL");
  if (misaligned(kv) || misaligned(payload) || misaligned(meta))
    return fail(CG_E_INVAL, "kv, payload and meta must be 16-byte aligned");
  uint64_t need_p, need_m;
  byte_counts(shape, codec, &need_p, &need_m);
  if (payload_cap < need_p) return fail(CG_E_SIZE, "payload_cap %llu < %llu",
                                        (unsigned long long)payload_cap, (unsigned long long)need_p);
  if (need_m && (!meta || meta_cap < need_m))
    return fail(CG_E_SIZE, "metadata buffer missing or smaller than %llu", (unsigned long long)need_m);
  if (nt == 0) return CG_OK;
  hipStream_t s = (hipStream_t)stream;
  const bool bf16 = shape->dtype == CG_DTYPE_BF16;
  const int g = gauge->group;
  hipError_t e = hipSuccess;
  switch (codec->backend) {
    case CG_BACKEND_NONE:
      e = cgk::gauge_rows_launch(bf16, false, false, g, kv, gauge->G, payload, tile_args(shape, t0, nt), s);
      break;
    case CG_BACKEND_ZFP:
      e = cgk::zfp_encode_launch(codec->bits, bf16, g, kv, gauge->G, (uint8_t *)payload,
                                 tile_args(shape, t0, nt), s);
      break;
    case CG_BACKEND_BLOCK_UNIFORM:
    case CG_BACKEND_KIVI: {
      cgq::QuantArgs q = cgq::make_args(shape->token_capacity, shape->tokens, t0, nt, n_fields(shape),
                                        shape->batch, shape->heads, codec->backend, codec->bits,
                                        codec->block_tokens, codec->residual_tokens, shape->kv);
      e = cgq::encode_launch(q, bf16, g, kv, gauge->G, (uint8_t *)payload, (float *)meta, s);
      break;
    }
  }
  if (e != hipSuccess) return hip_fail(e, "cg_encode launch");
  return CG_OK;
}

namespace {

// error partials per field of a decode launch (one per workgroup)
int64_t err_per_field(const cg_shape *s, const cg_codec *c, int g, int64_t nt) {
  const int64_t tiles = (nt + cgk::TILE_T - 1) / cgk::TILE_T;
  // zfp with the full-head gauge: bf16 storage takes the split bf16 kernels
  // (16-tile chunks), fp32 storage the fmaf-chain kernels (chunked like g <= 32)
  if (c->backend == CG_BACKEND_ZFP && g == 128 && s->dtype == CG_DTYPE_BF16)
    return (tiles + cgk::ZFP128_CHUNK - 1) / cgk::ZFP128_CHUNK;
  if (c->backend == CG_BACKEND_ZFP) {
    const int ct = cgk::zfp_chunk_tiles(n_fields(s), tiles);
    return (tiles + ct - 1) / ct;
  }
  if (c->backend == CG_BACKEND_BLOCK_UNIFORM || c->backend == CG_BACKEND_KIVI) {
    const int ct = cgq::quant_chunk_tiles(g, n_fields(s), tiles);
    return (tiles + ct - 1) / ct;
  }
  return tiles;
}

// keep: bit s set = fields with K/V index s are written in gauged coordinates
// (their inverse gauge is skipped); only without error sums
int decode_impl(const cg_shape *shape, const void *payload, uint64_t payload_cap, const void *meta,
                uint64_t meta_cap, const cg_gauge *gauge, const cg_codec *codec, int64_t t0,
                int64_t nt, void *kv_out, const void *ref, double *epart, int keep, void *stream) {
  int rc;
  if ((rc = check_shape(shape))) return rc;
  if ((rc = check_codec(codec, shape))) return rc;
  if ((rc = check_gauge(gauge, shape, codec))) return rc;
  if ((rc = check_rows(shape, codec, t0, nt))) return rc;
  if (!kv_out || !payload) return fail(CG_E_INVAL, "kv_out or payload is NULL");
  if (misaligned(kv_out) || misaligned(payload) || misaligned(meta) || misaligned(ref))
    return fail(CG_E_INVAL, "kv_out, payload, meta and kv_ref must be 16-byte aligned");
  uint64_t need_p, need_m;
  byte_counts(shape, codec, &need_p, &need_m);
  if (payload_cap < need_p) return fail(CG_E_SIZE, "payload_cap %llu < %llu",
                                        (unsigned long long)payload_cap, (unsigned long long)need_p);
  if (need_m && (!meta || meta_cap < need_m))
    return fail(CG_E_SIZE, "metadata buffer missing or smaller than %llu", (unsigned long long)need_m);
  if (nt == 0) return CG_OK;
  hipStream_t s = (hipStream_t)stream;
  const bool bf16 = shape->dtype == CG_DTYPE_BF16;
  const int64_t F = n_fields(shape), BH = (int64_t)shape->batch * shape->heads;
  // one launch over the fields {(i / sel) * step + base + i % sel : i < count}
  auto launch = [&](int g, int64_t count, int64_t sel, int64_t step, int64_t base) {
    switch (codec->backend) {
      case CG_BACKEND_NONE:
      case CG_BACKEND_ZFP: {
        cgk::TileArgs ta = tile_args(shape, t0, nt);
        ta.grid = count * ta.tiles;
        ta.fsel = sel; ta.fstep = step; ta.fbase = base;
        ta.ref = ref;
        ta.epart = epart;
        if (codec->backend == CG_BACKEND_NONE)
          return cgk::gauge_rows_launch(false, bf16, true, g, payload, gauge->G, kv_out, ta, s);
        return cgk::zfp_decode_launch(codec->bits, bf16, g, (const uint8_t *)payload, gauge->G,
                                      kv_out, ta, s);
      }
      default: {
        cgq::QuantArgs q = cgq::make_args(shape->token_capacity, shape->tokens, t0, nt, count,
                                          shape->batch, shape->heads, codec->backend, codec->bits,
                                          codec->block_tokens, codec->residual_tokens, shape->kv);
        q.fsel = sel; q.fstep = step; q.fbase = base;
        q.ref = ref;
        q.epart = epart;
        return cgq::decode_launch(q, bf16, g, (const uint8_t *)payload, (const float *)meta,
                                  gauge->G, kv_out, s);
      }
    }
  };
  const int all = (1 << shape->kv) - 1;
  hipError_t e;
  if (gauge->group == 0 || keep == 0) {
    e = launch(gauge->group, F, F, F, 0);
  } else if (keep == all) {
    e = launch(0, F, F, F, 0);
  } else {
    // two kinds, one kept: per layer, B*H fields of each kind
    const int kept = keep == 1 ? 0 : 1;
    const int64_t per = F / 2;
    e = launch(gauge->group, per, BH, 2 * BH, (1 - kept) * BH);
    if (e == hipSuccess) e = launch(0, per, BH, 2 * BH, kept * BH);
  }
  if (e != hipSuccess) return hip_fail(e, "cg_decode launch");
  return CG_OK;
}

}  // namespace

int cg_decode(const cg_shape *shape, const void *payload, uint64_t payload_cap, const void *meta,
              uint64_t meta_cap, const cg_gauge *gauge, const cg_codec *codec, int64_t t0,
              int64_t nt, void *kv_out, void *stream) {
  g_err.clear();
  return decode_impl(shape, payload, payload_cap, meta, meta_cap, gauge, codec, t0, nt, kv_out,
                     nullptr, nullptr, 0, stream);
}

int cg_decode_gauged(const cg_shape *shape, const void *payload, uint64_t payload_cap,
                     const void *meta, uint64_t meta_cap, const cg_gauge *gauge,
                     const cg_codec *codec, int64_t t0, int64_t nt, int32_t keep, void *kv_out,
                     void *stream) {
  g_err.clear();
  if (!shape) return fail(CG_E_INVAL, "shape is NULL");
  if (keep < 0 || keep > CG_KEEP_KEYS + CG_KEEP_VALUES)
    return fail(CG_E_INVAL, "keep %d: use CG_KEEP_KEYS | CG_KEEP_VALUES", keep);
  if ((keep & CG_KEEP_VALUES) && shape->kv != 2)
    return fail(CG_E_INVAL, "CG_KEEP_VALUES needs a shape with kv = 2");
  return decode_impl(shape, payload, payload_cap, meta, meta_cap, gauge, codec, t0, nt, kv_out,
                     nullptr, nullptr, keep, stream);
}

int cg_decode_error_workspace_bytes(const cg_shape *shape, const cg_gauge *gauge,
                                    const cg_codec *codec, int64_t t0, int64_t nt, size_t *bytes) {
  g_err.clear();
  int rc;
  if (!bytes) return fail(CG_E_INVAL, "bytes is NULL");
  if ((rc = check_shape(shape))) return rc;
  if ((rc = check_codec(codec, shape))) return rc;
  if ((rc = check_gauge(gauge, shape, codec))) return rc;
  if ((rc = check_rows(shape, codec, t0, nt))) return rc;
  *bytes = (size_t)n_fields(shape) * (size_t)err_per_field(shape, codec, gauge->group, nt) * 3 * sizeof(double);
  return CG_OK;
}

int cg_decode_error(const cg_shape *shape, const void *payload, uint64_t payload_cap,
                    const void *meta, uint64_t meta_cap, const cg_gauge *gauge,
                    const cg_codec *codec, int64_t t0, int64_t nt, void *kv_out,
                    const void *kv_ref, void *workspace, size_t ws_bytes, cg_field_error *err,
                    void *stream) {
  g_err.clear();
  size_t need = 0;
  int rc = cg_decode_error_workspace_bytes(shape, gauge, codec, t0, nt, &need);
  if (rc) return rc;
  if (!kv_ref || !err) return fail(CG_E_INVAL, "kv_ref or err is NULL");
  if (misaligned(workspace) || misaligned(err))
    return fail(CG_E_INVAL, "workspace and err must be 16-byte aligned");
  if (need && (!workspace || ws_bytes < need))
    return fail(CG_E_SIZE, "workspace missing or smaller than %zu bytes", need);
  if (nt == 0) {  // no rows: every field's sums are zero (written by the reduce kernel)
    hipError_t e = cgk::error_reduce_launch(nullptr, n_fields(shape), 0, 0.0, (double *)err,
                                            (hipStream_t)stream);
    return e == hipSuccess ? CG_OK : hip_fail(e, "cg_decode_error reduce");
  }
  double *epart = (double *)workspace;
  rc = decode_impl(shape, payload, payload_cap, meta, meta_cap, gauge, codec, t0, nt, kv_out, kv_ref,
                   epart, 0, stream);
  if (rc) return rc;
  hipError_t e = cgk::error_reduce_launch(epart, n_fields(shape), err_per_field(shape, codec, gauge->group, nt),
                                          (double)nt * shape->head_dim, (double *)err, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "cg_decode_error reduce");
  return CG_OK;
}

}  // extern "C"

namespace {

// Scratch of cg_decode_error_noalloc: the per-workgroup error partials live
// in this file-scope device array instead of a caller workspace.  Host code
// never passes the array's name to a kernel (on the host it is only a
// stand-in for the symbol); it passes the device address that
// hipGetSymbolAddress returns, looked up once per device with that device
// current and cached here.
constexpr int kMaxDevices = 64;
static __device__ __align__(256) double scratch[CG_NOALLOC_SCRATCH_BYTES / sizeof(double)];
std::mutex g_scratch_mu;
double *g_scratch_ptr[kMaxDevices] = {};

int noalloc_scratch(double **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(CG_E_UNSUPPORTED, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(CG_E_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = (double *)p;
  }
  *out = g_scratch_ptr[dev];
  return CG_OK;
}

}  // namespace

extern "C" {

int cg_decode_error_noalloc(const cg_shape *shape, const void *payload, uint64_t payload_cap,
                            const void *meta, uint64_t meta_cap, const cg_gauge *gauge,
                            const cg_codec *codec, int64_t t0, int64_t nt, void *kv_out,
                            const void *kv_ref, cg_field_error *err, void *stream) {
  g_err.clear();
  size_t need = 0;
  int rc = cg_decode_error_workspace_bytes(shape, gauge, codec, t0, nt, &need);
  if (rc) return rc;
  if (need > CG_NOALLOC_SCRATCH_BYTES)
    return fail(CG_E_SIZE, "this call needs %zu bytes of error partials; the built-in scratch "
                           "holds %zu (use cg_decode_error with a workspace)",
                need, (size_t)CG_NOALLOC_SCRATCH_BYTES);
  double *ws = nullptr;
  if ((rc = noalloc_scratch(&ws))) return rc;
  return cg_decode_error(shape, payload, payload_cap, meta, meta_cap, gauge, codec, t0, nt, kv_out,
                         kv_ref, ws, CG_NOALLOC_SCRATCH_BYTES, err, stream);
}

int cg_cache_error_summary(const cg_shape *shape, const cg_field_error *err, cg_cache_error *out) {
  g_err.clear();
  int rc;
  if ((rc = check_shape(shape))) return rc;
  if (!err || !out) return fail(CG_E_INVAL, "err or out is NULL");
  double sse[2] = {0.0, 0.0}, ssr[2] = {0.0, 0.0}, n[2] = {0.0, 0.0}, mx = 0.0;
  const int64_t F = n_fields(shape);
  for (int64_t f = 0; f < F; f++) {
    const int kind = (int)((f / ((int64_t)shape->batch * shape->heads)) % shape->kv);
    sse[kind] += err[f].sse;
    ssr[kind] += err[f].ref_ss;
    n[kind] += err[f].values;
    mx = fmax(mx, err[f].max_abs);
  }
  auto nrmse = [](double e, double r) { return r > 0.0 ? sqrt(e / r) : (e > 0.0 ? INFINITY : 0.0); };
  const double E = sse[0] + sse[1], Rr = ssr[0] + ssr[1], N = n[0] + n[1];
  out->values = N;
  out->mse = N > 0.0 ? E / N : 0.0;
  out->nrmse = nrmse(E, Rr);
  out->key_nrmse = nrmse(sse[0], ssr[0]);
  out->value_nrmse = shape->kv == 2 ? nrmse(sse[1], ssr[1]) : 0.0;
  out->max_abs = mx;
  return CG_OK;
}

int cg_roundtrip(const cg_shape *shape, const void *kv_in, const cg_gauge *gauge,
                 const cg_codec *codec, void *payload, uint64_t payload_cap, void *meta,
                 uint64_t meta_cap, void *kv_out, void *stream) {
  int rc = CG_OK;
  if ((rc = check_shape(shape))) return rc;
  rc = cg_encode(shape, kv_in, gauge, codec, 0, shape->tokens, payload, payload_cap, meta, meta_cap, stream);
  if (rc) return rc;
  return cg_decode(shape, payload, payload_cap, meta, meta_cap, gauge, codec, 0, shape->tokens, kv_out, stream);
}

int cg_gauge_apply(const cg_shape *shape, const void *kv, const cg_gauge *gauge, int32_t direction,
                   float *out, void *stream) {
  g_err.clear();
  int rc;
  if ((rc = check_shape(shape))) return rc;
  if ((rc = check_gauge(gauge, shape, nullptr))) return rc;
  if (!kv || !out) return fail(CG_E_INVAL, "kv or out is NULL");
  if (misaligned(kv) || misaligned(out)) return fail(CG_E_INVAL, "kv and out must be 16-byte aligned");
  if (direction != 0 && direction != 1) return fail(CG_E_INVAL, "direction must be 0 or 1");
  if (shape->tokens == 0) return CG_OK;
  const int64_t tiles = (shape->tokens + cgk::TILE_T - 1) / cgk::TILE_T;
  if (n_fields(shape) * tiles >= ((int64_t)1 << 31)) return fail(CG_E_SHAPE, "grid too large");
  hipStream_t s = (hipStream_t)stream;
  const bool bf16 = shape->dtype == CG_DTYPE_BF16;
  hipError_t e;
  if (gauge->group == 128 && bf16)
    e = cgq::gauge128_rows_launch(bf16, direction == 1, kv, gauge->G, out,
                                  shape->token_capacity, shape->tokens, n_fields(shape),
                                  shape->batch, shape->heads, s);
  else
    e = cgk::gauge_rows_launch(bf16, false, direction == 1, gauge->group, kv, gauge->G, out,
                               tile_args(shape, 0, shape->tokens), s);
  if (e != hipSuccess) return hip_fail(e, "cg_gauge_apply launch");
  return CG_OK;
}

int cg_gauge_heads(const cg_shape *shape, const cg_gauge *gauge, int32_t layer, int32_t kind,
                   int32_t q_heads, int64_t rows, int32_t dtype, const void *x, void *y,
                   void *stream) {
  g_err.clear();
  int rc;
  if ((rc = check_shape(shape))) return rc;
  if ((rc = check_gauge(gauge, shape, nullptr))) return rc;
  if (layer < 0 || layer >= shape->layers || kind < 0 || kind >= shape->kv)
    return fail(CG_E_SHAPE, "layer %d / kind %d outside the cache shape", layer, kind);
  if (q_heads <= 0 || q_heads % shape->heads || q_heads > 65535)
    return fail(CG_E_SHAPE, "q_heads %d must be a positive multiple of heads %d", q_heads,
                shape->heads);
  if (rows < 0) return fail(CG_E_SHAPE, "rows < 0");
  if (dtype != CG_DTYPE_F32 && dtype != CG_DTYPE_BF16) return fail(CG_E_INVAL, "bad dtype %d", dtype);
  if (rows == 0) return CG_OK;
  if (!x || !y) return fail(CG_E_INVAL, "x or y is NULL");
  if ((((uintptr_t)x | (uintptr_t)y) & (dtype == CG_DTYPE_BF16 ? 1u : 3u)) != 0)
    return fail(CG_E_INVAL, "x and y must be aligned to their element size");
  if ((rows + 63) / 64 >= ((int64_t)1 << 31)) return fail(CG_E_SHAPE, "too many rows");
  const int64_t esz = dtype == CG_DTYPE_BF16 ? 2 : 4, bytes = rows * q_heads * shape->head_dim * esz;
  const char *xb = (const char *)x, *yb = (const char *)y;
  if (xb < yb + bytes && yb < xb + bytes) return fail(CG_E_INVAL, "x and y overlap");
  const int g = gauge->group;
  const float *gk = g ? gauge->G + ((int64_t)layer * shape->kv + kind) * shape->heads *
                                       shape->head_dim * g
                      : nullptr;
  hipError_t e = cgk::gauge_heads_launch(g, dtype == CG_DTYPE_BF16, x, gk, y, rows, q_heads,
                                         q_heads / shape->heads, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "cg_gauge_heads launch");
  return CG_OK;
}

int cg_gauge_from_skew(int64_t n, int32_t g, const double *A_host, float *G_host) {
  g_err.clear();
  if (!A_host || !G_host) return fail(CG_E_INVAL, "A or G is NULL");
  if (n < 0 || g < 1 || g > 1024) return fail(CG_E_SHAPE, "bad n or g");
  const size_t gg = (size_t)g * g;
  std::vector<double> S(gg), E(gg);
  for (int64_t m = 0; m < n; m++) {
    const double *A = A_host + (size_t)m * gg;
    for (int i = 0; i < g; i++)
      for (int j = 0; j < g; j++) S[(size_t)i * g + j] = A[(size_t)i * g + j] - A[(size_t)j * g + i];
    if (!expm_pade13(g, S.data(), E.data())) return fail(CG_E_INTERNAL, "singular Pade denominator");
    for (size_t k = 0; k < gg; k++) G_host[(size_t)m * gg + k] = (float)E[k];
  }
  return CG_OK;
}

}  // extern "C"
