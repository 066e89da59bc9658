// Host side of gauge training and of the coordinate controls ("Codec-Gauge",
// arXiv HTML: gauge-training paragraph -- the gauge parameters are optimized
// with AdamW; main-grid and coordinate-control paragraphs -- identity,
// random orthogonal, Hadamard, DCT and PCA/KLT gauges with the learned
// gauge's block structure, KLT from the uncentered second moment).
//   cg_adamw_update              one AdamW step (decoupled weight decay)
//   cg_gauge_control             Hadamard / DCT / Q of a QR / KLT gauges, fp64 -> fp32
//   cg_second_moment(_workspace_bytes)  per-group second moments on the device
#include <hip/hip_runtime.h>
#include <math.h>
#include <string.h>

#include <algorithm>
#include <string>
#include <vector>

#include "../../include/codec_gauge.h"
#include "cg_launch.hpp"
#include "cg_stats.hpp"

namespace {

int fail(int code, const std::string &msg) {
  cgh::set_error(msg.c_str());
  return code;
}

bool pow2(int g) { return g > 0 && (g & (g - 1)) == 0; }

// Householder QR of the n x n matrix a (row-major, destroyed); q receives Q
// with the signs chosen so that diag(R) > 0
void qr_q(int n, std::vector<double> &a, std::vector<double> &q) {
  q.assign((size_t)n * n, 0.0);
  for (int i = 0; i < n; i++) q[(size_t)i * n + i] = 1.0;
  std::vector<double> v(n);
  for (int k = 0; k < n; k++) {
    double nx = 0.0;
    for (int i = k; i < n; i++) nx += a[(size_t)i * n + k] * a[(size_t)i * n + k];
    nx = sqrt(nx);
    if (nx == 0.0) continue;
    const double x0 = a[(size_t)k * n + k];
    const double alpha = x0 >= 0.0 ? -nx : nx;
    double nv = 0.0;
    for (int i = k; i < n; i++) {
      v[i] = a[(size_t)i * n + k] - (i == k ? alpha : 0.0);
      nv += v[i] * v[i];
    }
    nv = sqrt(nv);
    if (nv == 0.0) continue;
    for (int i = k; i < n; i++) v[i] /= nv;
    for (int j = 0; j < n; j++) {  // a <- (I - 2 v v^T) a
      double d = 0.0;
      for (int i = k; i < n; i++) d += v[i] * a[(size_t)i * n + j];
      for (int i = k; i < n; i++) a[(size_t)i * n + j] -= 2.0 * d * v[i];
    }
    for (int i = 0; i < n; i++) {  // q <- q (I - 2 v v^T)
      double d = 0.0;
      for (int j = k; j < n; j++) d += q[(size_t)i * n + j] * v[j];
      for (int j = k; j < n; j++) q[(size_t)i * n + j] -= 2.0 * d * v[j];
    }
  }
  for (int j = 0; j < n; j++)
    if (a[(size_t)j * n + j] < 0.0)
      for (int i = 0; i < n; i++) q[(size_t)i * n + j] = -q[(size_t)i * n + j];
}

// cyclic Jacobi eigenvalue iteration of the symmetric matrix a (destroyed):
// w = eigenvalues, columns of vec = eigenvectors
void jacobi_eigh(int n, std::vector<double> &a, std::vector<double> &w, std::vector<double> &vec) {
  vec.assign((size_t)n * n, 0.0);
  for (int i = 0; i < n; i++) vec[(size_t)i * n + i] = 1.0;
  auto A = [&](int i, int j) -> double & { return a[(size_t)i * n + j]; };
  for (int sweep = 0; sweep < 100; sweep++) {
    double off = 0.0, diag = 0.0;
    for (int i = 0; i < n; i++) {
      diag += A(i, i) * A(i, i);
      for (int j = i + 1; j < n; j++) off += A(i, j) * A(i, j);
    }
    if (off <= 1e-32 * diag || off == 0.0) break;
    for (int p = 0; p < n; p++)
      for (int q = p + 1; q < n; q++) {
        const double apq = A(p, q);
        if (apq == 0.0) continue;
        const double theta = (A(q, q) - A(p, p)) / (2.0 * apq);
        const double t = (theta >= 0.0 ? 1.0 : -1.0) / (fabs(theta) + sqrt(theta * theta + 1.0));
        const double c = 1.0 / sqrt(t * t + 1.0), s = t * c;
        for (int k = 0; k < n; k++) {  // columns p, q
          const double akp = A(k, p), akq = A(k, q);
          A(k, p) = c * akp - s * akq;
          A(k, q) = s * akp + c * akq;
        }
        for (int k = 0; k < n; k++) {  // rows p, q
          const double apk = A(p, k), aqk = A(q, k);
          A(p, k) = c * apk - s * aqk;
          A(q, k) = s * apk + c * aqk;
        }
        for (int k = 0; k < n; k++) {
          const double vkp = vec[(size_t)k * n + p], vkq = vec[(size_t)k * n + q];
          vec[(size_t)k * n + p] = c * vkp - s * vkq;
          vec[(size_t)k * n + q] = s * vkp + c * vkq;
        }
      }
  }
  w.resize(n);
  for (int i = 0; i < n; i++) w[i] = A(i, i);
}

int64_t n_fields(const cg_shape *s) { return (int64_t)s->layers * s->kv * s->batch * s->heads; }

int check_moment_args(const cg_shape *s, int g) {
  if (!s) return fail(CG_E_INVAL, "shape is NULL");
  if (s->layers < 1 || s->batch < 1 || s->heads < 1 || (s->kv != 1 && s->kv != 2))
    return fail(CG_E_SHAPE, "layers, batch, heads must be >= 1 and kv 1 or 2");
  if (s->dtype != CG_DTYPE_F32 && s->dtype != CG_DTYPE_BF16) return fail(CG_E_INVAL, "bad dtype");
  if (s->head_dim != 128) return fail(CG_E_UNSUPPORTED, "head_dim must be 128");
  if (s->tokens < 0 || s->tokens > s->token_capacity) return fail(CG_E_SHAPE, "bad token counts");
  if (g != 8 && g != 16 && g != 32 && g != 128)
    return fail(CG_E_UNSUPPORTED, "second moments are built for g = 8, 16, 32, 128");
  return CG_OK;
}

}  // namespace

extern "C" {

int cg_adamw_update(int64_t n, double *param, const double *grad, double *m, double *v,
                    int64_t step, double lr, double beta1, double beta2, double eps,
                    double weight_decay) {
  cgh::set_error("");
  if (n < 0 || step < 1) return fail(CG_E_INVAL, "need n >= 0 and step >= 1");
  if (n && (!param || !grad || !m || !v)) return fail(CG_E_INVAL, "NULL array");
  const double c1 = 1.0 - pow(beta1, (double)step), c2 = 1.0 - pow(beta2, (double)step);
  for (int64_t i = 0; i < n; i++) {
    double p = param[i] * (1.0 - lr * weight_decay);
    m[i] = beta1 * m[i] + (1.0 - beta1) * grad[i];
    v[i] = beta2 * v[i] + (1.0 - beta2) * grad[i] * grad[i];
    const double mh = m[i] / c1, vh = v[i] / c2;
    param[i] = p - lr * mh / (sqrt(vh) + eps);
  }
  return CG_OK;
}

int cg_gauge_control(int32_t kind, int64_t n, int32_t g, const double *M_host, float *G_host) {
  cgh::set_error("");
  if (n < 0 || g < 1 || !G_host) return fail(CG_E_INVAL, "need n >= 0, g >= 1 and G");
  const size_t gg = (size_t)g * g;
  std::vector<double> out(gg), a, q, w, vec;
  for (int64_t b = 0; b < n; b++) {
    switch (kind) {
      case CG_CONTROL_IDENTITY:
        for (int i = 0; i < g; i++)
          for (int j = 0; j < g; j++) out[(size_t)i * g + j] = i == j ? 1.0 : 0.0;
        break;
      case CG_CONTROL_HADAMARD: {  // Sylvester order: entry sign = parity of i & j
        if (!pow2(g)) return fail(CG_E_UNSUPPORTED, "Hadamard needs g a power of two");
        const double s = 1.0 / sqrt((double)g);
        for (int i = 0; i < g; i++)
          for (int j = 0; j < g; j++) out[(size_t)i * g + j] = (__builtin_popcount(i & j) & 1) ? -s : s;
        break;
      }
      case CG_CONTROL_DCT: {  // orthonormal DCT-II, rows = frequencies
        const double pi = 3.14159265358979323846;
        for (int k = 0; k < g; k++)
          for (int j = 0; j < g; j++)
            out[(size_t)k * g + j] =
                sqrt((k ? 2.0 : 1.0) / g) * cos(pi * (2.0 * j + 1.0) * k / (2.0 * g));
        break;
      }
      case CG_CONTROL_ORTHONORMALIZE:
        if (!M_host) return fail(CG_E_INVAL, "M is NULL");
        a.assign(M_host + b * gg, M_host + (b + 1) * gg);
        qr_q(g, a, q);
        out = q;
        break;
      case CG_CONTROL_KLT: {
        if (!M_host) return fail(CG_E_INVAL, "M is NULL");
        a.assign(M_host + b * gg, M_host + (b + 1) * gg);
        jacobi_eigh(g, a, w, vec);
        std::vector<int> order(g);
        for (int i = 0; i < g; i++) order[i] = i;
        std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return w[x] > w[y]; });
        for (int r = 0; r < g; r++) {
          const int c = order[r];
          int im = 0;
          for (int i = 1; i < g; i++)
            if (fabs(vec[(size_t)i * g + c]) > fabs(vec[(size_t)im * g + c])) im = i;
          const double sg = vec[(size_t)im * g + c] < 0.0 ? -1.0 : 1.0;
          for (int i = 0; i < g; i++) out[(size_t)r * g + i] = sg * vec[(size_t)i * g + c];
        }
        break;
      }
      default:
        return fail(CG_E_INVAL, "unknown control kind");
    }
    for (size_t i = 0; i < gg; i++) G_host[b * gg + i] = (float)out[i];
  }
  return CG_OK;
}

int cg_second_moment_workspace_bytes(const cg_shape *shape, int32_t g, size_t *bytes) {
  cgh::set_error("");
  int rc = check_moment_args(shape, g);
  if (rc) return rc;
  if (!bytes) return fail(CG_E_INVAL, "bytes is NULL");
  *bytes = (size_t)n_fields(shape) * cgk::moment_chunks(shape->tokens) * 128 * g * sizeof(double);
  return CG_OK;
}

int cg_second_moment(const cg_shape *shape, const void *kv, int32_t g, void *workspace,
                     size_t ws_bytes, double *M_host, void *stream) {
  size_t need = 0;
  int rc = cg_second_moment_workspace_bytes(shape, g, &need);
  if (rc) return rc;
  if (!kv || !M_host) return fail(CG_E_INVAL, "kv or M is NULL");
  if (((uintptr_t)kv | (uintptr_t)workspace) & 15u)
    return fail(CG_E_INVAL, "kv and workspace must be 16-byte aligned");
  if (!workspace || ws_bytes < need) return fail(CG_E_SIZE, "workspace missing or too small");
  const int64_t F = n_fields(shape), E = 128 * (int64_t)g, ngauge = (int64_t)shape->layers * shape->kv * shape->heads;
  memset(M_host, 0, (size_t)ngauge * E * sizeof(double));
  if (shape->tokens == 0) return CG_OK;
  hipStream_t s = (hipStream_t)stream;
  double *part = (double *)workspace;
  hipError_t e = cgk::second_moment_launch(shape->dtype == CG_DTYPE_BF16, g, kv, shape->token_capacity,
                                           shape->tokens, F, part, s);
  const int64_t chunks = cgk::moment_chunks(shape->tokens);
  std::vector<double> host((size_t)F * chunks * E);
  if (e == hipSuccess) e = hipMemcpyAsync(host.data(), part, host.size() * 8, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(CG_E_HIP, std::string("cg_second_moment: ") + hipGetErrorString(e));
  // fields (l, s, b, h) -> gauge (l, s, h): sum over the batch and the chunks in order
  for (int64_t f = 0; f < F; f++) {
    const int64_t ls = f / ((int64_t)shape->batch * shape->heads), h = f % shape->heads;
    double *dst = M_host + (size_t)(ls * shape->heads + h) * E;
    for (int64_t c = 0; c < chunks; c++) {
      const double *src = host.data() + ((size_t)f * chunks + c) * E;
      for (int64_t i = 0; i < E; i++) dst[i] += src[i];
    }
  }
  return CG_OK;
}

}  // extern "C"
