// cg_gauge_fit_stats / cg_gauge_fit_grad / cg_stats_workspace_bytes: host side of the gauge-fit
// statistics ("Codec-Gauge", arXiv HTML, frequency-objective and
// gauge-training paragraphs).  The host builds G = exp(A - A^T) and the DCT
// tables in fp64 (rounded to fp32 for the device), launches the statistics
// kernel and its fixed-order reduction, and finishes the gradient:
// dL/dA = Psi - Psi^T with Psi = L_exp(S^T, Gamma), the Frechet derivative of
// exp at S^T in the direction Gamma = dL/dG (the upper-right block of
// exp([[S^T, Gamma], [0, S^T]]), Van Loan 1978; Higham 2008, Thm 3.6),
// evaluated with exp itself in one Pade pass (Al-Mohy and Higham 2009).
#include <hip/hip_runtime.h>
#include <math.h>
#include <string.h>

#include <string>
#include <thread>
#include <vector>

#include "../../include/codec_gauge.h"
#include "cg_stats.hpp"

namespace {

constexpr int kD = 128;
constexpr int kTileT = 64;
constexpr int kTilesPerChunk = 64;  // 4096 tokens per workgroup

int fail(int code, const std::string &msg) {
  cgh::set_error(msg.c_str());
  return code;
}

int64_t n_fields(const cg_shape *s) { return (int64_t)s->layers * s->kv * s->batch * s->heads; }

struct Layout {
  size_t G, C128, C16, rtab, part, gpart, out, total;
  int64_t chunks;
  int ng;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// host worker threads for n independent items: at most 16 and at most n
unsigned host_threads(int64_t n) {
  unsigned nth = std::thread::hardware_concurrency();
  nth = nth == 0 ? 1 : (nth > 16 ? 16 : nth);
  if (n < 1) return 1;
  if ((int64_t)nth > n) nth = (unsigned)n;
  return nth;
}

Layout layout(const cg_shape *s, int g) {
  Layout L{};
  const int64_t F = n_fields(s);
  const int64_t ngauge = (int64_t)s->layers * s->kv * s->heads;
  const int64_t ntiles = (s->tokens + kTileT - 1) / kTileT;
  L.chunks = (ntiles + kTilesPerChunk - 1) / kTilesPerChunk;
  if (L.chunks < 1) L.chunks = 1;
  L.ng = g == 32 ? 16 * 256 : (g == 16 || g == 8 ? 8 * 256 : 0);
  size_t off = 0;
  L.G = off;     off += align256((size_t)(g ? ngauge * kD * g : 1) * 4);
  L.C128 = off;  off += align256((size_t)kD * kD * 4);
  L.C16 = off;   off += align256(16 * 16 * 4);
  L.rtab = off;  off += align256((size_t)16 * kD * 4);
  L.part = off;  off += align256((size_t)F * L.chunks * 4 * 8);
  L.gpart = off; off += align256((size_t)F * L.chunks * (L.ng ? L.ng : 1) * 4);
  L.out = off;   off += align256((size_t)F * (4 + L.ng) * 8);
  L.total = off;
  return L;
}

int validate(const cg_shape *s, int g, int T_b) {
  if (!s) return fail(CG_E_INVAL, "shape is NULL");
  if (s->layers < 1 || s->batch < 1 || s->heads < 1 || (s->kv != 1 && s->kv != 2))
    return fail(CG_E_SHAPE, "layers, batch, heads must be >= 1 and kv 1 or 2");
  if (s->dtype != CG_DTYPE_F32 && s->dtype != CG_DTYPE_BF16) return fail(CG_E_INVAL, "bad dtype");
  if (s->head_dim != kD) return fail(CG_E_UNSUPPORTED, "head_dim must be 128");
  if (s->tokens < 0 || s->tokens > s->token_capacity) return fail(CG_E_SHAPE, "bad token counts");
  if (T_b != 16) return fail(CG_E_UNSUPPORTED, "T_b must be 16");
  if (s->tokens % T_b) return fail(CG_E_SHAPE, "tokens must be a multiple of T_b");
  if (g != 0 && g != 8 && g != 16 && g != 32)
    return fail(CG_E_UNSUPPORTED, "gauge group must be 0, 8, 16 or 32");
  return CG_OK;
}

// Psi = L_exp(M, E), the Frechet derivative of exp at M in the direction E
// (equal to the upper-right block of exp([[M, E], [0, M]]))
bool frechet(int n, const double *M, const double *E, double *Psi) {
  return cgh::expm_frechet(n, M, E, nullptr, Psi);
}

}  // namespace

extern "C" int cg_stats_workspace_bytes(const cg_shape *shape, int32_t g, int32_t T_b, size_t *bytes) {
  int rc = validate(shape, g, T_b);
  if (rc) return rc;
  if (!bytes) return fail(CG_E_INVAL, "bytes is NULL");
  *bytes = layout(shape, g).total;
  return CG_OK;
}

namespace {

// per_gauge: dA_host holds one gradient per gauge (layer, kind, head), the sum
// over the batch of its fields' gradients, else one per field
int fit_stats(const cg_shape *shape, const void *kv, int32_t g, const double *A_host, int32_t T_b,
              float tau, float lambda_f, float lambda_r, void *workspace, size_t ws_bytes,
              cg_stats *out_host, double *dA_host, bool per_gauge, void *stream) {
  int rc = validate(shape, g, T_b);
  if (rc) return rc;
  if (!kv || !workspace || !out_host) return fail(CG_E_INVAL, "kv, workspace or out is NULL");
  if (((uintptr_t)kv | (uintptr_t)workspace) & 15u)
    return fail(CG_E_INVAL, "kv and workspace must be 16-byte aligned");
  if (g != 0 && !A_host) return fail(CG_E_INVAL, "A is NULL");
  if (!(tau > 0.0f)) return fail(CG_E_INVAL, "tau must be positive");
  const Layout L = layout(shape, g);
  if (ws_bytes < L.total) return fail(CG_E_SIZE, "workspace smaller than cg_stats_workspace_bytes");
  const int64_t F = n_fields(shape);
  const int R = g ? kD / g : 0;
  const int64_t ngauge = (int64_t)shape->layers * shape->kv * shape->heads;
  hipStream_t s = (hipStream_t)stream;
  uint8_t *ws = (uint8_t *)workspace;

  // host tables: gauges (fp64 expm -> fp32), DCT matrices, normalized radius
  std::vector<float> Gh(g ? (size_t)ngauge * R * g * g : 0);
  std::vector<double> Sfull;
  if (g) {  // G = exp(A - A^T) per group, spread over host threads
    const int64_t nq = ngauge * R;
    auto build = [&](int64_t q0, int64_t q1, int *bad) {
      std::vector<double> S((size_t)g * g), E((size_t)g * g);
      for (int64_t q = q0; q < q1; q++) {
        const double *A = A_host + (size_t)q * g * g;
        for (int i = 0; i < g; i++)
          for (int j = 0; j < g; j++) S[(size_t)i * g + j] = A[(size_t)i * g + j] - A[(size_t)j * g + i];
        if (!cgh::expm(g, S.data(), E.data())) { *bad = 1; return; }
        for (size_t k = 0; k < (size_t)g * g; k++) Gh[(size_t)q * g * g + k] = (float)E[k];
      }
    };
    const unsigned nth = host_threads(nq);
    std::vector<std::thread> pool;
    std::vector<int> bad(nth, 0);
    for (unsigned t = 0; t < nth; t++) pool.emplace_back(build, nq * t / nth, nq * (t + 1) / nth, &bad[t]);
    for (auto &th : pool) th.join();
    for (int b : bad)
      if (b) return fail(CG_E_INTERNAL, "expm failed");
  }
  std::vector<float> C128((size_t)kD * kD), C16(256), rt((size_t)16 * kD);
  const double pi = 3.14159265358979323846;
  for (int v = 0; v < kD; v++)
    for (int c = 0; c < kD; c++)
      C128[(size_t)v * kD + c] = (float)((v ? sqrt(2.0 / kD) : sqrt(1.0 / kD)) * cos(pi * (2 * c + 1) * v / (2.0 * kD)));
  for (int u = 0; u < 16; u++)
    for (int t = 0; t < 16; t++)
      C16[u * 16 + t] = (float)((u ? sqrt(2.0 / 16) : sqrt(1.0 / 16)) * cos(pi * (2 * t + 1) * u / 32.0));
  for (int u = 0; u < 16; u++)
    for (int v = 0; v < kD; v++) {
      const double a = u / 15.0, b = v / (kD - 1.0);
      rt[(size_t)u * kD + v] = (float)(sqrt(a * a + b * b) / sqrt(2.0));
    }
  hipError_t e = hipSuccess;
  if (g) e = hipMemcpyAsync(ws + L.G, Gh.data(), Gh.size() * 4, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipMemcpyAsync(ws + L.C128, C128.data(), C128.size() * 4, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipMemcpyAsync(ws + L.C16, C16.data(), C16.size() * 4, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipMemcpyAsync(ws + L.rtab, rt.data(), rt.size() * 4, hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return fail(CG_E_HIP, std::string("upload: ") + hipGetErrorString(e));

  const int64_t nb = shape->tokens / T_b;
  const double nc = (double)shape->tokens * kD;
  cgs::StatsArgs a{};
  a.tcap = shape->token_capacity;
  a.tokens = shape->tokens;
  a.chunks = L.chunks;
  a.tiles_per_chunk = kTilesPerChunk;
  a.batch = shape->batch;
  a.heads = shape->heads;
  a.grad = (dA_host != nullptr && g != 0) ? 1 : 0;
  a.tau2 = (float)((double)tau * tau);
  a.inv_tau2 = (float)(1.0 / ((double)tau * tau));
  a.lam_f_nb = nb ? (float)((double)lambda_f / (double)nb) : 0.f;
  a.lam_r_nc = nc > 0 ? (float)((double)lambda_r / nc) : 0.f;
  if (nb > 0) {
    e = cgs::stats_launch(shape->dtype == CG_DTYPE_BF16, g, kv, (const float *)(ws + L.G),
                          (const float *)(ws + L.C128), (const float *)(ws + L.C16),
                          (const float *)(ws + L.rtab), (double *)(ws + L.part),
                          (float *)(ws + L.gpart), (double *)(ws + L.out), a, F, s);
    if (e != hipSuccess) return fail(CG_E_HIP, std::string("stats launch: ") + hipGetErrorString(e));
  }
  const int width = 4 + L.ng;
  std::vector<double> res((size_t)F * width, 0.0);
  if (nb > 0) {
    e = hipMemcpyAsync(res.data(), ws + L.out, res.size() * 8, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return fail(CG_E_HIP, std::string("readback: ") + hipGetErrorString(e));
  }
  for (int64_t f = 0; f < F; f++) {
    const double *r = res.data() + (size_t)f * width;
    cg_stats st;
    st.L_freq = nb ? r[0] / (double)nb : 0.0;
    st.L_rate = nc > 0 ? r[1] / nc : 0.0;
    st.L = (double)lambda_f * st.L_freq + (double)lambda_r * st.L_rate;
    st.sum_E = r[2];
    out_host[f] = st;
  }
  if (!a.grad) return CG_OK;

  // dA per field (or per gauge) and group: Psi = L_exp(S^T, Gamma),
  // dA = Psi - Psi^T.  Per gauge, Gamma is the sum over the batch (b = 0, 1,
  // ... in order) of its fields' Gamma: the Frechet derivative is linear in
  // its direction, so this is the sum of the fields' gradients.
  const int gg = g * g;
  const int64_t B = shape->batch, H = shape->heads;
  const int64_t items = per_gauge ? ngauge : F;
  auto work = [&](int64_t i0, int64_t i1, int *bad) {
    std::vector<double> St(gg), Gam(gg), Psi(gg);
    for (int64_t it = i0; it < i1; it++) {
      // item -> its gauge and the fields whose Gamma it takes
      const int64_t gidx = per_gauge ? it : (it / (B * H)) * H + it % H;
      const int64_t ls = gidx / H, h = gidx % H;
      const int64_t fb0 = per_gauge ? ls * B * H + h : it;   // first field
      const int64_t nfb = per_gauge ? B : 1;                 // fields, H apart
      for (int q = 0; q < R; q++) {
        const double *A = A_host + ((size_t)gidx * R + q) * gg;
        for (int i = 0; i < g; i++)
          for (int j = 0; j < g; j++) St[i * g + j] = A[j * g + i] - A[i * g + j];  // S^T
        // Gamma tiles: g = 16 -> tile q holds [16][16]; g = 32 -> tiles 4q + 2a + b;
        // g = 8 -> diagonal block q % 2 of tile q / 2
        for (int i = 0; i < g; i++)
          for (int j = 0; j < g; j++) {
            double v = 0.0;
            for (int64_t b = 0; b < nfb; b++) {
              const double *r = res.data() + (size_t)(fb0 + b * H) * width + 4;
              if (g == 16) v += r[q * 256 + i * 16 + j];
              else if (g == 8) v += r[(q / 2) * 256 + (8 * (q % 2) + i) * 16 + 8 * (q % 2) + j];
              else v += r[(q * 4 + (i / 16) * 2 + (j / 16)) * 256 + (i % 16) * 16 + (j % 16)];
            }
            Gam[i * g + j] = v;
          }
        if (!frechet(g, St.data(), Gam.data(), Psi.data())) { *bad = 1; return; }
        double *out = dA_host + ((size_t)it * R + q) * gg;
        for (int i = 0; i < g; i++)
          for (int j = 0; j < g; j++) out[i * g + j] = Psi[i * g + j] - Psi[j * g + i];
      }
    }
  };
  const unsigned nth = host_threads(items);
  std::vector<std::thread> pool;
  std::vector<int> bad(nth, 0);
  for (unsigned t = 0; t < nth; t++) {
    const int64_t i0 = items * t / nth, i1 = items * (t + 1) / nth;
    pool.emplace_back(work, i0, i1, &bad[t]);
  }
  for (auto &th : pool) th.join();
  for (int b : bad)
    if (b) return fail(CG_E_INTERNAL, "Frechet derivative failed");
  return CG_OK;
}

}  // namespace

extern "C" int cg_gauge_fit_stats(const cg_shape *shape, const void *kv, int32_t g,
                                  const double *A_host, int32_t T_b, float tau, float lambda_f,
                                  float lambda_r, void *workspace, size_t ws_bytes,
                                  cg_stats *out_host, double *dA_host, void *stream) {
  return fit_stats(shape, kv, g, A_host, T_b, tau, lambda_f, lambda_r, workspace, ws_bytes,
                   out_host, dA_host, false, stream);
}

extern "C" int cg_gauge_fit_grad(const cg_shape *shape, const void *kv, int32_t g,
                                 const double *A_host, int32_t T_b, float tau, float lambda_f,
                                 float lambda_r, void *workspace, size_t ws_bytes,
                                 cg_stats *out_host, double *dA_gauge_host, void *stream) {
  if (g != 0 && !dA_gauge_host) return fail(CG_E_INVAL, "dA is NULL");
  return fit_stats(shape, kv, g, A_host, T_b, tau, lambda_f, lambda_r, workspace, ws_bytes,
                   out_host, dA_gauge_host, true, stream);
}

/* dL/dA from dL/dG for G = exp(A - A^T), per matrix (host, fp64). */
extern "C" int cg_gauge_grad(int64_t n, int32_t g, const double *A_host, const double *dG_host,
                             double *dA_host) {
  if (n < 0 || g < 1 || (n && (!A_host || !dG_host || !dA_host)))
    return fail(CG_E_INVAL, "need n >= 0, g >= 1 and non-NULL arrays");
  const int gg = g * g;
  std::vector<double> St(gg), Psi(gg);
  for (int64_t q = 0; q < n; q++) {
    const double *A = A_host + (size_t)q * gg;
    for (int i = 0; i < g; i++)
      for (int j = 0; j < g; j++) St[i * g + j] = A[j * g + i] - A[i * g + j];  // S^T
    if (!frechet(g, St.data(), dG_host + (size_t)q * gg, Psi.data()))
      return fail(CG_E_INTERNAL, "Frechet derivative failed");
    double *out = dA_host + (size_t)q * gg;
    for (int i = 0; i < g; i++)
      for (int j = 0; j < g; j++) out[i * g + j] = Psi[i * g + j] - Psi[j * g + i];
  }
  return CG_OK;
}

