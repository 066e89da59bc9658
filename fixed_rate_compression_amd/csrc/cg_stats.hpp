// Internal interface of the gauge-fit statistics path.  Not part of the
// public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cgh {
bool expm(int n, const double *M, double *E);
// R = exp(M) (may be NULL) and L = the Frechet derivative of exp at M in direction D
bool expm_frechet(int n, const double *M, const double *D, double *R, double *L);
void set_error(const char *msg);
}  // namespace cgh

namespace cgs {

struct StatsArgs {
  int64_t tcap, tokens;
  int64_t chunks;           // workgroups per field
  int32_t tiles_per_chunk;  // 64-token tiles per workgroup
  int32_t batch, heads;
  int32_t grad;             // also compute Gamma = dL/dG
  float tau2;              // tau^2
  float inv_tau2;          // 1 / tau^2
  float lam_f_nb;           // lambda_f / N_b (blocks per field)
  float lam_r_nc;           // lambda_r / N_c (coefficients per field)
};

hipError_t stats_launch(bool bf16, int g, const void *kv, const float *gauges, const float *C128,
                        const float *C16, const float *rtab, double *part, float *gpart,
                        double *out, const StatsArgs &a, int64_t fields, hipStream_t s);

}  // namespace cgs
