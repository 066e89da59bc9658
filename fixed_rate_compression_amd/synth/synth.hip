// Synthetic KV generator (input preparation only; none of the method's
// arithmetic).  Value model: x[t][c] = sigma_c * y_t, y an AR(1) process
// along tokens with unit stationary variance, driven by N(0,1) noise from
// Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as
// easy as 1, 2, 3", SC'11) and the Box-Muller transform.
//
// One thread per (field, channel) walks the tokens sequentially; a wave's 64
// threads cover 64 consecutive channels, so every store is a contiguous row
// segment.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

struct u4 {
  uint32_t x, y, z, w;
};

__device__ inline void mulhilo(uint32_t a, uint32_t b, uint32_t &hi, uint32_t &lo) {
  uint64_t p = (uint64_t)a * (uint64_t)b;
  hi = (uint32_t)(p >> 32);
  lo = (uint32_t)p;
}

// Philox4x32 with 10 rounds: multipliers 0xD2511F53 / 0xCD9E8D57, key
// (Weyl) increments 0x9E3779B9 / 0xBB67AE85.
__device__ inline u4 philox4x32_10(u4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; r++) {
    uint32_t hi0, lo0, hi1, lo1;
    mulhilo(0xD2511F53u, c.x, hi0, lo0);
    mulhilo(0xCD9E8D57u, c.z, hi1, lo1);
    u4 n;
    n.x = hi1 ^ c.y ^ k0;
    n.y = lo1;
    n.z = hi0 ^ c.w ^ k1;
    n.w = lo0;
    c = n;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}

__device__ inline float u01(uint32_t v) {  // in (0, 1)
  return ((float)(v >> 8) + 0.5f) * (1.0f / 16777216.0f);
}

__device__ inline void box_muller(uint32_t a, uint32_t b, float &z0, float &z1) {
  float r = sqrtf(-2.0f * logf(u01(a)));
  float th = 6.28318530717958647692f * u01(b);
  z0 = r * cosf(th);
  z1 = r * sinf(th);
}

__device__ inline uint16_t to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  uint32_t keep = u >> 16, rest = u & 0xFFFFu;
  if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u))) keep += 1u;
  return (uint16_t)keep;
}

template <bool BF16>
__global__ void k_generate(void *out, int64_t n_fields, int64_t Tcap, int64_t T, int d,
                           float rho, uint32_t seed, const int64_t *field_ids,
                           const float *scales) {
  int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= n_fields * d) return;
  int64_t f = gid / d;
  int c = (int)(gid % d);
  uint64_t fid = (uint64_t)field_ids[f];
  uint32_t k0 = seed, k1 = (uint32_t)fid ^ (uint32_t)(fid >> 32) * 0x85EBCA6Bu;
  float sig = scales[f * d + c];
  float cc = sqrtf(1.0f - rho * rho);
  float y = 0.0f;
  for (int64_t t = 0; t < T; t += 4) {
    u4 ctr = {(uint32_t)c, (uint32_t)(t >> 2), (uint32_t)((uint64_t)t >> 34), 0x5EEDu};
    u4 r = philox4x32_10(ctr, k0, k1);
    float e[4];
    box_muller(r.x, r.y, e[0], e[1]);
    box_muller(r.z, r.w, e[2], e[3]);
#pragma unroll
    for (int j = 0; j < 4; j++) {
      if (t + j >= T) break;                       // T need not be a multiple of 4
      y = (t + j == 0) ? e[j] : rho * y + cc * e[j];
      float v = sig * y;
      int64_t idx = (f * Tcap + t + j) * d + c;
      if (BF16)
        ((uint16_t *)out)[idx] = to_bf16_rne(v);
      else
        ((float *)out)[idx] = v;
    }
  }
}

}  // namespace

extern "C" int cgsynth_generate(void *out, int64_t n_fields, int64_t Tcap, int64_t T, int d,
                                float rho, uint32_t seed, const int64_t *field_ids,
                                const float *scales, int dtype, hipStream_t stream) {
  if (!out || !field_ids || !scales || n_fields <= 0 || d <= 0 || T < 0 || T > Tcap ||
      (dtype != 0 && dtype != 1))
    return -1;
  int64_t threads = n_fields * d;
  int block = 256;
  int64_t grid = (threads + block - 1) / block;
  if (dtype == 1)
    hipLaunchKernelGGL(k_generate<true>, dim3((unsigned)grid), dim3(block), 0, stream, out,
                       n_fields, Tcap, T, d, rho, seed, field_ids, scales);
  else
    hipLaunchKernelGGL(k_generate<false>, dim3((unsigned)grid), dim3(block), 0, stream, out,
                       n_fields, Tcap, T, d, rho, seed, field_ids, scales);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}
