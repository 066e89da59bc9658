// LDS read-pattern probe for gfx950 (measurement only; nothing on the codec
// path uses it).  A workgroup of 256 threads fills a 64-row tile in LDS and
// then repeatedly reads it as matrix-core A operands: wave lane l reads the
// 16 bytes at row 16 mt + l % 16, dword column 4 (l / 16) + 16 ks (mt, ks =
// 0..3: 16 ds_read_b128 per trip), the access of the codec kernels' tile
// products.  The row pitch (in dwords) and an optional XOR swizzle of the
// 16-byte column chunk vary by kind:
//   0: pitch 68 (272 B, the kernels' current pitch)   1: pitch 76
//   2: pitch 72   3: pitch 64, chunk ^ (row % 8)   4: pitch 64, no swizzle
//   5: pitch 64, chunk ^ ((row / 2) % 8)
// Time and the LDS bank-conflict counter per kind show which layout the
// hardware serves without conflicts.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

template <int KIND>
__device__ __forceinline__ int lds_off(int row, int col4) {  // col4: 16-byte chunk index 0..31
  if constexpr (KIND == 0) return row * 68 + 4 * col4;
  if constexpr (KIND == 1) return row * 76 + 4 * col4;
  if constexpr (KIND == 2) return row * 72 + 4 * col4;
  if constexpr (KIND == 3) return row * 64 + 4 * (col4 ^ (row & 7));
  if constexpr (KIND == 4) return row * 64 + 4 * col4;
  return row * 64 + 4 * (col4 ^ ((row >> 1) & 7));
}

template <int KIND>
__global__ __launch_bounds__(256) void k_lds(unsigned *out, int iters) {
  __shared__ __align__(16) unsigned tile[64 * 76];
  for (int i = threadIdx.x; i < 64 * 76; i += 256) tile[i] = i * 2654435761u;
  __syncthreads();
  const int lane = threadIdx.x & 63;
  uint4 acc = make_uint4(0, 0, 0, 0);
  for (int it = 0; it < iters; it++) {
#pragma unroll
    for (int ks = 0; ks < 4; ks++)
#pragma unroll
      for (int mt = 0; mt < 4; mt++) {
        const uint4 v = *(const uint4 *)(tile + lds_off<KIND>(16 * mt + (lane & 15), (lane >> 4) + 4 * ks));
        acc.x ^= v.x; acc.y += v.y; acc.z ^= v.z; acc.w += v.w;
      }
    __builtin_amdgcn_s_barrier();  // keep the waves' trips in step
  }
  out[blockIdx.x * 256 + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

typedef void (*lds_fn)(unsigned *, int);
const lds_fn kLds[] = {k_lds<0>, k_lds<1>, k_lds<2>, k_lds<3>, k_lds<4>, k_lds<5>};
constexpr int kBlocks = 2048;

}  // namespace

extern "C" {

int cgprobe_lds_kinds() { return (int)(sizeof(kLds) / sizeof(kLds[0])); }

// ms of one launch of LDS read pattern `kind` (`iters` trips, kBlocks x 256
// threads, after one untimed launch); `out` holds kBlocks * 256 uint32
int cgprobe_lds(int kind, int iters, void *out, void *stream, float *ms) {
  if (kind < 0 || kind >= cgprobe_lds_kinds() || iters <= 0 || !out || !ms) return -1;
  hipStream_t st = (hipStream_t)stream;
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return -2;
  hipLaunchKernelGGL(kLds[kind], dim3(kBlocks), dim3(256), 0, st, (unsigned *)out, iters);
  (void)hipEventRecord(e0, st);
  hipLaunchKernelGGL(kLds[kind], dim3(kBlocks), dim3(256), 0, st, (unsigned *)out, iters);
  (void)hipEventRecord(e1, st);
  float t = -1.f;
  if (hipEventSynchronize(e1) != hipSuccess || hipEventElapsedTime(&t, e0, e1) != hipSuccess) t = -1.f;
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  *ms = t;
  return t < 0.f ? -2 : 0;
}

}  // extern "C"
