// Streaming HBM kernels with no arithmetic: the practical memory ceiling the
// codec kernels are measured against.  Each moves bytes in a fixed
// read : write proportion with 16-byte vector loads and stores, every wave
// touching contiguous memory:
//   copy   1 : 1   (a plain copy of the KV tensor)
//   enc    4 : 1   (the proportion of gauge + encode at 4 bits/value on bf16:
//                   2 B read and 0.5 B written per value)
//   dec    1 : 4   (decode + inverse gauge: 0.5 B read, 2 B written)
// A workgroup of 256 threads handles chunks of RIN x 256 input and
// ROUT x 256 output pieces of 16 B (thread t takes pieces k * 256 + t), one
// chunk per workgroup.  The stored values depend on the loaded ones (an XOR)
// so no load can be dropped.  Measurement only: nothing on the codec path
// calls these kernels.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int NT = 256;

template <int RIN, int ROUT>
__global__ __launch_bounds__(NT) void k_stream(const uint4 *__restrict__ src, uint4 *__restrict__ dst) {
  const int64_t c = blockIdx.x;
  const uint4 *s = src + c * (RIN * NT) + threadIdx.x;
  uint4 *d = dst + c * (ROUT * NT) + threadIdx.x;
  uint4 a[RIN];
#pragma unroll
  for (int k = 0; k < RIN; k++) a[k] = s[k * NT];
  uint4 x = a[0];
#pragma unroll
  for (int k = 1; k < RIN; k++) {
    x.x ^= a[k].x; x.y ^= a[k].y; x.z ^= a[k].z; x.w ^= a[k].w;
  }
#pragma unroll
  for (int k = 0; k < ROUT; k++) d[k * NT] = make_uint4(x.x ^ k, x.y, x.z, x.w);
}

// The decode-shaped kernel with the row stores of the full-head decoders:
// the 16 KB output chunk is a tile of 64 rows x 256 B, and lane l of wave w
// writes, for mt = 0..3, the 16 B at row 16 mt + l % 16, byte 64 w + 16 (l /
// 16): each store instruction covers 64 contiguous bytes of 16 rows, and the
// two halves of a 128-byte line come from two waves.
__global__ __launch_bounds__(NT) void k_stream_rows(const uint4 *__restrict__ src, uint4 *__restrict__ dst) {
  const int64_t c = blockIdx.x;
  const uint4 x = src[c * NT + threadIdx.x];
  unsigned char *d = (unsigned char *)(dst + c * (4 * NT));
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
#pragma unroll
  for (int mt = 0; mt < 4; mt++)
    *(uint4 *)(d + (16 * mt + (l & 15)) * 256 + 64 * w + 16 * (l >> 4)) = make_uint4(x.x ^ mt, x.y, x.z, x.w);
}

// k_stream_rows with non-temporal stores (NT), or with 128-byte row segments
// (W128: wave w owns rows 32 (w / 2) .. + 31 and bytes 128 (w % 2) .. + 127;
// store k covers rows 32 (w / 2) + 8 k + l / 8, bytes 128 (w % 2) + 16 (l % 8))
template <bool NTS, bool W128>
__global__ __launch_bounds__(NT) void k_stream_rows2(const uint4 *__restrict__ src, uint4 *__restrict__ dst) {
  const int64_t c = blockIdx.x;
  const uint4 x = src[c * NT + threadIdx.x];
  unsigned char *d = (unsigned char *)(dst + c * (4 * NT));
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
#pragma unroll
  for (int k = 0; k < 4; k++) {
    const int off = W128 ? (32 * (w >> 1) + 8 * k + (l >> 3)) * 256 + 128 * (w & 1) + 16 * (l & 7)
                         : (16 * k + (l & 15)) * 256 + 64 * w + 16 * (l >> 4);
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = {x.x ^ (unsigned)k, x.y, x.z, x.w};
    if (NTS)
      __builtin_nontemporal_store(v, (u32x4 *)(d + off));
    else
      *(u32x4 *)(d + off) = v;
  }
}

}  // namespace

// mode 0 copy, 1 enc-shaped (4 : 1), 2 dec-shaped (1 : 4), 3 dec-shaped with
// the row stores of k_stream_rows, 4 the same non-temporal, 5 dec-shaped with
// 128-byte row segments per wave; src_bytes is the
// input size and must be a multiple of RIN x 4096 B; dst must hold
// src_bytes x ROUT / RIN bytes.  Returns 0, or -1 for bad arguments, or the
// HIP error code of the launch.
extern "C" int cgprobe_stream(int mode, const void *src, uint64_t src_bytes, void *dst,
                              uint64_t dst_bytes, hipStream_t stream) {
  const int rin = mode == 1 ? 4 : 1, rout = mode >= 2 ? 4 : 1;
  if (mode < 0 || mode > 5 || !src || !dst || ((uintptr_t)src | (uintptr_t)dst) & 15u) return -1;
  const uint64_t chunk = (uint64_t)rin * NT * 16;
  if (src_bytes == 0 || src_bytes % chunk) return -1;
  const uint64_t chunks = src_bytes / chunk;
  if (chunks >= (1ull << 31) || dst_bytes < chunks * rout * NT * 16) return -1;
  const dim3 grid((unsigned)chunks), block(NT);
  if (mode == 0)
    hipLaunchKernelGGL((k_stream<1, 1>), grid, block, 0, stream, (const uint4 *)src, (uint4 *)dst);
  else if (mode == 1)
    hipLaunchKernelGGL((k_stream<4, 1>), grid, block, 0, stream, (const uint4 *)src, (uint4 *)dst);
  else if (mode == 2)
    hipLaunchKernelGGL((k_stream<1, 4>), grid, block, 0, stream, (const uint4 *)src, (uint4 *)dst);
  else if (mode == 3)
    hipLaunchKernelGGL(k_stream_rows, grid, block, 0, stream, (const uint4 *)src, (uint4 *)dst);
  else if (mode == 4)
    hipLaunchKernelGGL((k_stream_rows2<true, false>), grid, block, 0, stream, (const uint4 *)src, (uint4 *)dst);
  else
    hipLaunchKernelGGL((k_stream_rows2<false, true>), grid, block, 0, stream, (const uint4 *)src, (uint4 *)dst);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? 0 : (int)e;
}
