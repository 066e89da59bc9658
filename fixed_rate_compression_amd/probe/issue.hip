// Instruction-issue probes for gfx950 (measurement only; nothing on the codec
// path uses them).
//
// cgprobe_issue(kind): every lane runs 8 independent register chains of one
// VALU instruction form, 32 instructions per loop trip, 2048 workgroups of
// 256 threads (8 waves per SIMD).  The instructions are written as ALU-only
// inline asm so the compiler cannot fold or re-select them; they read and
// write registers only.  Rate = wave64 instructions per second; a SIMD
// issues one per 4 cycles, so 614.4 G/s is single issue at 2.4 GHz and
// rates near twice that mean two waves' instructions were paired.
//
// cgprobe_overlap(mode): matrix-core chains and VALU fma chains alone, in
// the same wave, or in separate waves of one workgroup (half the work each),
// for the fp32 16x16x4 and the bf16 16x16x32 forms.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

#define CH8(INS, SC)                                                                          \
  asm volatile(INS : "+v"(a0) : SC(s), "v"(t)); asm volatile(INS : "+v"(a1) : SC(s), "v"(t)); \
  asm volatile(INS : "+v"(a2) : SC(s), "v"(t)); asm volatile(INS : "+v"(a3) : SC(s), "v"(t)); \
  asm volatile(INS : "+v"(a4) : SC(s), "v"(t)); asm volatile(INS : "+v"(a5) : SC(s), "v"(t)); \
  asm volatile(INS : "+v"(a6) : SC(s), "v"(t)); asm volatile(INS : "+v"(a7) : SC(s), "v"(t));

#define ISSUE_KERNEL(NAME, INS, SC)                                                          \
  __global__ __launch_bounds__(256) void NAME(unsigned *out, int iters, unsigned s, unsigned t) { \
    unsigned a0 = threadIdx.x, a1 = a0 + 1, a2 = a0 + 2, a3 = a0 + 3, a4 = a0 + 4,            \
             a5 = a0 + 5, a6 = a0 + 6, a7 = a0 + 7;                                         \
    for (int i = 0; i < iters; i++) { CH8(INS, SC) CH8(INS, SC) CH8(INS, SC) CH8(INS, SC) } \
    out[blockIdx.x * 256 + threadIdx.x] = a0 ^ a1 ^ a2 ^ a3 ^ a4 ^ a5 ^ a6 ^ a7;            \
  }

ISSUE_KERNEL(k_xor_v, "v_xor_b32 %0, %0, %1", "v")
ISSUE_KERNEL(k_xor_s, "v_xor_b32 %0, %1, %0", "s")
ISSUE_KERNEL(k_xor_lit, "v_xor_b32 %0, 0x80808080, %0", "v")
ISSUE_KERNEL(k_add_v, "v_add_u32 %0, %0, %1", "v")
ISSUE_KERNEL(k_bitop3_v, "v_bitop3_b32 %0, %0, %1, %2 bitop3:0x6c", "v")
ISSUE_KERNEL(k_bitop3_s, "v_bitop3_b32 %0, %0, %1, %2 bitop3:0x6c", "s")
ISSUE_KERNEL(k_lshr_c, "v_lshrrev_b32 %0, 1, %0", "v")
ISSUE_KERNEL(k_lshl_c, "v_lshlrev_b32 %0, 1, %0", "v")
ISSUE_KERNEL(k_bfe, "v_bfe_u32 %0, %0, %1, %2", "v")
ISSUE_KERNEL(k_perm, "v_perm_b32 %0, %0, %1, %2", "v")
ISSUE_KERNEL(k_lshl_or, "v_lshl_or_b32 %0, %0, %1, %2", "v")
ISSUE_KERNEL(k_bcnt, "v_bcnt_u32_b32 %0, %0, %1", "v")
ISSUE_KERNEL(k_ffbh, "v_ffbh_u32 %0, %0", "v")
ISSUE_KERNEL(k_min, "v_min_u32 %0, %0, %1", "v")
ISSUE_KERNEL(k_fma_v, "v_fma_f32 %0, %0, %1, %2", "v")
ISSUE_KERNEL(k_fma_s, "v_fma_f32 %0, %1, %0, %2", "s")
ISSUE_KERNEL(k_cvt, "v_cvt_f32_i32 %0, %0", "v")

typedef float f4 __attribute__((ext_vector_type(4)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));

// MODE 0: matrix only, 1: VALU only, 2: both in each wave, 3: even waves
// matrix, odd waves VALU.  BF: bf16 16x16x32 (8 x 4 per trip, 512 cycles) or
// fp32 16x16x4 (4 per trip, 128 cycles); VALU: 128 or 32 fmas per trip.
template <int MODE, bool BF>
__global__ __launch_bounds__(256) void k_overlap(float *out, int iters, float s) {
  f4 c0 = {0, 0, 0, 0}, c1 = c0, c2 = c0, c3 = c0;
  float x = threadIdx.x * 1e-3f, y0 = x + 1, y1 = x + 2, y2 = x + 3, y3 = x + 4, y4 = x + 5,
        y5 = x + 6, y6 = x + 7, y7 = x + 8;
  const bool do_m = MODE == 0 || MODE == 2 || (MODE == 3 && (threadIdx.x >> 6) % 2 == 0);
  const bool do_v = MODE == 1 || MODE == 2 || (MODE == 3 && (threadIdx.x >> 6) % 2 == 1);
  for (int i = 0; i < iters; i++) {
    if (do_m) {
      if constexpr (BF) {
        const b8 bx = {(__bf16)x, (__bf16)s, (__bf16)x, (__bf16)s, (__bf16)x, (__bf16)s, (__bf16)x, (__bf16)s};
#pragma unroll
        for (int r = 0; r < 8; r++) {
          c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bx, bx, c0, 0, 0, 0);
          c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bx, bx, c1, 0, 0, 0);
          c2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bx, bx, c2, 0, 0, 0);
          c3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bx, bx, c3, 0, 0, 0);
        }
      } else {
        c0 = __builtin_amdgcn_mfma_f32_16x16x4f32(x, s, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_16x16x4f32(x, s, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_16x16x4f32(x, s, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_16x16x4f32(x, s, c3, 0, 0, 0);
      }
    }
    if (do_v) {
#pragma unroll
      for (int r = 0; r < (BF ? 16 : 4); r++) {
        y0 = fmaf(y0, s, x); y1 = fmaf(y1, s, x); y2 = fmaf(y2, s, x); y3 = fmaf(y3, s, x);
        y4 = fmaf(y4, s, x); y5 = fmaf(y5, s, x); y6 = fmaf(y6, s, x); y7 = fmaf(y7, s, x);
      }
    }
  }
  out[blockIdx.x * 256 + threadIdx.x] =
      c0.x + c1.y + c2.z + c3.w + y0 + y1 + y2 + y3 + y4 + y5 + y6 + y7;
}

typedef void (*issue_fn)(unsigned *, int, unsigned, unsigned);
const issue_fn kIssue[] = {k_xor_v, k_xor_s, k_xor_lit, k_add_v, k_bitop3_v, k_bitop3_s,
                           k_lshr_c, k_lshl_c, k_bfe, k_perm, k_lshl_or, k_bcnt, k_ffbh,
                           k_min, k_fma_v, k_fma_s, k_cvt};
constexpr int kBlocks = 2048;

float timed(hipStream_t st, void (*launch)(hipStream_t, void *), void *arg) {
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return -1.f;
  launch(st, arg);  // warm-up
  (void)hipEventRecord(e0, st);
  launch(st, arg);
  (void)hipEventRecord(e1, st);
  float ms = -1.f;
  if (hipEventSynchronize(e1) != hipSuccess || hipEventElapsedTime(&ms, e0, e1) != hipSuccess) ms = -1.f;
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  return ms;
}

struct IssueArg { int kind, iters; unsigned *out; };
struct OverlapArg { int mode, iters; float *out; };

void launch_issue(hipStream_t st, void *p) {
  const IssueArg *a = (const IssueArg *)p;
  hipLaunchKernelGGL(kIssue[a->kind], dim3(kBlocks), dim3(256), 0, st, a->out, a->iters, 0x3f800001u,
                     0x03020100u);
}

void launch_overlap(hipStream_t st, void *p) {
  const OverlapArg *a = (const OverlapArg *)p;
  const int it = a->iters;
  switch (a->mode) {
    case 0: hipLaunchKernelGGL((k_overlap<0, false>), dim3(kBlocks), dim3(256), 0, st, a->out, it, 0.999f); break;
    case 1: hipLaunchKernelGGL((k_overlap<1, false>), dim3(kBlocks), dim3(256), 0, st, a->out, it, 0.999f); break;
    case 2: hipLaunchKernelGGL((k_overlap<2, false>), dim3(kBlocks), dim3(256), 0, st, a->out, it, 0.999f); break;
    case 3: hipLaunchKernelGGL((k_overlap<3, false>), dim3(kBlocks), dim3(256), 0, st, a->out, it, 0.999f); break;
    case 4: hipLaunchKernelGGL((k_overlap<0, true>), dim3(kBlocks), dim3(256), 0, st, a->out, it / 4, 0.999f); break;
    case 5: hipLaunchKernelGGL((k_overlap<1, true>), dim3(kBlocks), dim3(256), 0, st, a->out, it / 4, 0.999f); break;
    case 6: hipLaunchKernelGGL((k_overlap<2, true>), dim3(kBlocks), dim3(256), 0, st, a->out, it / 4, 0.999f); break;
    case 7: hipLaunchKernelGGL((k_overlap<3, true>), dim3(kBlocks), dim3(256), 0, st, a->out, it / 4, 0.999f); break;
  }
}

}  // namespace

extern "C" {

int cgprobe_issue_kinds() { return (int)(sizeof(kIssue) / sizeof(kIssue[0])); }

// ms of one launch of issue form `kind` (32 instructions per trip, `iters`
// trips, kBlocks x 256 threads); `out` holds kBlocks * 256 uint32
int cgprobe_issue(int kind, int iters, void *out, void *stream, float *ms) {
  if (kind < 0 || kind >= cgprobe_issue_kinds() || iters <= 0 || !out || !ms) return -1;
  IssueArg a{kind, iters, (unsigned *)out};
  *ms = timed((hipStream_t)stream, launch_issue, &a);
  return *ms < 0.f ? -2 : 0;
}

// ms of one launch of overlap mode 0..7 (see k_overlap); `out` holds
// kBlocks * 256 floats
int cgprobe_overlap(int mode, int iters, void *out, void *stream, float *ms) {
  if (mode < 0 || mode > 7 || iters <= 0 || !out || !ms) return -1;
  OverlapArg a{mode, iters, (float *)out};
  *ms = timed((hipStream_t)stream, launch_overlap, &a);
  return *ms < 0.f ? -2 : 0;
}

}  // extern "C"
