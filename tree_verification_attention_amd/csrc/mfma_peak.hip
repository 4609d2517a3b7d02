// mfma_peak.hip -- the matrix-core rate this GPU sustains, for the measurement beside the
// prefix pass's own figures (a peak taken on the machine rather than from its data sheet).
//
// Every wave keeps eight independent accumulator chains of v_mfma_f32_16x16x32_bf16 on
// register operands (no memory traffic inside the loop), so the products issue back to
// back; each lane stores one sum at the end so nothing is optimised away.  One product is
// 16 x 16 x 32 multiply-adds = 16384 flops.
#include "../../include/hta.h"
#include "hta_internal.h"

namespace hta {

namespace {

constexpr int kPeakThreads = 512;  // 8 waves: two per SIMD, as in the prefix pass
constexpr int kPeakChains = 8;

__global__ __launch_bounds__(kPeakThreads) void mfma_peak_loop(float* out, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(0.001f * (float)(lane + e));
    b[e] = (__bf16)(0.002f * (float)(lane - e));
  }
  f32x4 acc[kPeakChains];
#pragma unroll
  for (int c = 0; c < kPeakChains; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, (float)c};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < kPeakChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kPeakChains; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  out[(size_t)blockIdx.x * kPeakThreads + threadIdx.x] = s;
}

}  // namespace

}  // namespace hta

extern "C" {

hta_status hta_mfma_peak_probe(int32_t blocks, int32_t iters, float* out, void* stream,
                               double* flops) {
  if (!out || !flops) return HTA_ERR_NULL;
  if (blocks < 1 || blocks > (1 << 20) || iters < 1 || iters > (1 << 24)) return HTA_ERR_SHAPE;
  if (((uintptr_t)out & 15u) != 0) return HTA_ERR_ALIGN;
  hipLaunchKernelGGL(hta::mfma_peak_loop, dim3(blocks), dim3(hta::kPeakThreads), 0,
                     (hipStream_t)stream, out, iters);
  if (hipGetLastError() != hipSuccess) return HTA_ERR_HIP;
  *flops = (double)blocks * (hta::kPeakThreads / 64) * hta::kPeakChains * (double)iters * 16384.0;
  return HTA_OK;
}

}  // extern "C"
