// Matrix-core ceiling measured on the part itself, to set beside the
// published dense bf16 peak: every wavefront issues a long run of
// 16x16x32 bf16 MFMAs on register operands over a few independent
// accumulators, so that the matrix pipe never waits on a result. Nothing is
// read from memory; one float per thread is written at the end so that the
// work stays live.
#include "device_common.h"
#include "measure.h"

namespace comba {

__global__ __launch_bounds__(kPeakProbeThreads) void mfma_peak_kernel(float* __restrict__ sink, int iters) {
  const int lane = threadIdx.x & (kWave - 1);
  bf16x8 a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    // small exact values that depend on the lane, so that nothing folds
    a[j] = static_cast<__bf16>(static_cast<float>((lane + j) & 7) * 0.125f);
    b[j] = static_cast<__bf16>(static_cast<float>((lane * 3 + j) & 7) * 0.0625f);
  }
  f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0, c2 = c0, c3 = c0;
  static_assert(kPeakProbeChains == 4, "four named accumulators");
  int i = 0;
  do {  // iters >= 1 (checked on the host)
    c0 = mfma16x16x32(a, b, c0);
    c1 = mfma16x16x32(a, b, c1);
    c2 = mfma16x16x32(a, b, c2);
    c3 = mfma16x16x32(a, b, c3);
  } while (++i < iters);
  const f32x4 t = c0 + c1 + c2 + c3;
  const float s = t[0] + t[1] + t[2] + t[3];
  sink[static_cast<size_t>(blockIdx.x) * kPeakProbeThreads + threadIdx.x] = s;
}

hipError_t launch_mfma_peak_probe(float* sink, int blocks, int iters, hipStream_t st) {
  mfma_peak_kernel<<<blocks, kPeakProbeThreads, 0, st>>>(sink, iters);
  return hipGetLastError();
}

}  // namespace comba
