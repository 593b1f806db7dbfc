// Launchers of the measurement kernels (not part of the recurrence).
#pragma once

#include <hip/hip_runtime.h>

namespace comba {

// Threads per workgroup of the matrix-core ceiling kernel (four wavefronts).
constexpr int kPeakProbeThreads = 256;
// Independent accumulators per wavefront, each taking one MFMA per iteration.
constexpr int kPeakProbeChains = 4;

hipError_t launch_mfma_peak_probe(float* sink, int blocks, int iters, hipStream_t st);

}  // namespace comba
