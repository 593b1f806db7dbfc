// Launchers of the measurement kernels (not part of the recurrence).
#pragma once

#include <hip/hip_runtime.h>

namespace comba {

// Threads per workgroup of the matrix-core ceiling kernel (four wavefronts).
constexpr int kPeakProbeThreads = 256;
// Independent accumulators per wavefront, each taking one MFMA per iteration.
constexpr int kPeakProbeChains = 4;

hipError_t launch_mfma_peak_probe(float* sink, int blocks, int iters, hipStream_t st);

// LDS access-pattern probe: every wavefront repeats one LDS instruction whose
// 64 lane addresses are given, so that the LDS bank-conflict counters of a
// profiler can be read for that pattern alone.
constexpr int kLdsProbeThreads = 256;
constexpr int kLdsProbeBytes = 65536;  // LDS the probe allocates; offsets address it
struct LdsLaneOffsets {
  int v[64];  // byte offset of each lane's access
};
// kind: 0-3 reads of 16, 8, 4 bytes and the 8-byte transposing read
// (ds_read_b64_tr_b16); 4-7 writes of 16, 8, 4 and 2 bytes.
hipError_t launch_lds_probe(int kind, const LdsLaneOffsets& offs, int iters, unsigned* sink, int blocks,
                            hipStream_t st);

}  // namespace comba
