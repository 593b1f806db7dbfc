// Measurement kernels, not part of the recurrence.
//
// Matrix-core ceiling measured on the part itself, to set beside the
// published dense bf16 peak: every wavefront issues a long run of
// 16x16x32 bf16 MFMAs on register operands over a few independent
// accumulators, so that the matrix pipe never waits on a result. Nothing is
// read from memory; one float per thread is written at the end so that the
// work stays live.
#include "bf16_tiles.h"
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

// One LDS access pattern, repeated: lane l of every wavefront accesses byte
// offset offs.v[l] of a 64 KiB LDS array in each of `iters` iterations. The
// offset passes through an empty asm statement every iteration so that the
// access is not hoisted out of the loop. The host has checked each offset
// for alignment to the access width and for the 64 KiB bound.
template <int KIND>
__global__ __launch_bounds__(kLdsProbeThreads) void lds_probe_kernel(LdsLaneOffsets offs, int iters, unsigned* sink) {
  __shared__ unsigned lds[kLdsProbeBytes / 4];
  for (int i = threadIdx.x; i < kLdsProbeBytes / 4; i += kLdsProbeThreads) lds[i] = i * 2654435761u;
  __syncthreads();
  char* const base = reinterpret_cast<char*>(lds);
  const int off0 = offs.v[threadIdx.x & (kWave - 1)];
  unsigned acc = threadIdx.x;
  int i = 0;
  do {  // iters >= 1 (checked on the host)
    int o = off0;
    asm volatile("" : "+v"(o));
    if constexpr (KIND == 0) {
      const u32x4 x = *reinterpret_cast<const u32x4*>(base + o);
      acc += x.x ^ x.y ^ x.z ^ x.w;
    } else if constexpr (KIND == 1) {
      const u32x2 x = *reinterpret_cast<const u32x2*>(base + o);
      acc += x.x ^ x.y;
    } else if constexpr (KIND == 2) {
      acc += *reinterpret_cast<const unsigned*>(base + o);
    } else if constexpr (KIND == 3) {
      const s4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(base + o));
      acc += static_cast<unsigned>(x[0]) ^ static_cast<unsigned>(x[3]);
    } else if constexpr (KIND == 4) {
      *reinterpret_cast<u32x4*>(base + o) = u32x4{acc, acc + 1, acc + 2, acc + 3};
    } else if constexpr (KIND == 5) {
      *reinterpret_cast<u32x2*>(base + o) = u32x2{acc, acc + 1};
    } else if constexpr (KIND == 6) {
      *reinterpret_cast<unsigned*>(base + o) = acc;
    } else {
      *reinterpret_cast<unsigned short*>(base + o) = static_cast<unsigned short>(acc);
    }
    acc = acc * 3u + 1u;
  } while (++i < iters);
  __syncthreads();
  sink[static_cast<size_t>(blockIdx.x) * kLdsProbeThreads + threadIdx.x] = acc + lds[threadIdx.x];
}

hipError_t launch_lds_probe(int kind, const LdsLaneOffsets& offs, int iters, unsigned* sink, int blocks,
                            hipStream_t st) {
  switch (kind) {
    case 0: lds_probe_kernel<0><<<blocks, kLdsProbeThreads, 0, st>>>(offs, iters, sink); break;
    case 1: lds_probe_kernel<1><<<blocks, kLdsProbeThreads, 0, st>>>(offs, iters, sink); break;
    case 2: lds_probe_kernel<2><<<blocks, kLdsProbeThreads, 0, st>>>(offs, iters, sink); break;
    case 3: lds_probe_kernel<3><<<blocks, kLdsProbeThreads, 0, st>>>(offs, iters, sink); break;
    case 4: lds_probe_kernel<4><<<blocks, kLdsProbeThreads, 0, st>>>(offs, iters, sink); break;
    case 5: lds_probe_kernel<5><<<blocks, kLdsProbeThreads, 0, st>>>(offs, iters, sink); break;
    case 6: lds_probe_kernel<6><<<blocks, kLdsProbeThreads, 0, st>>>(offs, iters, sink); break;
    case 7: lds_probe_kernel<7><<<blocks, kLdsProbeThreads, 0, st>>>(offs, iters, sink); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace comba
