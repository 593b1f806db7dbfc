// Device-side preconditions of the chunk and decode entry points, checked on
// demand (a debug aid; no entry point runs it by itself). The gate alpha is the
// per-token decay of Comba's scalar-plus-low-rank transition and enters as
// log alpha, so it must lie in (0, 1]; a packed batch's cu_seqlens must start
// at 0, end at T and never decrease. One launch clears the caller's flag word
// (a plain store, so that the pair can be captured in a graph), a second ORs
// in one bit per violated precondition.
#include "comba.h"
#include "device_common.h"
#include "launch.h"

namespace comba {

constexpr int kCheckBlock = 256;

__global__ __launch_bounds__(64) void check_clear_kernel(uint32_t* __restrict__ flags) {
  if (threadIdx.x == 0) *flags = 0u;
}

__global__ __launch_bounds__(kCheckBlock) void check_inputs_kernel(const float* __restrict__ alpha, int64_t n_alpha,
                                                                   const int32_t* __restrict__ cu, int N, int T,
                                                                   uint32_t* __restrict__ flags) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kCheckBlock;
  const int64_t i0 = static_cast<int64_t>(blockIdx.x) * kCheckBlock + threadIdx.x;
  uint32_t f = 0u;
  for (int64_t i = i0; i < n_alpha; i += stride) {
    const float a = alpha[i];
    if (!(a > 0.f && a <= 1.f)) f |= COMBA_CHECK_ALPHA_RANGE;  // also true for NaN
  }
  if (cu) {
    for (int64_t n = i0; n < N; n += stride)
      if (cu[n + 1] < cu[n]) f |= COMBA_CHECK_CU_ORDER;
    if (i0 == 0 && (cu[0] != 0 || cu[N] != T)) f |= COMBA_CHECK_CU_BOUNDS;
  }
  // one atomic per wavefront that found something
  for (int m = 1; m < kWave; m <<= 1) f |= static_cast<uint32_t>(__shfl_xor(static_cast<int>(f), m, kWave));
  if ((threadIdx.x & (kWave - 1)) == 0 && f) atomicOr(flags, f);
}

hipError_t launch_check_inputs(const float* alpha, int64_t n_alpha, const int32_t* cu_seqlens, int N, int T,
                               uint32_t* flags, hipStream_t st) {
  check_clear_kernel<<<1, 64, 0, st>>>(flags);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t work = n_alpha > (cu_seqlens ? static_cast<int64_t>(N) : 0) ? n_alpha : N;
  const int64_t want = (work + kCheckBlock - 1) / kCheckBlock;
  const unsigned grid = static_cast<unsigned>(want < 1 ? 1 : (want > 2048 ? 2048 : want));
  check_inputs_kernel<<<grid, kCheckBlock, 0, st>>>(alpha, n_alpha, cu_seqlens, N, T, flags);
  return hipGetLastError();
}

}  // namespace comba
