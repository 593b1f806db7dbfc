// Longest-first order of packed sequences, from cu_seqlens alone (integer,
// exact). Sequence i goes to position rank(i) = #{j : len_j > len_i, or
// len_j == len_i and j < i}: a strict total order, so the result is a
// permutation even for malformed cu_seqlens. Used so that the chunk kernel
// starts the longest sequences first.
#include "launch.h"

namespace comba {

constexpr int kOrderBlock = 256;

__global__ __launch_bounds__(kOrderBlock) void varlen_order_kernel(const int32_t* __restrict__ cu,
                                                                   int N, int32_t* __restrict__ order) {
  __shared__ int32_t len_tile[kOrderBlock];
  const int i = blockIdx.x * kOrderBlock + threadIdx.x;
  const int li = i < N ? cu[i + 1] - cu[i] : 0;
  int rank = 0;
  for (int base = 0; base < N; base += kOrderBlock) {
    const int j = base + threadIdx.x;
    __syncthreads();
    len_tile[threadIdx.x] = j < N ? cu[j + 1] - cu[j] : 0;
    __syncthreads();
    const int m = min(kOrderBlock, N - base);
    for (int jj = 0; jj < m; ++jj) {
      const int lj = len_tile[jj];
      rank += (lj > li) || (lj == li && base + jj < i);
    }
  }
  if (i < N) order[rank] = i;
}

hipError_t launch_varlen_order(const int32_t* cu_seqlens, int N, int32_t* order, hipStream_t st) {
  varlen_order_kernel<<<(N + kOrderBlock - 1) / kOrderBlock, kOrderBlock, 0, st>>>(cu_seqlens, N, order);
  return hipGetLastError();
}

}  // namespace comba
