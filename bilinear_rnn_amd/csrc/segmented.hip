// Segment-parallel chunk forward for long sequences: the small kernels
// around the chunk kernel.
//
// A sequence split into segments j = 0 .. S-1 of L tokens is run as S packed
// sequences. The state map of a segment is affine in its initial state X
// (Comba write-up, section "Comba架构：基于闭环控制理论": every step multiplies
// the state by alpha_t I - beta_t k_t k_t^T on the right and adds beta_t v_t k_t^T):
//     S_end = X Phi_j + b_j,   Phi_j = prod_t (alpha_t I - beta_t k_t k_t^T),
// where b_j is the segment's final state from a zero state and Phi_j the final
// state of a run with v = 0 from the identity (a K x K "state"). The chunk
// kernel produces both; the scan below chains them, X_{j+1} = X_j Phi_j + b_j,
// and a last chunk-kernel pass reruns every segment from its true X_j.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace comba {

// cu[n] for segment n = b * S + j: b T + min(j L, T); cu[B S] = B T.
__global__ __launch_bounds__(256) void segment_bounds_kernel(int B, int T, int L, int S, int32_t* __restrict__ cu) {
  const int n = blockIdx.x * blockDim.x + threadIdx.x;
  const int total = B * S;
  if (n > total) return;
  if (n == total) {
    cu[n] = B * T;
    return;
  }
  const int b = n / S, j = n % S;
  cu[n] = b * T + min(j * L, T);
}

// One workgroup per (batch row b, head h, block of RB state rows). X rows
// live in LDS; thread (c, i0) owns column c of RPT rows. For each segment:
// store X_j as that segment's initial state, then X_{j+1} = X_j Phi_j + b_j in
// fp32 (Phi_j column c read from LDS, the X row element broadcast from LDS).
// Phi_j (K x K) and the rows of b_j are loaded one segment ahead: Phi with
// 16-byte loads into registers, then into the other half of a double-buffered
// LDS copy. After the last segment X_S is the sequence's final state.
template <int K>
__global__ __launch_bounds__(256) void segment_scan_kernel(const float* s0, const float* __restrict__ bst,
                                                           const float* __restrict__ phi, float* __restrict__ X,
                                                           float* sf, int H, int V, int S) {
  typedef float f4 __attribute__((ext_vector_type(4)));
  constexpr int RB = 8, RG = 256 / K, RPT = RB / RG, PP = K * K / 4 / 256;
  static_assert(RPT >= 1 && PP * 4 * 256 == K * K, "whole pieces per thread");
  __shared__ f4 phs[2][K * K / 4];
  __shared__ float xs[RB][K];
  const int nrb = V / RB;
  const int rb = blockIdx.x % nrb, bh = blockIdx.x / nrb, h = bh % H, b = bh / H;
  const int tid = threadIdx.x, c = tid % K, i0 = tid / K;
  auto seg = [&](int j) { return static_cast<int64_t>(b) * S + j; };
  auto row_off = [&](int64_t n, int r) { return ((n * H + h) * V + rb * RB + i0 + r * RG) * K + c; };
  f4 pr[PP];
  float bn[RPT];
  auto fetch = [&](int j) {
    const f4* src = reinterpret_cast<const f4*>(phi + (seg(j) * H + h) * K * K);
#pragma unroll
    for (int p = 0; p < PP; ++p) pr[p] = src[tid + p * 256];
#pragma unroll
    for (int r = 0; r < RPT; ++r) bn[r] = bst[row_off(seg(j), r)];
  };
  float x[RPT];
#pragma unroll
  for (int r = 0; r < RPT; ++r) {
    x[r] = s0 ? s0[row_off(b, r)] : 0.f;
    xs[i0 + r * RG][c] = x[r];
  }
  if (S > 0) fetch(0);
#pragma unroll
  for (int p = 0; p < PP; ++p) phs[0][tid + p * 256] = pr[p];
  __syncthreads();
  for (int j = 0; j < S; ++j) {
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      X[row_off(seg(j), r)] = x[r];
      x[r] = bn[r];
    }
    if (j + 1 < S) fetch(j + 1);  // in flight during this segment's product
    const float* ph = reinterpret_cast<const float*>(phs[j & 1]) + c;
#pragma unroll 8
    for (int m = 0; m < K; ++m) {
      const float p = ph[m * K];
#pragma unroll
      for (int r = 0; r < RPT; ++r) x[r] += xs[i0 + r * RG][m] * p;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < RPT; ++r) xs[i0 + r * RG][c] = x[r];
    if (j + 1 < S) {
#pragma unroll
      for (int p = 0; p < PP; ++p) phs[(j + 1) & 1][tid + p * 256] = pr[p];
    }
    __syncthreads();
  }
  if (sf) {
#pragma unroll
    for (int r = 0; r < RPT; ++r) sf[row_off(b, r)] = x[r];
  }
}

hipError_t launch_segment_bounds(int B, int T, int L, int S, int32_t* cu, hipStream_t st) {
  const int n = B * S + 1;
  segment_bounds_kernel<<<(n + 255) / 256, 256, 0, st>>>(B, T, L, S, cu);
  return hipGetLastError();
}

hipError_t launch_segment_scan(const float* s0, const float* bst, const float* phi, float* X, float* sf, int B,
                               int H, int K, int V, int S, hipStream_t st) {
  const int grid = B * H * (V / 8);
  if (K == 128)
    segment_scan_kernel<128><<<grid, 256, 0, st>>>(s0, bst, phi, X, sf, H, V, S);
  else
    segment_scan_kernel<64><<<grid, 256, 0, st>>>(s0, bst, phi, X, sf, H, V, S);
  return hipGetLastError();
}

}  // namespace comba
