// Pieces of the chunk-wise Comba forward shared by the bf16 (matrix-core) and
// fp32 kernels: decay bookkeeping and the unit-lower-triangular inverse.
//
// Chunk algebra (one chunk of n <= 64 tokens, incoming state h = S^T, K x V;
// g = log alpha, G / Gx inclusive / exclusive in-chunk cumulative sums):
//   A[t,s] = beta_t exp(Gx_t - G_s) (k_t . k_s)   for s < t    (strictly lower)
//   Tinv   = (I + A)^-1                                         (one inverse)
//   R      = diag(beta) V - diag(beta exp(Gx)) K h
//   Ubar   = Tinv R               (row t: beta_t (v_t - S_{t-1} k_t))
//   O      = diag(exp G) (Q h - d K h) + P Ubar,
//            P[t,s] = (q_t . k_s - d k_t . k_s) exp(G_t - G_s) for s <= t
//   h'     = exp(G_n) h + K^T diag(exp(G_n - G)) Ubar
// This is the write-up's "recurrent across chunks, parallel inside" scheme
// (section "硬件高效的分块并行计算") with its intermediates W = Tinv diag(beta
// exp(Gx)) K and U = Tinv diag(beta) V folded as Ubar = U - W h = Tinv R.
// Comba's decay does not scale the erase term, so A and the write use the
// exclusive sum Gx. Rows past the end of a sequence are padded with k = q = v
// = 0, alpha = 1, beta = 0, which leaves h and every real row unchanged.
#pragma once

#include "device_common.h"

namespace comba {

constexpr int kLdF = 68;  // fp32 row stride of the 64x64 A / Tinv matrices in LDS

struct ChunkGates {
  float G[64];      // inclusive cumulative log-decay
  float Gx[64];     // exclusive cumulative log-decay
  float beta[64];   // beta (0 on padded rows)
  float bEGx[64];   // beta exp(Gx)
  float EG[64];     // exp(G)
  float EGnG[64];   // exp(G_n - G)
  float raw_a[64];  // staged alpha of the chunk
  float raw_b[64];  // staged beta of the chunk
  // G and Gx again, summed in double. A decay factor is the exponential of a
  // difference of two cumulative sums; taken in float, that difference loses
  // ulp(|G|) to cancellation once earlier tokens of the chunk have decayed
  // strongly (|G| in the thousands when alpha is near zero), which the
  // double sums avoid.
  double Gd[64];
  double Gxd[64];
};

// Run by one wavefront: lane = row of the chunk.
__device__ __forceinline__ void chunk_gates(ChunkGates& gt, int lane, int nrows) {
  const bool valid = lane < nrows;
  const float a = valid ? gt.raw_a[lane] : 1.f;
  const float be = valid ? gt.raw_b[lane] : 0.f;
  // alpha below the smallest normal float is taken as that float, so that
  // log alpha stays finite (the state is then forgotten within the token).
  const float g = logf(fmaxf(a, 1.17549435e-38f));
  const double G = wave_inclusive_scan_f64(static_cast<double>(g), lane);
  const double Gn = __shfl(G, 63, kWave);
  const double Gx = G - static_cast<double>(g);
  gt.Gd[lane] = G;
  gt.Gxd[lane] = Gx;
  gt.G[lane] = static_cast<float>(G);
  gt.Gx[lane] = static_cast<float>(Gx);
  gt.beta[lane] = be;
  gt.bEGx[lane] = be * expf(static_cast<float>(Gx));
  gt.EG[lane] = expf(static_cast<float>(G));
  gt.EGnG[lane] = expf(static_cast<float>(Gn - G));
}

// exp(G_t - G_s) and exp(Gx_t - G_s) with the difference taken in double.
__device__ __forceinline__ float decay_G(const ChunkGates& gt, int t, int s) {
  return expf(static_cast<float>(gt.Gd[t] - gt.Gd[s]));
}
__device__ __forceinline__ float decay_Gx(const ChunkGates& gt, int t, int s) {
  return expf(static_cast<float>(gt.Gxd[t] - gt.Gd[s]));
}

// One level of the off-diagonal blocks of the 64x64 inverse below: every
// block at distance L = i - j below the diagonal,
//   T_ij = -T_ii sum_{j <= m < i} A_im T_mj,
// from the diagonal blocks and the levels closer to it. The reduction lengths
// are compile-time constants, so the LDS reads issue back to back (A rows as
// 16-byte reads); the sums run over m in increasing order. The upper part of
// a diagonal block T_ii is exactly zero, so its product runs over all 16
// columns.
template <int L, int NT>
__device__ __forceinline__ void inverse_level(const float* Am, float* Tm, float* Ys, int tid) {
  constexpr int nb = 4 - L;
  for (int e = tid; e < nb * 256; e += NT) {
    const int j = e >> 8, r = (e >> 4) & 15, c = e & 15, i = j + L;
    const float* arow = Am + (16 * i + r) * kLdF + 16 * j;
    const float* tcol = Tm + (16 * j) * kLdF + 16 * j + c;
    float acc = 0.f;
#pragma unroll
    for (int m4 = 0; m4 < 4 * L; ++m4) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(arow + 4 * m4);
#pragma unroll
      for (int u = 0; u < 4; ++u) acc += a[u] * tcol[(4 * m4 + u) * kLdF];
    }
    Ys[e] = acc;
  }
  __syncthreads();
  for (int e = tid; e < nb * 256; e += NT) {
    const int j = e >> 8, r = (e >> 4) & 15, c = e & 15, i = j + L;
    const float* trow = Tm + (16 * i + r) * kLdF + 16 * i;
    const float* ycol = Ys + (j << 8) + c;
    float acc = 0.f;
#pragma unroll
    for (int m4 = 0; m4 < 4; ++m4) {
      const f32x4 t = *reinterpret_cast<const f32x4*>(trow + 4 * m4);
#pragma unroll
      for (int u = 0; u < 4; ++u) acc += t[u] * ycol[(4 * m4 + u) << 4];
    }
    Tm[(16 * i + r) * kLdF + 16 * j + c] = -acc;
  }
  __syncthreads();
}

// Tm = (I + Am)^-1 for a 64x64 strictly lower Am (fp32, row stride kLdF).
// Only the lower 16x16 blocks of Am are read; the lower blocks of Tm are
// written (zeros above the diagonal inside diagonal blocks). Ys: 768 floats.
// Diagonal blocks: column-wise forward substitution, one lane per column;
// then the off-diagonal blocks level by level (inverse_level).
// Must be called by all NT threads; ends with a barrier.
template <int NT>
__device__ __forceinline__ void unit_lower_inverse64(const float* Am, float* Tm, float* Ys, int tid) {
  if (tid < 64) {
    const int blk = tid >> 4, c = tid & 15;
    const float* Ab = Am + (16 * blk) * kLdF + 16 * blk;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r] = (r == c) ? 1.f : 0.f;
#pragma unroll
    for (int j = 0; j < 15; ++j) {
#pragma unroll
      for (int r = j + 1; r < 16; ++r) x[r] -= Ab[r * kLdF + j] * x[j];
    }
    float* Tb = Tm + (16 * blk) * kLdF + 16 * blk;
#pragma unroll
    for (int r = 0; r < 16; ++r) Tb[r * kLdF + c] = x[r];
  }
  __syncthreads();
  inverse_level<1, NT>(Am, Tm, Ys, tid);
  inverse_level<2, NT>(Am, Tm, Ys, tid);
  inverse_level<3, NT>(Am, Tm, Ys, tid);
}

// Work unit of a block: units are (sequence rank, head) pairs dealt
// round-robin over the 8 XCDs; the nvt tiles of one unit are consecutive
// blocks on one XCD. Returns false for padding blocks.
__device__ __forceinline__ bool unit_of_block(int bid, int nvt, int units, int& unit, int& vt) {
  const int xcd = bid & 7, slot = bid >> 3;
  unit = (slot / nvt) * 8 + xcd;
  vt = slot % nvt;
  return unit < units;
}

}  // namespace comba
