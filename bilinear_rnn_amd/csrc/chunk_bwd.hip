// Chunk-wise backward of the Comba mixer: gradients of q, k, v, alpha, beta,
// d and the initial state for given dL/do and dL/dS_final.
//
// Chunk form (one chunk of n <= 64 tokens, h = S^T the K x V incoming state,
// notation of the forward: A, Tinv = (I + A)^-1, R, Ubar, P, M[t,s] =
// e^(G_t - G_s), E[t,s] = e^(Gx_t - G_s), b1 = beta e^Gx, qt = q - d k). The
// forward is the write-up's chunk scheme (section "硬件高效的分块并行计算");
// its reverse mode, with dh the gradient of the chunk's outgoing state:
//   dUbar = P^T dO + diag(e^(Gn - G)) K dh          dR = Tinv^T dUbar
//   dV    = diag(beta) dR
//   dh_in = e^Gn dh + Qt^T diag(e^G) dO - K^T diag(b1) dR
//   dA    = -(dR Ubar^T) (s < t),   dP = dO Ubar^T (s <= t),   W = dA (.) E
//   dQt   = diag(e^G) dO h^T + (dP (.) M) K
//   dK    = (dP (.) M)^T Qt + diag(beta) W K + W^T diag(beta) K
//           - diag(b1) dR h^T + diag(e^(Gn - G)) Ubar dh^T - d dQt
//   dq = dQt,  dd = -sum(dQt (.) K)
//   dbeta_t = sum_s W_ts k_t.k_s + dR_t . (v_t - e^Gx_t (K h)_t)
// and for the decays, with G the in-chunk cumulative log alpha:
//   dG_t  = e^G_t (Qt h)_t . dO_t + rowsum(dP (.) P)_t - colsum(dP (.) P)_t
//           - colsum(dA (.) A)_t - e^(Gn - G_t) (K dh)_t . Ubar_t
//   dGx_t = rowsum(dA (.) A)_t - b1_t (K h)_t . dR_t
//   dGn   = e^Gn <h, dh> + sum_t e^(Gn - G_t) (K dh)_t . Ubar_t   (added to dG at the last row)
//   dlog(alpha_t) = -dGx_t + sum_{s >= t} (dG_s + dGx_s),   dalpha_t = dlog(alpha_t) / alpha_t.
// An fp64 prototype of exactly these formulas matches the reverse-mode oracle
// of the token recurrence to 1e-15.
//
// Three launches after a forward pass that stores every chunk's incoming
// state (the chunk kernels' checkpoint option):
//   chunk_bwd_dh_kernel    reverse scan over chunks, one workgroup per
//                          (sequence, head, 32 value channels): stores each
//                          chunk's outgoing-state gradient dh, writes dS_0;
//   chunk_bwd_grad_kernel  one workgroup per (chunk, head), all chunks at once:
//                          every per-token gradient and a partial of dd;
//   dd_reduce_kernel       dd per head, summed over chunks in a fixed order.
// All arithmetic is fp32 on the vector units.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "chunk_common.h"
#include "launch.h"

namespace comba {

namespace {

constexpr int kDhVT = 32;  // value channels per workgroup of the reverse scan
constexpr int kGrVT = 8;   // value channels per tile of the gradient kernel

template <typename InT>
__device__ __forceinline__ float ld(const InT* p, int64_t i) {
  return Elem<InT>::load(p, i);
}

// q~ = q - d k and k of the chunk's rows (zeros past the end), fp32, row stride K + 1.
template <int K, typename InT>
__device__ __forceinline__ void stage_qk(const InT* q, const InT* k, float (*Qt)[K + 1], float (*Kc)[K + 1],
                                         int64_t tok0, int H, int nrows, float dh, int tid, int nt) {
  for (int e = tid; e < 64 * K; e += nt) {
    const int row = e / K, c = e % K;
    float kv = 0.f, qv = 0.f;
    if (row < nrows) {
      const int64_t off = (tok0 + static_cast<int64_t>(row) * H) * K + c;
      kv = ld(k, off);
      qv = ld(q, off);
    }
    Kc[row][c] = kv;
    Qt[row][c] = qv - dh * kv;
  }
}

// A (strictly lower, full 64 x 64 with zeros elsewhere) from staged k rows.
template <int K>
__device__ __forceinline__ void form_A(const float (*Kc)[K + 1], const ChunkGates& gt, float* Am, int tid, int nt) {
  for (int e = tid; e < 64 * 64; e += nt) {
    const int t = e >> 6, s = e & 63;
    float a = 0.f;
    if (s < t) {
      float kk = 0.f;
      #pragma unroll 8
      for (int c = 0; c < K; ++c) kk += Kc[t][c] * Kc[s][c];
      a = gt.beta[t] * expf(gt.Gx[t] - gt.G[s]) * kk;
    }
    Am[t * kLdF + s] = a;
  }
}

// P (lower with diagonal, full 64 x 64 with zeros elsewhere).
template <int K>
__device__ __forceinline__ void form_P(const float (*Qt)[K + 1], const float (*Kc)[K + 1], const ChunkGates& gt,
                                       float* Pm, int tid, int nt) {
  for (int e = tid; e < 64 * 64; e += nt) {
    const int t = e >> 6, s = e & 63;
    float p = 0.f;
    if (s <= t) {
      float qk = 0.f;
      #pragma unroll 8
      for (int c = 0; c < K; ++c) qk += Qt[t][c] * Kc[s][c];
      p = qk * expf(fminf(gt.G[t] - gt.G[s], 0.f));
    }
    Pm[t * kLdF + s] = p;
  }
}

template <int K>
struct SmemDh {
  float Kc[64][K + 1];
  float Qt[64][K + 1];
  float Tm[64 * kLdF];
  float Pm[64 * kLdF];  // A, then P
  float Ys[768];
  float dh[K][kDhVT + 1];
  float dO[64][kDhVT + 1];
  float dU[64][kDhVT + 1];  // dUbar, then dR
  ChunkGates gt;
};

// Reverse scan over the chunks of one (sequence, head, value tile).
template <int K, int V, typename InT>
__global__ __launch_bounds__(256) void chunk_bwd_dh_kernel(
    const InT* __restrict__ q, const InT* __restrict__ k, const float* __restrict__ alpha,
    const float* __restrict__ beta, const float* __restrict__ d, const InT* __restrict__ dO,
    const int32_t* __restrict__ cu_seqlens, int T, int H, int N, const float* __restrict__ dsf,
    float* __restrict__ dhck, float* __restrict__ ds0) {
  constexpr int NT = 256, VT = kDhVT, NVT = V / VT;
  __shared__ SmemDh<K> sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int unit, vt;
  if (!unit_of_block(blockIdx.x, NVT, N * H, unit, vt)) return;
  const int h = unit % H, n = unit / H;
  int b, t0, t1;
  sequence_range(cu_seqlens, n, T, b, t0, t1);
  const float dh_ = d[h];
  const int nch = (t1 - t0 + 63) / 64;
  const bool packed = cu_seqlens != nullptr;
  const int64_t srow = (static_cast<int64_t>(n) * H + h) * V + vt * VT;  // state row of channel 0 of the tile

  for (int e = tid; e < K * VT; e += NT) {
    const int kk = e % K, c = e / K;
    sm.dh[kk][c] = dsf ? dsf[(srow + c) * K + kk] : 0.f;
  }
  for (int ci = nch - 1; ci >= 0; --ci) {
    const int c0 = t0 + 64 * ci, nrows = min(64, t1 - c0);
    const int64_t tok0 = (static_cast<int64_t>(b) * T + c0) * H + h;
    __syncthreads();
    stage_qk<K>(q, k, sm.Qt, sm.Kc, tok0, H, nrows, dh_, tid, NT);
    for (int e = tid; e < 64 * VT; e += NT) {
      const int row = e / VT, c = e % VT;
      sm.dO[row][c] = row < nrows ? ld(dO, (tok0 + static_cast<int64_t>(row) * H) * V + vt * VT + c) : 0.f;
    }
    if (tid < 64) {
      sm.gt.raw_a[tid] = tid < nrows ? alpha[tok0 + static_cast<int64_t>(tid) * H] : 1.f;
      sm.gt.raw_b[tid] = tid < nrows ? beta[tok0 + static_cast<int64_t>(tid) * H] : 0.f;
    }
    // the gradient of this chunk's outgoing state, for the gradient kernel
    {
      float* dst = dhck + (chunk_slot(packed, t0, n, ci, T) * H + h) * V * K + static_cast<int64_t>(vt) * VT * K;
      for (int e = tid; e < K * VT; e += NT) {
        const int kk = e % K, c = e / K;
        dst[static_cast<int64_t>(c) * K + kk] = sm.dh[kk][c];
      }
    }
    __syncthreads();
    if (wave == 0) chunk_gates(sm.gt, lane, nrows);
    __syncthreads();
    form_A<K>(sm.Kc, sm.gt, sm.Pm, tid, NT);
    __syncthreads();
    unit_lower_inverse64<NT>(sm.Pm, sm.Tm, sm.Ys, tid);
    form_P<K>(sm.Qt, sm.Kc, sm.gt, sm.Pm, tid, NT);
    __syncthreads();
    // dUbar = P^T dO + diag(e^(Gn - G)) K dh
    for (int e = tid; e < 64 * VT; e += NT) {
      const int t = e / VT, c = e % VT;
      float acc = 0.f;
      for (int t2 = t; t2 < 64; ++t2) acc += sm.Pm[t2 * kLdF + t] * sm.dO[t2][c];
      float kd = 0.f;
      #pragma unroll 8
      for (int kk = 0; kk < K; ++kk) kd += sm.Kc[t][kk] * sm.dh[kk][c];
      sm.dU[t][c] = acc + sm.gt.EGnG[t] * kd;
    }
    __syncthreads();
    // dR = Tinv^T dUbar
    float r[64 * VT / NT];
#pragma unroll
    for (int j = 0; j < 64 * VT / NT; ++j) {
      const int e = tid + j * NT, s = e / VT, c = e % VT;
      float acc = 0.f;
      for (int t = s; t < 64; ++t) acc += sm.Tm[t * kLdF + s] * sm.dU[t][c];
      r[j] = acc;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 64 * VT / NT; ++j) {
      const int e = tid + j * NT;
      sm.dU[e / VT][e % VT] = r[j];
    }
    __syncthreads();
    // dh_in = e^Gn dh + Qt^T diag(e^G) dO - K^T diag(b1) dR
    const float eGn = sm.gt.EG[63];
    float nd[K * VT / NT];
#pragma unroll
    for (int j = 0; j < K * VT / NT; ++j) {
      const int e = tid + j * NT, kk = e % K, c = e / K;
      float acc = eGn * sm.dh[kk][c];
      for (int t = 0; t < 64; ++t)
        acc += sm.Qt[t][kk] * (sm.gt.EG[t] * sm.dO[t][c]) - sm.Kc[t][kk] * (sm.gt.bEGx[t] * sm.dU[t][c]);
      nd[j] = acc;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < K * VT / NT; ++j) {
      const int e = tid + j * NT;
      sm.dh[e % K][e / K] = nd[j];
    }
  }
  __syncthreads();
  if (ds0) {
    for (int e = tid; e < K * VT; e += NT) {
      const int kk = e % K, c = e / K;
      ds0[(srow + c) * K + kk] = sm.dh[kk][c];
    }
  }
}

template <int K>
struct SmemGrad {
  float Kc[64][K + 1];
  float Qt[64][K + 1];
  float Tm[64 * kLdF];  // Tinv, then k_t.k_s, then X = W (.) KK
  float Pm[64 * kLdF];  // P, then dP (.) P
  float dA[64 * kLdF];  // A, then dA, then W = dA (.) E
  float dP[64 * kLdF];  // dP, then dP (.) M
  union {
    float Ys[768];  // inverse scratch (before the value tiles)
    struct {
      float hc[K][kGrVT + 1];
      float dh[K][kGrVT + 1];
    } st;
  } u;
  float dO[64][kGrVT + 1];
  float U[64][kGrVT + 1];   // R, then Ubar
  float dR[64][kGrVT + 1];  // dUbar, then dR
  ChunkGates gt;
  float vec[8][64];  // per-token sums over the value channels / rows / columns
  float red[16];
};

// Gradients of one (chunk, head).
template <int K, int V, typename InT>
__global__ __launch_bounds__(512) void chunk_bwd_grad_kernel(
    const InT* __restrict__ q, const InT* __restrict__ k, const InT* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta, const float* __restrict__ d,
    const InT* __restrict__ dO, const int32_t* __restrict__ cu_seqlens, int T, int H, int N, int64_t nslots,
    const float* __restrict__ hck, const float* __restrict__ dhck, float* __restrict__ dq, float* __restrict__ dk,
    float* __restrict__ dv, float* __restrict__ dalpha, float* __restrict__ dbeta, float* __restrict__ dd_part) {
  constexpr int NT = 512, VT = kGrVT, NTILE = V / VT, CK = 64 * K / NT;
  __shared__ SmemGrad<K> sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.x % H;
  const int64_t slot = blockIdx.x / H;
  if (slot >= nslots) return;
  // chunk of this slot
  const bool packed = cu_seqlens != nullptr;
  int n, c, b, t0, t1;
  if (packed) {
    int lo = 0, hi = N - 1;  // largest n with t0(n) / 64 + n <= slot
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      int bb, a0, a1;
      sequence_range(cu_seqlens, mid, T, bb, a0, a1);
      if (static_cast<int64_t>(a0 / 64) + mid <= slot) lo = mid; else hi = mid - 1;
    }
    n = lo;
    sequence_range(cu_seqlens, n, T, b, t0, t1);
    c = static_cast<int>(slot - (t0 / 64 + n));
  } else {
    const int nch = (T + 63) / 64;
    n = static_cast<int>(slot / nch);
    c = static_cast<int>(slot % nch);
    sequence_range(cu_seqlens, n, T, b, t0, t1);
  }
  const int c0 = t0 + 64 * c;
  const bool valid = c >= 0 && c0 < t1;
  if (!valid) {  // a slot between packed sequences: no chunk
    if (tid == 0) dd_part[slot * H + h] = 0.f;
    return;
  }
  const int nrows = min(64, t1 - c0);
  const int64_t tok0 = (static_cast<int64_t>(b) * T + c0) * H + h;
  const float dh_ = d[h];
  const float* hsrc = hck + (slot * H + h) * V * K;
  const float* dhsrc = dhck + (slot * H + h) * V * K;

  stage_qk<K>(q, k, sm.Qt, sm.Kc, tok0, H, nrows, dh_, tid, NT);
  if (tid < 64) {
    sm.gt.raw_a[tid] = tid < nrows ? alpha[tok0 + static_cast<int64_t>(tid) * H] : 1.f;
    sm.gt.raw_b[tid] = tid < nrows ? beta[tok0 + static_cast<int64_t>(tid) * H] : 0.f;
  }
  __syncthreads();
  if (wave == 0) chunk_gates(sm.gt, lane, nrows);
  __syncthreads();
  form_A<K>(sm.Kc, sm.gt, sm.dA, tid, NT);
  __syncthreads();
  unit_lower_inverse64<NT>(sm.dA, sm.Tm, sm.u.Ys, tid);
  form_P<K>(sm.Qt, sm.Kc, sm.gt, sm.Pm, tid, NT);
  __syncthreads();

  // this thread's (row, channel) in a value tile, its 8 entries of the 64 x 64
  // accumulators and its CK entries of the 64 x K ones
  const int tr = tid >> 3, tv = tid & 7;
  const float be_t = sm.gt.beta[tr], b1_t = sm.gt.bEGx[tr], eGnG_t = sm.gt.EGnG[tr], eGx_t = expf(sm.gt.Gx[tr]);
  float accA[8], accP[8], accQ[CK], accK[CK];
#pragma unroll
  for (int i = 0; i < 8; ++i) accA[i] = accP[i] = 0.f;
#pragma unroll
  for (int i = 0; i < CK; ++i) accQ[i] = accK[i] = 0.f;
  float sQh = 0.f, sbR = 0.f, sKhdR = 0.f, st2 = 0.f, shdh = 0.f;

  for (int jt = 0; jt < NTILE; ++jt) {
    const int v0 = jt * VT;
    __syncthreads();
    for (int e = tid; e < K * VT; e += NT) {
      const int kk = e % K, cc = e / K;
      const float hv = hsrc[static_cast<int64_t>(v0 + cc) * K + kk];
      const float dv_ = dhsrc[static_cast<int64_t>(v0 + cc) * K + kk];
      sm.u.st.hc[kk][cc] = hv;
      sm.u.st.dh[kk][cc] = dv_;
      shdh += hv * dv_;
    }
    {
      const float x = tr < nrows ? ld(dO, (tok0 + static_cast<int64_t>(tr) * H) * V + v0 + tv) : 0.f;
      sm.dO[tr][tv] = x;
    }
    __syncthreads();
    float kh = 0.f, qh = 0.f, kdh = 0.f;
    #pragma unroll 8
    for (int kk = 0; kk < K; ++kk) {
      const float kv = sm.Kc[tr][kk];
      kh += kv * sm.u.st.hc[kk][tv];
      qh += sm.Qt[tr][kk] * sm.u.st.hc[kk][tv];
      kdh += kv * sm.u.st.dh[kk][tv];
    }
    const float vv = tr < nrows ? ld(v, (tok0 + static_cast<int64_t>(tr) * H) * V + v0 + tv) : 0.f;
    sm.U[tr][tv] = be_t * vv - b1_t * kh;  // R
    __syncthreads();
    float ub = 0.f;  // Ubar = Tinv R
    for (int s = 0; s <= tr; ++s) ub += sm.Tm[tr * kLdF + s] * sm.U[s][tv];
    float du = eGnG_t * kdh;  // dUbar = P^T dO + diag(e^(Gn - G)) K dh
    for (int t2 = tr; t2 < 64; ++t2) du += sm.Pm[t2 * kLdF + tr] * sm.dO[t2][tv];
    __syncthreads();
    sm.U[tr][tv] = ub;
    sm.dR[tr][tv] = du;
    __syncthreads();
    float dr = 0.f;  // dR = Tinv^T dUbar
    for (int t2 = tr; t2 < 64; ++t2) dr += sm.Tm[t2 * kLdF + tr] * sm.dR[t2][tv];
    __syncthreads();
    sm.dR[tr][tv] = dr;
    if (tr < nrows) dv[(tok0 + static_cast<int64_t>(tr) * H) * V + v0 + tv] = be_t * dr;
    // this (row, channel)'s terms of the sums over the value channels
    sQh += qh * sm.dO[tr][tv];
    sbR += dr * (vv - eGx_t * kh);
    sKhdR += kh * dr;
    st2 += kdh * ub;
    __syncthreads();
    // dA -= dR Ubar^T (s < t), dP += dO Ubar^T (s <= t)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int e2 = tid + i * NT, t = e2 >> 6, s = e2 & 63;
      float xa = 0.f, xp = 0.f;
#pragma unroll
      for (int cc = 0; cc < VT; ++cc) {
        const float us = sm.U[s][cc];
        xa += sm.dR[t][cc] * us;
        xp += sm.dO[t][cc] * us;
      }
      if (s < t) accA[i] -= xa;
      if (s <= t) accP[i] += xp;
    }
    // dQt += dO h^T;  dK += -diag(b1) dR h^T + diag(e^(Gn - G)) Ubar dh^T
#pragma unroll
    for (int i = 0; i < CK; ++i) {
      const int e3 = tid + i * NT, t = e3 / K, kk = e3 % K;
      const float b1 = sm.gt.bEGx[t], eg = sm.gt.EGnG[t];
      float xq = 0.f, xk = 0.f;
#pragma unroll
      for (int cc = 0; cc < VT; ++cc) {
        const float hv = sm.u.st.hc[kk][cc];
        xq += sm.dO[t][cc] * hv;
        xk += eg * sm.U[t][cc] * sm.u.st.dh[kk][cc] - b1 * sm.dR[t][cc] * hv;
      }
      accQ[i] += xq;
      accK[i] += xk;
    }
  }
  __syncthreads();

  // per-token sums over the 8 channel lanes of a row; <h, dh> over the block
#pragma unroll
  for (int m = 1; m < 8; m <<= 1) {
    sQh += __shfl_xor(sQh, m, kWave);
    sbR += __shfl_xor(sbR, m, kWave);
    sKhdR += __shfl_xor(sKhdR, m, kWave);
    st2 += __shfl_xor(st2, m, kWave);
  }
  if (tv == 0) {
    sm.vec[0][tr] = sQh;
    sm.vec[1][tr] = sbR;
    sm.vec[2][tr] = sKhdR;
    sm.vec[3][tr] = st2;
  }
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) shdh += __shfl_xor(shdh, m, kWave);
  if (lane == 0) sm.red[wave] = shdh;
  // k_t . k_s (Tinv is no longer needed), dA, dP
  for (int e = tid; e < 64 * 64; e += NT) {
    const int t = e >> 6, s = e & 63;
    float kk = 0.f;
    #pragma unroll 8
    for (int cc = 0; cc < K; ++cc) kk += sm.Kc[t][cc] * sm.Kc[s][cc];
    sm.Tm[t * kLdF + s] = kk;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int e2 = tid + i * NT, t = e2 >> 6, s = e2 & 63;
    sm.dA[t * kLdF + s] = accA[i];
    sm.dP[t * kLdF + s] = accP[i];
  }
  __syncthreads();
  // dP (.) P, dP (.) M, W = dA (.) E, X = W (.) KK
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int e2 = tid + i * NT, t = e2 >> 6, s = e2 & 63, o = t * kLdF + s;
    const float M = s <= t ? expf(fminf(sm.gt.G[t] - sm.gt.G[s], 0.f)) : 0.f;
    const float E = s < t ? expf(fminf(sm.gt.Gx[t] - sm.gt.G[s], 0.f)) : 0.f;
    const float dpv = sm.dP[o], w = sm.dA[o] * E;
    sm.Pm[o] = dpv * sm.Pm[o];
    sm.dP[o] = dpv * M;
    sm.dA[o] = w;
    sm.Tm[o] = w * sm.Tm[o];
  }
  __syncthreads();
  // row and column sums (fixed order)
  if (tid < 64) {
    float rp = 0.f, rx = 0.f;
    for (int s = 0; s < 64; ++s) {
      rp += sm.Pm[tid * kLdF + s];
      rx += sm.Tm[tid * kLdF + s];
    }
    sm.vec[4][tid] = rp;
    sm.vec[5][tid] = rx;
  } else if (tid < 128) {
    const int s = tid - 64;
    float cp = 0.f, cx = 0.f;
    for (int t = 0; t < 64; ++t) {
      cp += sm.Pm[t * kLdF + s];
      cx += sm.gt.beta[t] * sm.Tm[t * kLdF + s];
    }
    sm.vec[6][s] = cp;
    sm.vec[7][s] = cx;
  }
  // dq, dk and this thread's part of dd
  float ddp = 0.f;
#pragma unroll
  for (int i = 0; i < CK; ++i) {
    const int e3 = tid + i * NT, t = e3 / K, kk = e3 % K;
    float xq = sm.gt.EG[t] * accQ[i];
    for (int s = 0; s <= t; ++s) xq += sm.dP[t * kLdF + s] * sm.Kc[s][kk];
    float xk = accK[i] - dh_ * xq;
    const float be = sm.gt.beta[t];
    for (int t2 = t; t2 < 64; ++t2) xk += sm.dP[t2 * kLdF + t] * sm.Qt[t2][kk];
    for (int s = 0; s < t; ++s) xk += be * sm.dA[t * kLdF + s] * sm.Kc[s][kk];
    for (int t2 = t + 1; t2 < 64; ++t2) xk += sm.dA[t2 * kLdF + t] * sm.gt.beta[t2] * sm.Kc[t2][kk];
    ddp -= xq * sm.Kc[t][kk];
    if (t < nrows) {
      const int64_t off = (tok0 + static_cast<int64_t>(t) * H) * K + kk;
      dq[off] = xq;
      dk[off] = xk;
    }
  }
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) ddp += __shfl_xor(ddp, m, kWave);
  __syncthreads();
  if (lane == 0) sm.red[8 + wave] = ddp;
  __syncthreads();
  if (wave == 0) {
    // per-token scalars, lane = row
    const int t = lane;
    float hd = 0.f;
    for (int w = 0; w < NT / 64; ++w) hd += sm.red[w];
    const float be = sm.gt.beta[t], b1 = sm.gt.bEGx[t];
    const float t2 = sm.gt.EGnG[t] * sm.vec[3][t];
    float dG = sm.gt.EG[t] * sm.vec[0][t] + sm.vec[4][t] - sm.vec[6][t] - sm.vec[7][t] - t2;
    const float dGx = be * sm.vec[5][t] - b1 * sm.vec[2][t];
    float sum_t2 = t2;
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) sum_t2 += __shfl_xor(sum_t2, m, kWave);
    if (t == 63) dG += sm.gt.EG[63] * hd + sum_t2;  // dGn
    // reverse inclusive sum of dG + dGx over the chunk
    const float x = dG + dGx;
    const float xr = __shfl(x, 63 - t, kWave);
    const float sr = wave_inclusive_scan(xr, t);
    const float rev = __shfl(sr, 63 - t, kWave);
    const float dlog = rev - dGx;
    if (t < nrows) {
      const int64_t off = tok0 + static_cast<int64_t>(t) * H;
      dbeta[off] = sm.vec[5][t] + sm.vec[1][t];
      dalpha[off] = dlog / sm.gt.raw_a[t];
    }
    if (t == 0) {
      float s = 0.f;
      for (int w = 0; w < NT / 64; ++w) s += sm.red[8 + w];
      dd_part[slot * H + h] = s;
    }
  }
}

__global__ void dd_reduce_kernel(const float* __restrict__ dd_part, int64_t nslots, int H, float* __restrict__ dd) {
  const int h = blockIdx.x * blockDim.x + threadIdx.x;
  if (h >= H) return;
  float s = 0.f;
  for (int64_t i = 0; i < nslots; ++i) s += dd_part[i * H + h];
  dd[h] = s;
}

template <int K, int V, typename InT>
hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t st) {
  const bool packed = a.cu_seqlens != nullptr;
  const int64_t nslots = chunk_slots(packed, a.B, a.T, a.N);
  chunk_bwd_dh_kernel<K, V, InT><<<xcd_grid(a.N * a.H, V / kDhVT), 256, 0, st>>>(
      static_cast<const InT*>(a.q), static_cast<const InT*>(a.k), a.alpha, a.beta, a.d,
      static_cast<const InT*>(a.dO), a.cu_seqlens, a.T, a.H, a.N, a.dsf, a.dhck, a.ds0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  chunk_bwd_grad_kernel<K, V, InT><<<static_cast<unsigned>(nslots * a.H), 512, 0, st>>>(
      static_cast<const InT*>(a.q), static_cast<const InT*>(a.k), static_cast<const InT*>(a.v), a.alpha, a.beta,
      a.d, static_cast<const InT*>(a.dO), a.cu_seqlens, a.T, a.H, a.N, nslots, a.hck, a.dhck, a.dq, a.dk, a.dv,
      a.dalpha, a.dbeta, a.dd_part);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  dd_reduce_kernel<<<(a.H + 63) / 64, 64, 0, st>>>(a.dd_part, nslots, a.H, a.dd);
  return hipGetLastError();
}

template <int K, int V>
hipError_t launch_bwd_kv(const BwdArgs& a, hipStream_t st) {
  if (a.in_dtype == 0) return launch_bwd_t<K, V, u16>(a, st);
  return launch_bwd_t<K, V, float>(a, st);
}

}  // namespace

hipError_t launch_chunk_bwd(const BwdArgs& a, hipStream_t st) {
  if (a.K == 128 && a.V == 128) return launch_bwd_kv<128, 128>(a, st);
  if (a.K == 128 && a.V == 64) return launch_bwd_kv<128, 64>(a, st);
  if (a.K == 64 && a.V == 128) return launch_bwd_kv<64, 128>(a, st);
  return launch_bwd_kv<64, 64>(a, st);
}

}  // namespace comba
