// Chunk-wise Comba forward for fp32 q/k/v: the same chunk algebra as the
// bf16 kernel (see chunk_common.h) in plain fp32 vector arithmetic, so that
// fp32 inputs keep fp32 accuracy end to end. One workgroup owns one
// (sequence, head, value tile of 16 channels); the state slice lives in LDS.
#include "chunk_common.h"
#include "launch.h"
#include "comba.h"

namespace comba {

template <int K>
struct alignas(16) SmemF32 {
  static constexpr int VT = 16;
  static constexpr int LDH = VT + 1;
  float Qs[64 * (K + 1)];
  float Ks[64 * (K + 1)];
  float Vs[64 * VT];
  float Am[64 * kLdF];
  float Tm[64 * kLdF];
  float Pm[64 * kLdF];
  float Hs[K * LDH];    // h = S^T slice, K x VT
  float Rs[64 * LDH];   // R, then Ubar
  float Os[64 * LDH];   // output accumulator
  float Ys[3 * 256];
  ChunkGates gt;
};

template <int K, int V, typename OutT>
__global__ __launch_bounds__(256) void chunk_fwd_fp32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta, const float* __restrict__ d,
    const float* s0, const int32_t* __restrict__ cu_seqlens,
    const int32_t* __restrict__ order, int T, int H, int Hk, int N, OutT* o,
    float* sf, unsigned fusion, float* hck) {
  constexpr int NT = 256, VT = SmemF32<K>::VT, LDH = SmemF32<K>::LDH, NVT = V / VT, LQ = K + 1;
  __shared__ SmemF32<K> sm;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  int unit, vt;
  if (!unit_of_block(blockIdx.x, NVT, N * H, unit, vt)) return;
  const int h = unit % H, hk = h / (H / Hk);
  int n = unit / H;
  if (order) n = order[n];
  int b, t0, t1;
  sequence_range(cu_seqlens, n, T, b, t0, t1);
  const float dh = d[h];
  const int64_t sbase = (static_cast<int64_t>(n) * H + h) * V * K;

  for (int e = tid; e < K * VT; e += NT) {
    const int kk = e % K, c = e / K;
    sm.Hs[kk * LDH + c] = (fusion & kModeIdentityInit) ? (vt * VT + c == kk ? 1.f : 0.f)
                          : s0 ? s0[sbase + static_cast<int64_t>(vt * VT + c) * K + kk] : 0.f;
  }

  const int nchunks = (t1 - t0 + 63) / 64;
  for (int ci = 0; ci < nchunks; ++ci) {
    const int c0 = t0 + ci * 64;
    const int nrows = min(64, t1 - c0);
    __syncthreads();
    if (hck) {  // keep the chunk's incoming state (for the backward)
      float* dst = hck + ((chunk_slot(cu_seqlens != nullptr, t0, n, ci, T) * H + h) * V + vt * VT) * K;
      for (int e = tid; e < K * VT; e += NT) {
        const int kk = e % K, c = e / K;
        dst[static_cast<int64_t>(c) * K + kk] = sm.Hs[kk * LDH + c];
      }
    }
    for (int e = tid; e < 64 * K; e += NT) {
      const int row = e / K, c = e % K, t = c0 + row;
      const int64_t off = ((static_cast<int64_t>(b) * T + t) * Hk + hk) * K + c;
      sm.Qs[row * LQ + c] = row < nrows ? q[off] : 0.f;
      sm.Ks[row * LQ + c] = row < nrows ? k[off] : 0.f;
    }
    for (int e = tid; e < 64 * VT; e += NT) {
      const int row = e / VT, c = e % VT, t = c0 + row;
      sm.Vs[e] = (row < nrows && !(fusion & kModeZeroV)) ? v[((static_cast<int64_t>(b) * T + t) * H + h) * V + vt * VT + c]
                                                        : 0.f;
    }
    if (tid < 64) {
      const int64_t tok = (static_cast<int64_t>(b) * T + c0 + tid) * H + h;
      float ra = 1.f, rb = 0.f;  // padding rows: no decay, no write
      if (tid < nrows) {
        ra = alpha[tok];
        rb = beta[tok];
        if (fusion & kFuseGateLogits) {
          ra = sigmoid_stable(ra);
          rb = sigmoid_stable(rb);
        }
      }
      sm.gt.raw_a[tid] = ra;
      sm.gt.raw_b[tid] = rb;
    }
    __syncthreads();
    if (fusion & kFuseQkL2Norm) {  // normalise the staged q and k rows in place
      if (tid < 128) {
        float* row = (tid < 64 ? sm.Qs : sm.Ks) + (tid & 63) * LQ;
        float ss = 0.f;
        for (int c = 0; c < K; ++c) ss += row[c] * row[c];
        const float r = 1.f / sqrtf(ss + kL2NormEps);
        for (int c = 0; c < K; ++c) row[c] *= r;
      }
      __syncthreads();
    }
    if (wave == 0) chunk_gates(sm.gt, lane, nrows);
    __syncthreads();

    // A (strictly lower) and P (lower) from K K^T and Q K^T
    for (int e = tid; e < 64 * 64; e += NT) {
      const int t = e >> 6, s = e & 63;
      if ((s >> 4) > (t >> 4)) continue;
      float qk = 0.f, kk = 0.f;
      for (int c = 0; c < K; ++c) {
        qk += sm.Qs[t * LQ + c] * sm.Ks[s * LQ + c];
        kk += sm.Ks[t * LQ + c] * sm.Ks[s * LQ + c];
      }
      sm.Am[t * kLdF + s] = (s < t) ? sm.gt.beta[t] * decay_Gx(sm.gt, t, s) * kk : 0.f;
      sm.Pm[t * kLdF + s] = (s <= t) ? (qk - dh * kk) * decay_G(sm.gt, t, s) : 0.f;
    }
    __syncthreads();
    unit_lower_inverse64<NT>(sm.Am, sm.Tm, sm.Ys, tid);

    // R = beta V - beta exp(Gx) K h ;  O = exp(G) (Q h - d K h)
    for (int e = tid; e < 64 * VT; e += NT) {
      const int t = e / VT, c = e % VT;
      float kh = 0.f, qh = 0.f;
      for (int kk = 0; kk < K; ++kk) {
        const float hv = sm.Hs[kk * LDH + c];
        kh += sm.Ks[t * LQ + kk] * hv;
        qh += sm.Qs[t * LQ + kk] * hv;
      }
      sm.Rs[t * LDH + c] = sm.gt.beta[t] * sm.Vs[t * VT + c] - sm.gt.bEGx[t] * kh;
      sm.Os[t * LDH + c] = sm.gt.EG[t] * (qh - dh * kh);
    }
    __syncthreads();
    // Ubar = Tinv R (kept in registers, then written over R)
    float ub[64 * VT / NT];
#pragma unroll
    for (int j = 0; j < 64 * VT / NT; ++j) {
      const int e = tid + j * NT, t = e / VT, c = e % VT;
      float acc = 0.f;
      for (int r = 0; r <= t; ++r) acc += sm.Tm[t * kLdF + r] * sm.Rs[r * LDH + c];
      ub[j] = acc;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 64 * VT / NT; ++j) {
      const int e = tid + j * NT, t = e / VT, c = e % VT;
      sm.Rs[t * LDH + c] = ub[j];
    }
    __syncthreads();
    // O += P Ubar, write out
    for (int e = tid; e < 64 * VT; e += NT) {
      const int t = e / VT, c = e % VT;
      float acc = sm.Os[t * LDH + c];
      for (int s = 0; s <= t; ++s) acc += sm.Pm[t * kLdF + s] * sm.Rs[s * LDH + c];
      if (t < nrows && !(fusion & kModeNoOutput))
        Elem<OutT>::store(o, ((static_cast<int64_t>(b) * T + c0 + t) * H + h) * V + vt * VT + c, acc);
    }
    // h' = exp(G_n) h + K^T diag(exp(G_n - G)) Ubar
    const float eGn = sm.gt.EG[63];
    for (int e = tid; e < K * VT; e += NT) {
      const int kk = e / VT, c = e % VT;
      float acc = 0.f;
      for (int t = 0; t < 64; ++t) acc += sm.Ks[t * LQ + kk] * sm.gt.EGnG[t] * sm.Rs[t * LDH + c];
      sm.Hs[kk * LDH + c] = eGn * sm.Hs[kk * LDH + c] + acc;
    }
  }
  __syncthreads();
  if (sf) {
    for (int e = tid; e < K * VT; e += NT) {
      const int kk = e % K, c = e / K;
      sf[sbase + static_cast<int64_t>(vt * VT + c) * K + kk] = sm.Hs[kk * LDH + c];
    }
  }
}

template <int K, int V, typename OutT>
static hipError_t launch_f32_t(const FwdArgs& a, hipStream_t st) {
  constexpr int NVT = V / SmemF32<K>::VT;
  chunk_fwd_fp32_kernel<K, V, OutT><<<xcd_grid(a.N * a.H, NVT), 256, 0, st>>>(
      static_cast<const float*>(a.q), static_cast<const float*>(a.k), static_cast<const float*>(a.v),
      a.alpha, a.beta, a.d, a.s0, a.cu_seqlens, a.order, a.T, a.H, a.Hk, a.N, static_cast<OutT*>(a.o), a.sf, a.fusion,
      a.hck);
  return hipGetLastError();
}

template <int K, int V>
static hipError_t launch_f32_kv(const FwdArgs& a, hipStream_t st) {
  if (a.out_dtype == COMBA_BF16) return launch_f32_t<K, V, u16>(a, st);
  return launch_f32_t<K, V, float>(a, st);
}

hipError_t launch_chunk_fp32(const FwdArgs& a, hipStream_t st) {
  if (a.K == 128 && a.V == 128) return launch_f32_kv<128, 128>(a, st);
  if (a.K == 128 && a.V == 64) return launch_f32_kv<128, 64>(a, st);
  if (a.K == 64 && a.V == 128) return launch_f32_kv<64, 128>(a, st);
  return launch_f32_kv<64, 64>(a, st);
}

}  // namespace comba
