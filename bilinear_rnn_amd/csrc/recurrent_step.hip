// Recurrent (token-by-token) Comba kernel; with one token it is the decode step.
//
// Per head and value row i (the recurrence expanded for one step):
//   a = S[i,:] . k,  b = S[i,:] . qt,  qt = q - d k,  u = v_i - a
//   S'[i,:] = alpha S[i,:] + beta u k^T,   o_i = alpha b + beta u (k . qt)
// One read and one write of the fp32 state per token range: the kernel is
// bound by HBM bandwidth. A state row (K floats) is spread over the 16 lanes
// of one DPP row, each holding K/16 floats as 16-byte pieces at columns
// 4 j + 64 f (lane j of the row, piece f): every load instruction reads
// 256 contiguous bytes of four rows. The two K-reductions per row are four
// DPP steps inside those 16 lanes (no LDS traffic). The state stays in
// registers across tokens.
#include "device_common.h"
#include "launch.h"
#include "comba.h"

namespace comba {

template <typename InT> struct Load4;
template <> struct Load4<float> {
  __device__ static void get(const float* p, int64_t i, float (&x)[4]) {
    const f32x4 t = *reinterpret_cast<const f32x4*>(p + i);
    x[0] = t[0]; x[1] = t[1]; x[2] = t[2]; x[3] = t[3];
  }
};
template <> struct Load4<u16> {
  __device__ static void get(const u16* p, int64_t i, float (&x)[4]) {
    const uint2 t = *reinterpret_cast<const uint2*>(p + i);
    x[0] = __uint_as_float(t.x << 16);
    x[1] = __uint_as_float(t.x & 0xffff0000u);
    x[2] = __uint_as_float(t.y << 16);
    x[3] = __uint_as_float(t.y & 0xffff0000u);
  }
};

// One workgroup per (sequence, head, block of VB value rows).
template <int K, int V, int VB, typename InT, typename OutT>
__global__ __launch_bounds__(256) void recurrent_kernel(
    const InT* __restrict__ q, const InT* __restrict__ k, const InT* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta, const float* __restrict__ d,
    const float* s0, const int32_t* __restrict__ cu_seqlens, int T, int H, int Hk,
    OutT* __restrict__ o, float* sf, unsigned fusion) {
  constexpr int F4 = K / 64;   // 16-byte pieces per lane and row
  constexpr int RPP = 16;       // rows per pass: 4 per wavefront
  constexpr int NP = VB / RPP;  // passes
  constexpr int NB = V / VB;    // row blocks per (sequence, head)
  const int vb = blockIdx.x % NB;
  const int h = (blockIdx.x / NB) % H, hk = h / (H / Hk);
  const int n = blockIdx.x / (NB * H);
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int rw = lane >> 4, j = lane & 15;
  int b, t0, t1;
  sequence_range(cu_seqlens, n, T, b, t0, t1);

  const int64_t sbase = (static_cast<int64_t>(n) * H + h) * V * K + 4 * j;
  f32x4 S[NP][F4];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int row = vb * VB + p * RPP + w * 4 + rw;
#pragma unroll
    for (int f = 0; f < F4; ++f)
      S[p][f] = s0 ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(s0 + sbase + row * K + 64 * f))
                   : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float dh = d[h];

  for (int t = t0; t < t1; ++t) {
    const int64_t tok = (static_cast<int64_t>(b) * T + t) * H + h;     // value head h
    const int64_t tqk = (static_cast<int64_t>(b) * T + t) * Hk + hk;   // its q / k head
    float kk[F4][4], qt[F4][4];
    float kq = 0.f;
#pragma unroll
    for (int f = 0; f < F4; ++f) {
      Load4<InT>::get(k, tqk * K + 4 * j + 64 * f, kk[f]);
      Load4<InT>::get(q, tqk * K + 4 * j + 64 * f, qt[f]);
    }
    if (fusion & kFuseQkL2Norm) {  // q, k / sqrt(sum of squares + eps), in float32
      float sk = 0.f, sq = 0.f;
#pragma unroll
      for (int f = 0; f < F4; ++f)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sk += kk[f][e] * kk[f][e];
          sq += qt[f][e] * qt[f][e];
        }
      const float rk = 1.f / sqrtf(row16_sum(sk) + kL2NormEps), rq = 1.f / sqrtf(row16_sum(sq) + kL2NormEps);
#pragma unroll
      for (int f = 0; f < F4; ++f)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kk[f][e] *= rk;
          qt[f][e] *= rq;
        }
    }
#pragma unroll
    for (int f = 0; f < F4; ++f)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qt[f][e] -= dh * kk[f][e];
        kq += kk[f][e] * qt[f][e];
      }
    kq = row16_sum(kq);
    float a = alpha[tok], be = beta[tok];
    if (fusion & kFuseGateLogits) {
      a = sigmoid_stable(a);
      be = sigmoid_stable(be);
    }
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int row = vb * VB + p * RPP + w * 4 + rw;
      float sk = 0.f, sq = 0.f;
#pragma unroll
      for (int f = 0; f < F4; ++f)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sk += S[p][f][e] * kk[f][e];
          sq += S[p][f][e] * qt[f][e];
        }
      sk = row16_sum(sk);
      sq = row16_sum(sq);
      const float u = Elem<InT>::load(v, tok * V + row) - sk;
      const float bu = be * u;
#pragma unroll
      for (int f = 0; f < F4; ++f)
#pragma unroll
        for (int e = 0; e < 4; ++e) S[p][f][e] = a * S[p][f][e] + bu * kk[f][e];
      if (j == 0) Elem<OutT>::store(o, tok * V + row, a * sq + bu * kq);
    }
  }
  if (sf) {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int row = vb * VB + p * RPP + w * 4 + rw;
#pragma unroll
      for (int f = 0; f < F4; ++f)
        __builtin_nontemporal_store(S[p][f], reinterpret_cast<f32x4*>(sf + sbase + row * K + 64 * f));
    }
  }
}

template <int K, int V, typename InT, typename OutT>
static hipError_t launch_rec_t(const FwdArgs& a, hipStream_t st) {
  // 32 value rows per workgroup (16 KB of state at K = 128): few enough
  // registers for eight wavefronts per SIMD and a grid of N H V / 32
  // workgroups. Measured on the decode workload: 16 rows per workgroup is
  // slower (more redundant k / q loads), 64 rows too (fewer waves in flight).
  constexpr int VB = 32;
  const int grid = a.N * a.H * (V / VB);
  recurrent_kernel<K, V, VB, InT, OutT><<<grid, 256, 0, st>>>(
      static_cast<const InT*>(a.q), static_cast<const InT*>(a.k), static_cast<const InT*>(a.v),
      a.alpha, a.beta, a.d, a.s0, a.cu_seqlens, a.T, a.H, a.Hk, static_cast<OutT*>(a.o), a.sf, a.fusion);
  return hipGetLastError();
}

template <int K, int V>
static hipError_t launch_rec_kv(const FwdArgs& a, hipStream_t st) {
  const bool ib = a.in_dtype == COMBA_BF16, ob = a.out_dtype == COMBA_BF16;
  if (ib && ob) return launch_rec_t<K, V, u16, u16>(a, st);
  if (ib) return launch_rec_t<K, V, u16, float>(a, st);
  if (ob) return launch_rec_t<K, V, float, u16>(a, st);
  return launch_rec_t<K, V, float, float>(a, st);
}

hipError_t launch_recurrent(const FwdArgs& a, hipStream_t st) {
  if (a.K == 128 && a.V == 128) return launch_rec_kv<128, 128>(a, st);
  if (a.K == 128 && a.V == 64) return launch_rec_kv<128, 64>(a, st);
  if (a.K == 64 && a.V == 128) return launch_rec_kv<64, 128>(a, st);
  return launch_rec_kv<64, 64>(a, st);
}

}  // namespace comba
