// Recurrent (token-by-token) Comba kernel; with one token it is the decode step.
//
// Per head and value row i (the recurrence expanded for one step):
//   a = S[i,:] . k,  b = S[i,:] . qt,  qt = q - d k,  u = v_i - a
//   S'[i,:] = alpha S[i,:] + beta u k^T,   o_i = alpha b + beta u (k . qt)
// One read and one write of the fp32 state per token range: the kernel is
// bound by HBM bandwidth. Each state row (K floats) is spread over K/4 lanes
// holding 4 contiguous floats (one 16-byte access per lane), so a wavefront
// reads whole 512-byte rows; the two K-reductions per row are butterfly
// shuffles inside those lanes. The state stays in registers across tokens.
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

template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int m = LPR / 2; m > 0; m >>= 1) x += __shfl_xor(x, m, LPR);
  return x;
}

template <int K, int V, typename InT, typename OutT>
__global__ __launch_bounds__(256) void recurrent_kernel(
    const InT* __restrict__ q, const InT* __restrict__ k, const InT* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta, const float* __restrict__ d,
    const float* s0, const int32_t* __restrict__ cu_seqlens, int T, int H,
    OutT* __restrict__ o, float* sf) {
  constexpr int LPR = K / 4;        // lanes per state row
  constexpr int RPW = kWave / LPR;  // rows per wavefront
  constexpr int RPP = RPW * 4;      // rows per pass of the 4 wavefronts
  constexpr int NP = V / RPP;       // passes
  const int h = blockIdx.x % H;
  const int n = blockIdx.x / H;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int rw = lane / LPR, c4 = lane % LPR;
  int b, t0, t1;
  sequence_range(cu_seqlens, n, T, b, t0, t1);

  const int64_t sbase = (static_cast<int64_t>(n) * H + h) * V * K + 4 * c4;
  f32x4 S[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int row = p * RPP + w * RPW + rw;
    if (s0)
      S[p] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(s0 + sbase + row * K));
    else
      S[p] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float dh = d[h];

  for (int t = t0; t < t1; ++t) {
    const int64_t tok = (static_cast<int64_t>(b) * T + t) * H + h;
    float kk[4], qt[4];
    Load4<InT>::get(k, tok * K + 4 * c4, kk);
    Load4<InT>::get(q, tok * K + 4 * c4, qt);
#pragma unroll
    for (int j = 0; j < 4; ++j) qt[j] -= dh * kk[j];
    const float kq = group_sum<LPR>(kk[0] * qt[0] + kk[1] * qt[1] + kk[2] * qt[2] + kk[3] * qt[3]);
    const float a = alpha[tok], be = beta[tok];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int row = p * RPP + w * RPW + rw;
      float sk = S[p][0] * kk[0] + S[p][1] * kk[1] + S[p][2] * kk[2] + S[p][3] * kk[3];
      float sq = S[p][0] * qt[0] + S[p][1] * qt[1] + S[p][2] * qt[2] + S[p][3] * qt[3];
      sk = group_sum<LPR>(sk);
      sq = group_sum<LPR>(sq);
      const float u = Elem<InT>::load(v, tok * V + row) - sk;
      const float bu = be * u;
#pragma unroll
      for (int j = 0; j < 4; ++j) S[p][j] = a * S[p][j] + bu * kk[j];
      if (c4 == 0) Elem<OutT>::store(o, tok * V + row, a * sq + bu * kq);
    }
  }
  if (sf) {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int row = p * RPP + w * RPW + rw;
      __builtin_nontemporal_store(S[p], reinterpret_cast<f32x4*>(sf + sbase + row * K));
    }
  }
}

template <int K, int V, typename InT, typename OutT>
static hipError_t launch_rec_t(const FwdArgs& a, hipStream_t st) {
  const int grid = a.N * a.H;
  recurrent_kernel<K, V, InT, OutT><<<grid, 256, 0, st>>>(
      static_cast<const InT*>(a.q), static_cast<const InT*>(a.k), static_cast<const InT*>(a.v),
      a.alpha, a.beta, a.d, a.s0, a.cu_seqlens, a.T, a.H, static_cast<OutT*>(a.o), a.sf);
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
