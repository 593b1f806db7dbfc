// Chunk-wise Comba forward for bf16 q/k/v on the gfx950 matrix cores.
//
// One workgroup owns one (sequence, head, value tile of VT channels) and walks
// the sequence chunk by chunk; the state slice h[:, tile] (K x VT, fp32) never
// leaves registers. Wavefront w owns 16 value channels of the tile and runs
// the whole state-dependent chain for them on its own:
//   X = [Q; K] h  ->  R  ->  Ubar = Tinv R  ->  O, h'
// The h-independent part of a chunk (decays, Q K^T and K K^T, the one
// unit-lower-triangular inverse, the masked score matrix P) is shared by the
// wavefronts through LDS.
//
// Precision: q, k, v are exact bf16 matrix-core operands. Every other operand
// (h, Tinv, P, R, Ubar) is split into a high and a low bf16 part and the
// products hi*hi + hi*lo + lo*hi (or hi + lo against an exact operand) are
// accumulated in fp32, about 16 significant bits per operand. The output
// correction is applied by linearity in fp32 (Q h - d K h and
// Q K^T - d K K^T), never by rounding q - d k.
//
// Operand layout: the 16x16x32 bf16 MFMA takes 8 reduction elements per lane.
// fp32 accumulators hold rows 4*(lane/16)+i of a 16-row block, so two
// accumulator blocks give exactly the 8 reduction indices a lane needs if the
// other operand stores its reduction axis in perm32 order. Every LDS operand
// with a reduction axis (Q, K, K^T, Tinv, P) is stored that way, and all
// state-dependent operands move from one product to the next without leaving
// the lane.
#include "chunk_common.h"
#include "launch.h"
#include "comba.h"

namespace comba {

template <int K, int VT>
struct SmemBf16 {
  static constexpr int LDQ = K + 8;   // Qs, Ks row stride (bf16)
  static constexpr int LDKT = 64 + 8; // Kt row stride
  static constexpr int LDV = VT + 8;  // Vs row stride
  static constexpr int LDP = 64 + 8;  // Th, Tl, Ph, Pl row stride
  u16 Qs[64 * LDQ];                   // Q rows, reduction axis permuted
  u16 Ks[64 * LDQ];                   // K rows, reduction axis permuted
  u16 Kt[K * LDKT];                   // K^T (rows = key channel), token axis permuted
  u16 Vs[64 * LDV];                   // V tile rows, natural order
  float Am[64 * kLdF];                // A, then the fp32 output staging
  float Tm[64 * kLdF];                // Tinv in fp32
  u16 Th[64 * LDP], Tl[64 * LDP];     // Tinv hi / lo, columns permuted
  u16 Ph[64 * LDP], Pl[64 * LDP];     // P hi / lo, columns permuted
  float Ys[3 * 256];
  ChunkGates gt;
};

__device__ __forceinline__ bf16x8 lds8(const u16* p) { return *reinterpret_cast<const bf16x8*>(p); }

// Build the two B-operand halves (hi, lo) from accumulator blocks m0 (first
// 16 reduction rows) and m1 (next 16), optionally scaled per row.
__device__ __forceinline__ void split_pair(const f32x4& m0, const f32x4& m1, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    __bf16 a, b;
    split_bf16(m0[j], a, b);
    hi[j] = a;
    lo[j] = b;
    split_bf16(m1[j], a, b);
    hi[j + 4] = a;
    lo[j + 4] = b;
  }
}

template <int K, int V, int VT, typename OutT>
__global__ __launch_bounds__(VT / 16 * 64) void chunk_fwd_bf16_kernel(
    const u16* __restrict__ q, const u16* __restrict__ k, const u16* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta, const float* __restrict__ d,
    const float* __restrict__ s0, const int32_t* __restrict__ cu_seqlens,
    const int32_t* __restrict__ order, int T, int H, int N, OutT* __restrict__ o,
    float* __restrict__ sf) {
  constexpr int NW = VT / 16, NT = NW * 64, NVT = V / VT;
  using Sm = SmemBf16<K, VT>;
  constexpr int LDQ = Sm::LDQ, LDKT = Sm::LDKT, LDV = Sm::LDV, LDP = Sm::LDP;
  constexpr int KP = K / 8;            // 16-byte pieces per q/k row
  constexpr int QPT = 64 * KP / NT;    // pieces per thread per chunk
  constexpr int VPR = VT / 8;          // 16-byte pieces per v-tile row
  constexpr int VPT = 64 * VPR / NT;
  static_assert(QPT * NT == 64 * KP && VPT * NT == 64 * VPR, "tile split");
  __shared__ Sm sm;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
  int unit, vt;
  if (!unit_of_block(blockIdx.x, NVT, N * H, unit, vt)) return;
  const int h = unit % H;
  int n = unit / H;
  if (order) n = order[n];
  int b, t0, t1;
  sequence_range(cu_seqlens, n, T, b, t0, t1);
  const float dh = d[h];
  const int vcol = vt * VT + wave * 16 + l16;  // this lane's value channel

  // State slice: hs[kb][i] = h[16 kb + 4 g + i][vcol] = S[vcol][16 kb + 4 g + i].
  f32x4 hs[K / 16];
  const int64_t srow = ((static_cast<int64_t>(n) * H + h) * V + vcol) * K;
#pragma unroll
  for (int kb = 0; kb < K / 16; ++kb)
    hs[kb] = s0 ? *reinterpret_cast<const f32x4*>(s0 + srow + 16 * kb + 4 * g) : f32x4{0.f, 0.f, 0.f, 0.f};

  // Upper blocks of Tinv / P are read as zeros by the triangular products and
  // never written afterwards.
  for (int e = tid; e < 64 * LDP; e += NT) {
    sm.Th[e] = 0;
    sm.Tl[e] = 0;
    sm.Ph[e] = 0;
    sm.Pl[e] = 0;
  }

  uint4 rq[QPT], rk[QPT], rv[VPT];
  float ra = 1.f, rb = 0.f;
  auto fetch = [&](int c0) {
#pragma unroll
    for (int j = 0; j < QPT; ++j) {
      const int piece = tid + j * NT, row = piece / KP, c8 = piece % KP, t = c0 + row;
      if (t < t1) {
        const int64_t off = ((static_cast<int64_t>(b) * T + t) * H + h) * K + c8 * 8;
        rq[j] = *reinterpret_cast<const uint4*>(q + off);
        rk[j] = *reinterpret_cast<const uint4*>(k + off);
      } else {
        rq[j] = make_uint4(0, 0, 0, 0);
        rk[j] = make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int piece = tid + j * NT, row = piece / VPR, c8 = piece % VPR, t = c0 + row;
      if (t < t1) {
        const int64_t off = ((static_cast<int64_t>(b) * T + t) * H + h) * V + vt * VT + c8 * 8;
        rv[j] = *reinterpret_cast<const uint4*>(v + off);
      } else {
        rv[j] = make_uint4(0, 0, 0, 0);
      }
    }
    if (tid < 64) {
      const int t = c0 + tid;
      if (t < t1) {
        const int64_t tok = (static_cast<int64_t>(b) * T + t) * H + h;
        ra = alpha[tok];
        rb = beta[tok];
      } else {
        ra = 1.f;
        rb = 0.f;
      }
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int j = 0; j < QPT; ++j) {
      const int piece = tid + j * NT, row = piece / KP, c8 = piece % KP;
      const int p0 = perm_col(c8 * 8), p1 = perm_col(c8 * 8 + 4);
      *reinterpret_cast<uint2*>(&sm.Qs[row * LDQ + p0]) = make_uint2(rq[j].x, rq[j].y);
      *reinterpret_cast<uint2*>(&sm.Qs[row * LDQ + p1]) = make_uint2(rq[j].z, rq[j].w);
      *reinterpret_cast<uint2*>(&sm.Ks[row * LDQ + p0]) = make_uint2(rk[j].x, rk[j].y);
      *reinterpret_cast<uint2*>(&sm.Ks[row * LDQ + p1]) = make_uint2(rk[j].z, rk[j].w);
      const int tp = perm_col(row);
      const uint32_t w4[4] = {rk[j].x, rk[j].y, rk[j].z, rk[j].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sm.Kt[(c8 * 8 + 2 * e) * LDKT + tp] = static_cast<u16>(w4[e] & 0xffffu);
        sm.Kt[(c8 * 8 + 2 * e + 1) * LDKT + tp] = static_cast<u16>(w4[e] >> 16);
      }
    }
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int piece = tid + j * NT, row = piece / VPR, c8 = piece % VPR;
      *reinterpret_cast<uint4*>(&sm.Vs[row * LDV + c8 * 8]) = rv[j];
    }
    if (tid < 64) {
      sm.gt.raw_a[tid] = ra;
      sm.gt.raw_b[tid] = rb;
    }
  };

  const int nchunks = (t1 - t0 + 63) / 64;
  if (nchunks > 0) fetch(t0);
  for (int ci = 0; ci < nchunks; ++ci) {
    const int c0 = t0 + ci * 64;
    const int nrows = min(64, t1 - c0);
    __syncthreads();
    stash();
    __syncthreads();
    if (ci + 1 < nchunks) fetch(c0 + 64);
    if (wave == 0) chunk_gates(sm.gt, lane, nrows);
    __syncthreads();

    // ---- Q K^T and K K^T on the lower 16x16 blocks; A and P ----
    for (int task = wave; task < 10; task += NW) {
      const int bt = task < 1 ? 0 : task < 3 ? 1 : task < 6 ? 2 : 3;
      const int bs = task - (bt * (bt + 1)) / 2;
      f32x4 aqk = {0.f, 0.f, 0.f, 0.f}, akk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < K / 32; ++s) {
        const bf16x8 aq = lds8(&sm.Qs[(16 * bt + l16) * LDQ + 32 * s + 8 * g]);
        const bf16x8 ak = lds8(&sm.Ks[(16 * bt + l16) * LDQ + 32 * s + 8 * g]);
        const bf16x8 bk = lds8(&sm.Ks[(16 * bs + l16) * LDQ + 32 * s + 8 * g]);
        aqk = mfma16x16x32(aq, bk, aqk);
        akk = mfma16x16x32(ak, bk, akk);
      }
      const int s_ = 16 * bs + l16;
      const float Gs = sm.gt.G[s_];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * bt + 4 * g + i;
        sm.Am[t * kLdF + s_] = (s_ < t) ? sm.gt.beta[t] * expf(sm.gt.Gx[t] - Gs) * akk[i] : 0.f;
        const float p = (s_ <= t) ? (aqk[i] - dh * akk[i]) * expf(sm.gt.G[t] - Gs) : 0.f;
        __bf16 ph, pl;
        split_bf16(p, ph, pl);
        sm.Ph[t * LDP + perm_col(s_)] = __builtin_bit_cast(u16, ph);
        sm.Pl[t * LDP + perm_col(s_)] = __builtin_bit_cast(u16, pl);
      }
    }
    __syncthreads();
    unit_lower_inverse64<NT>(sm.Am, sm.Tm, sm.Ys, tid);
    for (int e = tid; e < 64 * 64; e += NT) {
      const int t = e >> 6, s = e & 63;
      if ((s >> 4) <= (t >> 4)) {
        __bf16 th, tl;
        split_bf16(sm.Tm[t * kLdF + s], th, tl);
        sm.Th[t * LDP + perm_col(s)] = __builtin_bit_cast(u16, th);
        sm.Tl[t * LDP + perm_col(s)] = __builtin_bit_cast(u16, tl);
      }
    }
    __syncthreads();

    // ---- state-dependent chain, per wavefront (16 value channels) ----
    bf16x8 hbh[K / 32], hbl[K / 32];
#pragma unroll
    for (int s = 0; s < K / 32; ++s) split_pair(hs[2 * s], hs[2 * s + 1], hbh[s], hbl[s]);

    f32x4 QH[4], KH[4];
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      QH[r4] = f32x4{0.f, 0.f, 0.f, 0.f};
      KH[r4] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < K / 32; ++s) {
        const bf16x8 aq = lds8(&sm.Qs[(16 * r4 + l16) * LDQ + 32 * s + 8 * g]);
        const bf16x8 ak = lds8(&sm.Ks[(16 * r4 + l16) * LDQ + 32 * s + 8 * g]);
        QH[r4] = mfma16x16x32(aq, hbh[s], QH[r4]);
        QH[r4] = mfma16x16x32(aq, hbl[s], QH[r4]);
        KH[r4] = mfma16x16x32(ak, hbh[s], KH[r4]);
        KH[r4] = mfma16x16x32(ak, hbl[s], KH[r4]);
      }
    }

    // R = beta V - beta exp(Gx) K h
    f32x4 R[4];
    const int vloc = wave * 16 + l16;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * r4 + 4 * g + i;
        R[r4][i] = sm.gt.beta[t] * bf16_bits_to_float(sm.Vs[t * LDV + vloc]) - sm.gt.bEGx[t] * KH[r4][i];
      }

    // Ubar = Tinv R (Tinv lower triangular: row block r4 needs k-steps 0..r4/2)
    bf16x8 rbh[2], rbl[2];
    split_pair(R[0], R[1], rbh[0], rbl[0]);
    split_pair(R[2], R[3], rbh[1], rbl[1]);
    f32x4 U[4];
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      U[r4] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s <= (r4 >> 1); ++s) {
        const bf16x8 th = lds8(&sm.Th[(16 * r4 + l16) * LDP + 32 * s + 8 * g]);
        const bf16x8 tl = lds8(&sm.Tl[(16 * r4 + l16) * LDP + 32 * s + 8 * g]);
        U[r4] = mfma16x16x32(th, rbh[s], U[r4]);
        U[r4] = mfma16x16x32(th, rbl[s], U[r4]);
        U[r4] = mfma16x16x32(tl, rbh[s], U[r4]);
      }
    }

    // O = exp(G) (Q h - d K h) + P Ubar  -> fp32 staging (reuses Am)
    bf16x8 ubh[2], ubl[2];
    split_pair(U[0], U[1], ubh[0], ubl[0]);
    split_pair(U[2], U[3], ubh[1], ubl[1]);
    float* Os = sm.Am;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      f32x4 acc;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * r4 + 4 * g + i;
        acc[i] = sm.gt.EG[t] * (QH[r4][i] - dh * KH[r4][i]);
      }
#pragma unroll
      for (int s = 0; s <= (r4 >> 1); ++s) {
        const bf16x8 ph = lds8(&sm.Ph[(16 * r4 + l16) * LDP + 32 * s + 8 * g]);
        const bf16x8 pl = lds8(&sm.Pl[(16 * r4 + l16) * LDP + 32 * s + 8 * g]);
        acc = mfma16x16x32(ph, ubh[s], acc);
        acc = mfma16x16x32(ph, ubl[s], acc);
        acc = mfma16x16x32(pl, ubh[s], acc);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) Os[(16 * r4 + 4 * g + i) * kLdF + vloc] = acc[i];
    }

    // h' = exp(G_n) h + K^T diag(exp(G_n - G)) Ubar
    f32x4 Us[4];
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
#pragma unroll
      for (int i = 0; i < 4; ++i) Us[r4][i] = U[r4][i] * sm.gt.EGnG[16 * r4 + 4 * g + i];
    bf16x8 ush[2], usl[2];
    split_pair(Us[0], Us[1], ush[0], usl[0]);
    split_pair(Us[2], Us[3], ush[1], usl[1]);
    const float eGn = sm.gt.EG[63];
#pragma unroll
    for (int kb = 0; kb < K / 16; ++kb) {
      hs[kb] *= eGn;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const bf16x8 a = lds8(&sm.Kt[(16 * kb + l16) * LDKT + 32 * s + 8 * g]);
        hs[kb] = mfma16x16x32(a, ush[s], hs[kb]);
        hs[kb] = mfma16x16x32(a, usl[s], hs[kb]);
      }
    }
    __syncthreads();

    // write the chunk's outputs (rows < nrows)
    constexpr int OPR = VT / 4;  // 4-element groups per row
    for (int e = tid; e < 64 * OPR; e += NT) {
      const int row = e / OPR, c4 = e % OPR;
      if (row < nrows) {
        const float* src = &Os[row * kLdF + 4 * c4];
        const int64_t off = ((static_cast<int64_t>(b) * T + c0 + row) * H + h) * V + vt * VT + 4 * c4;
        if constexpr (sizeof(OutT) == 2) {
          const uint32_t lo = float_to_bf16_bits(src[0]) | (static_cast<uint32_t>(float_to_bf16_bits(src[1])) << 16);
          const uint32_t hi = float_to_bf16_bits(src[2]) | (static_cast<uint32_t>(float_to_bf16_bits(src[3])) << 16);
          *reinterpret_cast<uint2*>(o + off) = make_uint2(lo, hi);
        } else {
          *reinterpret_cast<f32x4*>(o + off) = f32x4{src[0], src[1], src[2], src[3]};
        }
      }
    }
  }

  if (sf) {
#pragma unroll
    for (int kb = 0; kb < K / 16; ++kb) *reinterpret_cast<f32x4*>(sf + srow + 16 * kb + 4 * g) = hs[kb];
  }
}

template <int K, int V, int VT, typename OutT>
static hipError_t launch_bf16_t(const FwdArgs& a, hipStream_t st) {
  constexpr int NVT = V / VT;
  const int units = a.N * a.H;
  chunk_fwd_bf16_kernel<K, V, VT, OutT><<<xcd_grid(units, NVT), VT / 16 * 64, 0, st>>>(
      static_cast<const u16*>(a.q), static_cast<const u16*>(a.k), static_cast<const u16*>(a.v), a.alpha,
      a.beta, a.d, a.s0, a.cu_seqlens, a.order, a.T, a.H, a.N, static_cast<OutT*>(a.o), a.sf);
  return hipGetLastError();
}

template <int K, int V>
static hipError_t launch_bf16_kv(const FwdArgs& a, hipStream_t st) {
  if (a.out_dtype == COMBA_BF16) return launch_bf16_t<K, V, 64, u16>(a, st);
  return launch_bf16_t<K, V, 64, float>(a, st);
}

hipError_t launch_chunk_bf16(const FwdArgs& a, hipStream_t st) {
  if (a.K == 128 && a.V == 128) return launch_bf16_kv<128, 128>(a, st);
  if (a.K == 128 && a.V == 64) return launch_bf16_kv<128, 64>(a, st);
  if (a.K == 64 && a.V == 128) return launch_bf16_kv<64, 128>(a, st);
  return launch_bf16_kv<64, 64>(a, st);
}

}  // namespace comba
