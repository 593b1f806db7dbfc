// Chunk-wise Comba forward for bf16 q/k/v on the gfx950 matrix cores.
//
// One workgroup owns one (sequence, head, value tile of 64 channels) and walks
// the sequence chunk by chunk. Its 8 wavefronts split into two roles that run
// one chunk apart, so the state-independent work of chunk c+1 overlaps the
// state-dependent chain of chunk c:
//
//   consumers (waves 0-3, 16 value channels each), chunk c:
//     X = [Q; K] h  ->  R = diag(beta) V - diag(beta e^Gx) K h  ->  Ubar = Tinv R
//     ->  O = diag(e^G)(Q h - d K h) + P Ubar,   h' = e^Gn h + K^T diag(e^(Gn-G)) Ubar
//     The fp32 state slice h[:, 16 channels] never leaves a consumer's registers.
//   producers (waves 4-7, one 16-row block each), chunk c+1:
//     stage q/k/v/alpha/beta in LDS, decays, Q K^T and K K^T, A and P, and the
//     unit-lower-triangular inverse Tinv = (I + A)^-1: diagonal 16x16 blocks by
//     forward substitution (vector ALU), off-diagonal blocks by column block,
//     T_ij = -T_ii sum_m A_im T_mj, on the matrix cores.
//
// Double-buffered LDS holds everything a consumer reads for one chunk. One
// workgroup barrier per chunk hands a buffer from producers to consumers;
// the producers synchronise among themselves through an LDS counter.
//
// Precision: q, k, v are exact bf16 operands. Every other operand (h, Tinv,
// P, R, Ubar, A) is split into a high and a low bf16 part; products
// hi*hi + hi*lo + lo*hi (or hi + lo against an exact operand) accumulate in
// fp32, about 16 significant bits per operand. The output correction is
// applied by linearity (Q h - d K h, Q K^T - d K K^T), never by rounding
// q - d k.
//
// Operand layout: a 16x16x32 MFMA takes 8 reduction elements per lane. An
// fp32 accumulator block holds rows 4*(lane/16)+i, so two accumulator blocks
// supply exactly the 8 reduction indices a lane needs when the other operand
// stores its reduction axis in perm32 order. Q and K tiles are stored that
// way (16-byte chunks XOR-swizzled by row against bank conflicts); K^T
// operands for the state update come from the same K tile through the
// transposing LDS read (ds_read_b64_tr_b16), so no transposed copy is kept.
#include "chunk_common.h"
#include "launch.h"
#include "comba.h"

namespace comba {

typedef short s4 __attribute__((ext_vector_type(4)));
typedef short s8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s4 lds_s4;

constexpr int kTP = 32 * 32 + 32 * 64;  // packed lower 64x64: rows 0-31 keep 32 columns, rows 32-63 keep 64

// Offset of (row, stored position) in a row-major tile of L bf16 per row whose
// 16-byte chunks are XOR-swizzled by the row index.
template <int L>
__device__ __forceinline__ int swz(int row, int pos) {
  constexpr int mask = (L / 8 - 1) < 7 ? (L / 8 - 1) : 7;
  return row * L + (((pos >> 3) ^ (row & mask)) << 3) + (pos & 7);
}
// Packed lower-triangular 64x64 (Tinv, P): the upper blocks (0,1) and (2,3)
// are stored (as zeros) because the 32-wide reduction steps read them.
__device__ __forceinline__ int tp_off(int row, int pos) {
  return row < 32 ? swz<32>(row, pos) : 1024 + swz<64>(row - 32, pos);
}
__device__ __forceinline__ int bidx(int i, int m) { return i * (i + 1) / 2 + m; }

template <int K, int VT>
struct ChunkBuf {
  u16 Q[64 * K];   // Q rows, reduction axis in perm32 order
  u16 Kc[64 * K];  // K rows, same order
  u16 Vv[64 * VT]; // V tile rows, natural order
  u16 Th[kTP], Tl[kTP], Ph[kTP], Pl[kTP];
  float beta[64], bEGx[64], EG[64], EGnG[64];
  float raw_a[64], raw_b[64];
};

struct ProdScratch {
  float Am[10 * 256];  // lower 16x16 blocks of A, fp32, row-major
  float Tm[10 * 256];  // lower 16x16 blocks of Tinv, fp32, row-major
};

template <int K, int VT>
struct SmemV2 {
  ChunkBuf<K, VT> buf[2];
  ProdScratch ps;
  int prod_bar;
};

__device__ __forceinline__ bf16x8 lds8(const u16* p) { return *reinterpret_cast<const bf16x8*>(p); }

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

__device__ __forceinline__ void split4(const f32x4& x, s4& hi, s4& lo) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    __bf16 a, b;
    split_bf16(x[j], a, b);
    hi[j] = __builtin_bit_cast(short, a);
    lo[j] = __builtin_bit_cast(short, b);
  }
}

__device__ __forceinline__ f32x4 mfma16x16x16(s4 a, s4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void put_split(u16* hi, u16* lo, int off, float x) {
  __bf16 a, b;
  split_bf16(x, a, b);
  hi[off] = __builtin_bit_cast(u16, a);
  lo[off] = __builtin_bit_cast(u16, b);
}

// Producer-only barrier (4 wavefronts) through a monotonically increasing LDS counter.
__device__ __forceinline__ void producer_sync(int* bar, int& epoch, int lane) {
  epoch += 4;
  if (lane == 0) __hip_atomic_fetch_add(bar, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
  while (__hip_atomic_load(bar, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < epoch)
    __builtin_amdgcn_s_sleep(1);
}

// A operand of K^T (rows = key channels 16kb..16kb+15, reduction = tokens
// 32s2 + {4g..4g+3, 16+4g..16+4g+3}) read from the row-major K tile.
template <int K>
__device__ __forceinline__ bf16x8 kt_frag(const u16* Kc, int kb, int s2, int g, int l16) {
  const int pos = perm_col(16 * kb + 4 * (l16 & 3));
  const int row0 = 32 * s2 + 4 * g + (l16 >> 2);
  const s4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(Kc + swz<K>(row0, pos)));
  const s4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(Kc + swz<K>(row0 + 16, pos)));
  // Whole-vector reinterpretation: element-wise short -> __bf16 casts of the
  // transposed-read result are folded into a splat of element 0 by this compiler.
  const s8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, both);
}

// ---- producer pieces --------------------------------------------------------------------

// Q K^T and K K^T for row block P, then A (fp32, scratch), P (hi/lo, buffer)
// and the diagonal block of Tinv.
template <int P, int K, int VT>
__device__ __forceinline__ void producer_rows(ChunkBuf<K, VT>& bf, ProdScratch& ps, int lane, float dh,
                                              float G, float rinv, float be) {
  const int g = lane >> 4, l16 = lane & 15;
  f32x4 aqk[P + 1], akk[P + 1];
#pragma unroll
  for (int bs = 0; bs <= P; ++bs) {
    aqk[bs] = f32x4{0.f, 0.f, 0.f, 0.f};
    akk[bs] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int s = 0; s < K / 32; ++s) {
    const bf16x8 aq = lds8(&bf.Q[swz<K>(16 * P + l16, 32 * s + 8 * g)]);
    const bf16x8 ak = lds8(&bf.Kc[swz<K>(16 * P + l16, 32 * s + 8 * g)]);
#pragma unroll
    for (int bs = 0; bs <= P; ++bs) {
      const bf16x8 bk = lds8(&bf.Kc[swz<K>(16 * bs + l16, 32 * s + 8 * g)]);
      aqk[bs] = mfma16x16x32(aq, bk, aqk[bs]);
      akk[bs] = mfma16x16x32(ak, bk, akk[bs]);
    }
  }
  float Gt[4], bt[4], rt[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = 16 * P + 4 * g + i;
    Gt[i] = __shfl(G, t, kWave);
    bt[i] = __shfl(be, t, kWave);
    rt[i] = __shfl(rinv, t, kWave);
  }
#pragma unroll
  for (int bs = 0; bs <= P; ++bs) {
    const int s_ = 16 * bs + l16;
    const float Gs = __shfl(G, s_, kWave);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * P + 4 * g + i;
      const float M = __expf(fminf(Gt[i] - Gs, 0.f));  // exp(G_t - G_s), s <= t
      const float kk = akk[bs][i];
      ps.Am[bidx(P, bs) * 256 + (4 * g + i) * 16 + l16] = (s_ < t) ? bt[i] * (M * rt[i]) * kk : 0.f;
      const float pv = (s_ <= t) ? (aqk[bs][i] - dh * kk) * M : 0.f;
      put_split(bf.Ph, bf.Pl, tp_off(t, perm_col(s_)), pv);
    }
  }
  // Diagonal block: column substitution, one lane per column.
  if (g == 0) {
    const float* Ab = &ps.Am[bidx(P, P) * 256];
    const int c = l16;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r] = (r == c) ? 1.f : 0.f;
#pragma unroll
    for (int j = 0; j < 15; ++j) {
#pragma unroll
      for (int r = j + 1; r < 16; ++r) x[r] -= Ab[r * 16 + j] * x[j];
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      ps.Tm[bidx(P, P) * 256 + r * 16 + c] = x[r];
      put_split(bf.Th, bf.Tl, tp_off(16 * P + r, perm_col(16 * P + c)), x[r]);
    }
  }
}

// Off-diagonal blocks of block column P: T_iP = -T_ii sum_{m=P}^{i-1} A_im T_mP.
template <int P, int K, int VT>
__device__ __forceinline__ void producer_offdiag(ChunkBuf<K, VT>& bf, ProdScratch& ps, int lane) {
  const int g = lane >> 4, l16 = lane & 15;
#pragma unroll
  for (int i = P + 1; i < 4; ++i) {
    f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = P; m < i; ++m) {
      const f32x4 av = *reinterpret_cast<const f32x4*>(&ps.Am[bidx(i, m) * 256 + l16 * 16 + 4 * g]);
      f32x4 bv;
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = ps.Tm[bidx(m, P) * 256 + (4 * g + j) * 16 + l16];
      s4 ah, al, bh, bl;
      split4(av, ah, al);
      split4(bv, bh, bl);
      y = mfma16x16x16(ah, bh, y);
      y = mfma16x16x16(ah, bl, y);
      y = mfma16x16x16(al, bh, y);
    }
    const f32x4 tv = *reinterpret_cast<const f32x4*>(&ps.Tm[bidx(i, i) * 256 + l16 * 16 + 4 * g]);
    s4 th, tl, yh, yl;
    split4(tv, th, tl);
    split4(y, yh, yl);
    f32x4 z = {0.f, 0.f, 0.f, 0.f};
    z = mfma16x16x16(th, yh, z);
    z = mfma16x16x16(th, yl, z);
    z = mfma16x16x16(tl, yh, z);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float val = -z[r];
      ps.Tm[bidx(i, P) * 256 + (4 * g + r) * 16 + l16] = val;
      put_split(bf.Th, bf.Tl, tp_off(16 * i + 4 * g + r, perm_col(16 * P + l16)), val);
    }
  }
}

// ---- kernel -------------------------------------------------------------------------------

template <int K, int V, int VT, typename OutT>
__global__ __launch_bounds__(512) void chunk_fwd_bf16_kernel(
    const u16* __restrict__ q, const u16* __restrict__ k, const u16* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta, const float* __restrict__ d,
    const float* __restrict__ s0, const int32_t* __restrict__ cu_seqlens,
    const int32_t* __restrict__ order, int T, int H, int N, OutT* __restrict__ o,
    float* __restrict__ sf) {
  static_assert(VT == 64, "four consumer wavefronts of 16 channels");
  constexpr int NVT = V / VT;
  __shared__ SmemV2<K, VT> sm;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wavefront-uniform role
  const int lane = tid & 63, g = lane >> 4, l16 = lane & 15;
  int unit, vt;
  if (!unit_of_block(blockIdx.x, NVT, N * H, unit, vt)) return;
  const int h = unit % H;
  int n = unit / H;
  if (order) n = order[n];
  int b, t0, t1;
  sequence_range(cu_seqlens, n, T, b, t0, t1);
  const float dh = d[h];
  const int nchunks = (t1 - t0 + 63) / 64;

  // Zero both buffers' Tinv / P storage once: the upper blocks (0,1), (2,3)
  // are read by the 32-wide reduction steps and never written.
  for (int e = tid; e < kTP; e += 512) {
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      sm.buf[bb].Th[e] = 0;
      sm.buf[bb].Tl[e] = 0;
      sm.buf[bb].Ph[e] = 0;
      sm.buf[bb].Pl[e] = 0;
    }
  }
  if (tid == 0) sm.prod_bar = 0;
  __syncthreads();

  if (wave >= 4) {
    // ======================= producers: prepare chunk i in iteration i =======================
    const int p = wave - 4;
    const int ptid = tid - 256;
    constexpr int KP = K / 8, QPT = 64 * KP / 256, VPR = VT / 8, VPT = 64 * VPR / 256;
    uint4 rq[QPT], rk[QPT], rv[VPT];
    float ra = 1.f, rb = 0.f;
    int epoch = 0;
    auto fetch = [&](int c0) {
#pragma unroll
      for (int j = 0; j < QPT; ++j) {
        const int piece = ptid + j * 256, row = piece / KP, c8 = piece % KP, t = c0 + row;
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
        const int piece = ptid + j * 256, row = piece / VPR, c8 = piece % VPR, t = c0 + row;
        if (t < t1) {
          const int64_t off = ((static_cast<int64_t>(b) * T + t) * H + h) * V + vt * VT + c8 * 8;
          rv[j] = *reinterpret_cast<const uint4*>(v + off);
        } else {
          rv[j] = make_uint4(0, 0, 0, 0);
        }
      }
      if (ptid < 64) {
        const int t = c0 + ptid;
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
    if (nchunks > 0) fetch(t0);
    for (int it = 0; it <= nchunks; ++it) {
      if (it < nchunks) {
        ChunkBuf<K, VT>& bf = sm.buf[it & 1];
#pragma unroll
        for (int j = 0; j < QPT; ++j) {
          const int piece = ptid + j * 256, row = piece / KP, c8 = piece % KP;
          const int p0 = perm_col(c8 * 8), p1 = perm_col(c8 * 8 + 4);
          *reinterpret_cast<uint2*>(&bf.Q[swz<K>(row, p0)]) = make_uint2(rq[j].x, rq[j].y);
          *reinterpret_cast<uint2*>(&bf.Q[swz<K>(row, p1)]) = make_uint2(rq[j].z, rq[j].w);
          *reinterpret_cast<uint2*>(&bf.Kc[swz<K>(row, p0)]) = make_uint2(rk[j].x, rk[j].y);
          *reinterpret_cast<uint2*>(&bf.Kc[swz<K>(row, p1)]) = make_uint2(rk[j].z, rk[j].w);
        }
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
          const int piece = ptid + j * 256, row = piece / VPR, c8 = piece % VPR;
          *reinterpret_cast<uint4*>(&bf.Vv[swz<VT>(row, c8 * 8)]) = rv[j];
        }
        if (ptid < 64) {
          bf.raw_a[ptid] = ra;
          bf.raw_b[ptid] = rb;
        }
        if (it + 1 < nchunks) fetch(t0 + (it + 1) * 64);
        producer_sync(&sm.prod_bar, epoch, lane);

        // decays: every producer wave computes all 64 rows (lane = row)
        const float a = bf.raw_a[lane], be = bf.raw_b[lane];
        const float lg = __logf(a);
        const float G = wave_inclusive_scan(lg, lane);
        const float Gn = __shfl(G, 63, kWave);
        const float rinv = 1.f / a;
        if (p == 0) {
          bf.beta[lane] = be;
          bf.bEGx[lane] = be * __expf(G - lg);
          bf.EG[lane] = __expf(G);
          bf.EGnG[lane] = __expf(Gn - G);
        }
        switch (p) {
          case 0: producer_rows<0>(bf, sm.ps, lane, dh, G, rinv, be); break;
          case 1: producer_rows<1>(bf, sm.ps, lane, dh, G, rinv, be); break;
          case 2: producer_rows<2>(bf, sm.ps, lane, dh, G, rinv, be); break;
          default: producer_rows<3>(bf, sm.ps, lane, dh, G, rinv, be); break;
        }
        producer_sync(&sm.prod_bar, epoch, lane);
        switch (p) {
          case 0: producer_offdiag<0>(bf, sm.ps, lane); break;
          case 1: producer_offdiag<1>(bf, sm.ps, lane); break;
          case 2: producer_offdiag<2>(bf, sm.ps, lane); break;
          default: break;
        }
      }
      __syncthreads();
    }
  } else {
    // ======================= consumers: run chunk i-1 in iteration i =======================
    const int vloc = wave * 16 + l16;
    const int vcol = vt * VT + vloc;
    f32x4 hs[K / 16];
    const int64_t srow = ((static_cast<int64_t>(n) * H + h) * V + vcol) * K;
#pragma unroll
    for (int kb = 0; kb < K / 16; ++kb)
      hs[kb] = s0 ? *reinterpret_cast<const f32x4*>(s0 + srow + 16 * kb + 4 * g) : f32x4{0.f, 0.f, 0.f, 0.f};

    for (int it = 0; it <= nchunks; ++it) {
      if (it > 0) {
        const int c = it - 1;
        const ChunkBuf<K, VT>& bf = sm.buf[c & 1];
        const int c0 = t0 + c * 64;
        const int nrows = min(64, t1 - c0);

        bf16x8 hbh[K / 32], hbl[K / 32];
#pragma unroll
        for (int s = 0; s < K / 32; ++s) split_pair(hs[2 * s], hs[2 * s + 1], hbh[s], hbl[s]);

        // X = [Q; K] h
        f32x4 QH[4], KH[4];
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          QH[r4] = f32x4{0.f, 0.f, 0.f, 0.f};
          KH[r4] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < K / 32; ++s) {
            const bf16x8 aq = lds8(&bf.Q[swz<K>(16 * r4 + l16, 32 * s + 8 * g)]);
            const bf16x8 ak = lds8(&bf.Kc[swz<K>(16 * r4 + l16, 32 * s + 8 * g)]);
            QH[r4] = mfma16x16x32(aq, hbh[s], QH[r4]);
            QH[r4] = mfma16x16x32(aq, hbl[s], QH[r4]);
            KH[r4] = mfma16x16x32(ak, hbh[s], KH[r4]);
            KH[r4] = mfma16x16x32(ak, hbl[s], KH[r4]);
          }
        }

        // R = beta V - beta e^Gx K h
        f32x4 R[4];
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = 16 * r4 + 4 * g + i;
            R[r4][i] = bf.beta[t] * bf16_bits_to_float(bf.Vv[swz<VT>(t, vloc)]) - bf.bEGx[t] * KH[r4][i];
          }

        // Ubar = Tinv R (row block r4 needs reduction steps 0..r4/2)
        bf16x8 rbh[2], rbl[2];
        split_pair(R[0], R[1], rbh[0], rbl[0]);
        split_pair(R[2], R[3], rbh[1], rbl[1]);
        f32x4 U[4];
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          U[r4] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s <= (r4 >> 1); ++s) {
            const int off = tp_off(16 * r4 + l16, 32 * s + 8 * g);
            const bf16x8 th = lds8(&bf.Th[off]);
            const bf16x8 tl = lds8(&bf.Tl[off]);
            U[r4] = mfma16x16x32(th, rbh[s], U[r4]);
            U[r4] = mfma16x16x32(th, rbl[s], U[r4]);
            U[r4] = mfma16x16x32(tl, rbh[s], U[r4]);
          }
        }

        // O = e^G (Q h - d K h) + P Ubar, stored straight from the accumulators
        bf16x8 ubh[2], ubl[2];
        split_pair(U[0], U[1], ubh[0], ubl[0]);
        split_pair(U[2], U[3], ubh[1], ubl[1]);
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          f32x4 acc;
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[i] = bf.EG[16 * r4 + 4 * g + i] * (QH[r4][i] - dh * KH[r4][i]);
#pragma unroll
          for (int s = 0; s <= (r4 >> 1); ++s) {
            const int off = tp_off(16 * r4 + l16, 32 * s + 8 * g);
            const bf16x8 ph = lds8(&bf.Ph[off]);
            const bf16x8 pl = lds8(&bf.Pl[off]);
            acc = mfma16x16x32(ph, ubh[s], acc);
            acc = mfma16x16x32(ph, ubl[s], acc);
            acc = mfma16x16x32(pl, ubh[s], acc);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = 16 * r4 + 4 * g + i;
            if (t < nrows)
              Elem<OutT>::store(o, ((static_cast<int64_t>(b) * T + c0 + t) * H + h) * V + vcol, acc[i]);
          }
        }

        // h' = e^Gn h + K^T diag(e^(Gn - G)) Ubar
        f32x4 Us[4];
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
#pragma unroll
          for (int i = 0; i < 4; ++i) Us[r4][i] = U[r4][i] * bf.EGnG[16 * r4 + 4 * g + i];
        bf16x8 ush[2], usl[2];
        split_pair(Us[0], Us[1], ush[0], usl[0]);
        split_pair(Us[2], Us[3], ush[1], usl[1]);
        const float eGn = bf.EG[63];
#pragma unroll
        for (int kb = 0; kb < K / 16; ++kb) {
          hs[kb] *= eGn;
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            const bf16x8 a = kt_frag<K>(bf.Kc, kb, s2, g, l16);
            hs[kb] = mfma16x16x32(a, ush[s2], hs[kb]);
            hs[kb] = mfma16x16x32(a, usl[s2], hs[kb]);
          }
        }
      }
      __syncthreads();
    }
    if (sf) {
#pragma unroll
      for (int kb = 0; kb < K / 16; ++kb) *reinterpret_cast<f32x4*>(sf + srow + 16 * kb + 4 * g) = hs[kb];
    }
  }
}

template <int K, int V, typename OutT>
static hipError_t launch_bf16_t(const FwdArgs& a, hipStream_t st) {
  constexpr int VT = 64, NVT = V / VT;
  const int units = a.N * a.H;
  chunk_fwd_bf16_kernel<K, V, VT, OutT><<<xcd_grid(units, NVT), 512, 0, st>>>(
      static_cast<const u16*>(a.q), static_cast<const u16*>(a.k), static_cast<const u16*>(a.v), a.alpha,
      a.beta, a.d, a.s0, a.cu_seqlens, a.order, a.T, a.H, a.N, static_cast<OutT*>(a.o), a.sf);
  return hipGetLastError();
}

template <int K, int V>
static hipError_t launch_bf16_kv(const FwdArgs& a, hipStream_t st) {
  if (a.out_dtype == COMBA_BF16) return launch_bf16_t<K, V, u16>(a, st);
  return launch_bf16_t<K, V, float>(a, st);
}

hipError_t launch_chunk_bf16(const FwdArgs& a, hipStream_t st) {
  if (a.K == 128 && a.V == 128) return launch_bf16_kv<128, 128>(a, st);
  if (a.K == 128 && a.V == 64) return launch_bf16_kv<128, 64>(a, st);
  if (a.K == 64 && a.V == 128) return launch_bf16_kv<64, 128>(a, st);
  return launch_bf16_kv<64, 64>(a, st);
}

}  // namespace comba
