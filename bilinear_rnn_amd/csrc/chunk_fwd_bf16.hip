// Chunk-wise Comba forward for bf16 q/k/v on the gfx950 matrix cores.
//
// One workgroup owns one (sequence, head, value tile of 64 channels) and walks
// the sequence chunk by chunk. Its 8 wavefronts split into two roles that run
// one chunk apart, so the state-independent work of chunk c+1 overlaps the
// state-dependent chain of chunk c:
//
//   consumers (waves 0-3, 16 value channels each), chunk c:
//     X = [Q; K] h,  R = diag(beta) V - diag(beta e^Gx) K h,
//     Ubar = (I + A)^-1 R by 32-token blocks:
//         Ubar_top = T1 R_top,  Ubar_bot = T2 (R_bot - A21 Ubar_top),
//     O = diag(e^G)(Q h - d K h) + P Ubar,   h' = e^Gn h + K^T diag(e^(Gn-G)) Ubar
//     The fp32 state slice h[:, 16 channels] never leaves a consumer's registers.
//   producers (waves 4-7), chunk c+1:
//     stage q/k/v/alpha/beta in LDS, decays, then the ten lower-triangular
//     16x16 blocks of Q K^T and K K^T shared out in balanced sets (wave p
//     always holds diagonal block p), scaled into A (strictly lower) and P
//     (masked scores), and the two 32x32 diagonal inverses T1 = (I + A11)^-1,
//     T2 = (I + A22)^-1: wave p inverts its 16x16 diagonal block by fp32
//     forward substitution; after a producer-only sync the odd waves form the
//     off-diagonal block T_{p,p-1} = -T_pp A_{p,p-1} T_{p-1,p-1} on the
//     matrix cores.
//
// Double-buffered LDS holds everything a consumer reads for one chunk; one
// workgroup barrier per chunk hands a buffer from producers to consumers.
//
// Instantiations: output in bf16 or fp32; q / k normalised in the kernel or
// not; a state-only form (no Q K^T, P or output stage) for passes that need
// final states only; and chunk_fwd_bf16_pair_kernel, a state-only form with a
// second group of four consumers (waves 8-11) that runs the same chunks from
// the identity with v = 0, for the segment-parallel forward's segment maps.
//
// Precision: q, k, v are exact bf16 operands. Every other operand (h, T1, T2,
// A21, P, R, Ubar) is split into a high and a low bf16 part; the products
// hi*hi + hi*lo + lo*hi (or hi + lo against an exact operand) accumulate in
// fp32, about 16 significant bits per operand. The output correction is
// applied by linearity (Q h - d K h, Q K^T - d K K^T), never by rounding
// q - d k.
//
// Operand layout: a 16x16x32 MFMA takes 8 reduction elements per lane. An
// fp32 accumulator block holds rows 4*(lane/16)+i, so two accumulator blocks
// supply exactly the 8 reduction indices a lane needs when the other operand
// stores its reduction axis in perm32 order. Q, K, T and P are stored that way
// (16-byte chunks XOR-swizzled by row against bank conflicts). Fragments are
// read as one 16-byte LDS read each: the compiler fuses two 8-byte reads whose
// addresses differ by a multiple of 512 bytes into one two-address read, which
// costs about three times as much as a conflict-free 16-byte read. K^T operands
// for the state update and V for R come from row-major tiles through the
// transposing LDS read (ds_read_b64_tr_b16).
#include "bf16_tiles.h"
#include "chunk_common.h"
#include "launch.h"
#include "comba.h"

namespace comba {

constexpr int kTP = 32 * 32 + 32 * 64;  // packed 64x64: rows 0-31 keep 32 columns, rows 32-63 keep 64

__device__ __forceinline__ int tp_off(int row, int pos) {
  // rows 0-31: 32 per row (64 bytes, four rows per 256 bytes), 16-byte chunks
  // swizzled by (row >> 2) & 3; rows 32-63: 64 per row after the first 1024 (two
  // rows per 256 bytes), swizzled by (row >> 1) & 7. Measured with the LDS
  // bank-conflict counter: fragment reads of rows 32-63 are conflict-free; those
  // of rows 0-31, and the producers' 8-byte writes, are two-way under every XOR
  // swizzle of the four (or eight) chunks of a row.
  const int big = row >> 5;
  const int base = row * (32 << big) - 1024 * big;
  const int sw = big ? (row >> 1) & 7 : (row >> 2) & 3;
  return base + (((pos >> 3) ^ sw) << 3) + (pos & 7);
}

// Offset of position pos of row `row` in a q / k tile (K bf16 per row): the
// 16-byte chunk index is XOR-ed with a linear function of the row bits. The
// functions (and the producers' staging rows below) were chosen against the
// LDS bank-conflict counter, measured on gfx950 for each access pattern of
// the kernel: the 16-byte row fragments of sixteen consecutive rows (K h, Q h
// and the producers' blocks) and the producers' 8-byte staging writes are
// conflict-free, and the transposed K^T reads of the state update two-way, the
// least for 8-byte pieces that all sit in the same half of their chunks. The
// part's bank mapping is not the plain one on address bits 2-7: swizzles that
// are conflict-free under it (row bits 0-3 reversed or rotated) measure
// two-way on the fragments.
//   K = 128: row bits 0, 1, 2 -> chunk bits {1}, {2}, {0, 3}.
//   K = 64:  row bits 0-2 -> chunk bits 0-2 (chunk c of row r at c ^ (r mod 8)).
template <int K>
__device__ __forceinline__ int qk_off(int row, int pos) {
  static_assert(K == 128 || K == 64, "64 or 128 keys");
  const int sw = K == 128 ? ((row & 3) << 1) ^ (9 * ((row >> 2) & 1)) : row & 7;
  return row * K + (((pos >> 3) ^ sw) << 3) + (pos & 7);
}

// Position of row t of a chunk in the lane-ordered gate arrays: lane group g
// of a consumer reads its 16 rows t = 16 r4 + 4 g + i as four float4.
__device__ __forceinline__ int gate_pos(int t) { return ((t >> 2) & 3) * 16 + (t >> 4) * 4 + (t & 3); }

// 16-byte aligned so that buf[1] keeps every b128 / b64 LDS access aligned.
template <int K, int VT>
struct alignas(16) ChunkBuf {
  u16 Q[64 * K];    // Q rows, reduction axis in perm32 order
  u16 Kc[64 * K];   // K rows, same order
  u16 Vv[64 * VT];  // V tile rows, natural order
  // Th/Tl: rows 0-31 hold T1; rows 32-63 hold -A21 (columns 0-31) and T2
  // (columns 32-63). Ph/Pl: the masked score matrix P. hi / lo bf16 parts.
  u16 Th[kTP], Tl[kTP], Ph[kTP], Pl[kTP];
  // beta, beta e^Gx r_k, e^G r_q, e^(Gn-G) r_k, d e^G r_k in gate_pos order (r_q, r_k:
  // the per-token L2 factors of q and k when they are normalised in the kernel, else 1)
  float gl[5][64];
  float raw_a[64], raw_b[64];
  float rn[2][64];  // r_q, r_k by token (normalisation only)
  float eGn;
};

// Row stride of the fp32 16x16 scratch blocks: 20 floats puts the four rows
// that a lane quad reads together on different banks.
constexpr int kSS = 20;

struct alignas(16) ProdScratch {  // one per producer wave, fp32 16x16 blocks, row-major
  float Aown[16 * kSS];           // A_pp
  float Aoff[16 * kSS];           // A_{p,p-1} (odd p)
  float Town[16 * kSS];           // T_pp
  // Per-token decay factors of this wave's blocks, indexed by token in chunk:
  // diagonal block: G_t and Gx_t (inclusive and exclusive cumulative log2 alpha), beta_t and,
  // when q and k are normalised in the kernel, G_t - log2 r_k(t) (column factor); off-diagonal
  // block j (column
  // block C, last token r = 16 C + 15): beta_t e^(Gx_t - G_r), e^(G_t - G_r)
  // (rows) and e^(G_r - G_s) (columns).
  float dG[64], dB[64], dGx[64], dGk[64];
  float oA[2][64], oP[2][64], oS[2][64];
};

template <int K, int VT>
struct alignas(16) SmemV3 {
  ChunkBuf<K, VT> buf[2];
  ProdScratch ps[4];
  int prod_bar;
  int pair_flag[2];
};

__device__ __forceinline__ f32x4 lds_f4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }

// 2^x with the hardware instruction (about 1 ulp; x <= 0 here, underflow to 0 is exact enough).
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// sigmoid(x) = 1 / (1 + e^-x), from e = e^-|x| in (0, 1] so that nothing
// overflows; hardware exp2 and reciprocal (about 1 ulp each).
__device__ __forceinline__ float sigmoid_fast(float x) {
  const float e = exp2_fast(-fabsf(x) * 1.44269504f);
  const float r = __builtin_amdgcn_rcpf(1.f + e);
  return x >= 0.f ? r : e * r;
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

// K^T operand (rows = key channels 16kb..16kb+15, reduction = tokens
// 32s2 + {4g..4g+3, 16+4g..16+4g+3}) from the row-major K tile.
template <int K>
__device__ __forceinline__ bf16x8 kt_frag(const u16* Kc, int kb, int s2, int g, int l16) {
  const int pos = perm_col(16 * kb + 4 * (l16 & 3));
  const int row0 = 32 * s2 + 4 * g + (l16 >> 2);
  const s4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(Kc + qk_off<K>(row0, pos)));
  const s4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(Kc + qk_off<K>(row0 + 16, pos)));
  // Whole-vector reinterpretation: element-wise short -> __bf16 casts of the
  // transposed-read result are folded into a splat of element 0 by this compiler.
  const s8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, both);
}

// V[16 r4 + 4g + j][col0 + l16], j = 0..3, from the row-major V tile.
template <int VT>
__device__ __forceinline__ f32x4 v_frag(const u16* Vv, int r4, int col0, int g, int l16) {
  const int row = 16 * r4 + 4 * g + (l16 >> 2);
  const s4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(Vv + swz<VT>(row, col0 + 4 * (l16 & 3))));
  const uint2 w = __builtin_bit_cast(uint2, x);  // whole-vector reinterpretation (see kt_frag)
  return f32x4{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u), __uint_as_float(w.y << 16),
               __uint_as_float(w.y & 0xffff0000u)};
}

// ---- producer pieces ---------------------------------------------------------------------

// (I + A)^-1 of a 16x16 diagonal block whose strictly lower part is in Ab
// (fp32, row-major, zeros on and above the diagonal): forward substitution by
// columns, four lanes per column (lane = 4c + q holds rows 4q..4q+3 of
// column c), the pivot broadcast inside each lane quad with DPP. All of A is
// read before the substitution starts, so the chain waits on LDS once. The
// result goes to Tb (fp32, for the off-diagonal step) and, split into hi / lo
// bf16, straight from the registers into the T tile at (row0, row0).
template <int K, int VT>
__device__ __forceinline__ void invert16(ChunkBuf<K, VT>& bf, const float* Ab, float* Tb, int row0, int lane) {
  const int c = lane >> 2, q = lane & 3;
  f32x4 a[4][4];  // [column block j4][row 4q + r]: A[4q + r][4 j4 .. 4 j4 + 3]
#pragma unroll
  for (int j4 = 0; j4 < 4; ++j4)
#pragma unroll
    for (int r = 0; r < 4; ++r) a[j4][r] = lds_f4(Ab + (4 * q + r) * kSS + 4 * j4);
  float x[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) x[r] = (4 * q + r == c) ? 1.f : 0.f;
#pragma unroll
  for (int j4 = 0; j4 < 4; ++j4) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int j = 4 * j4 + jj;
      if (j == 15) break;
      // x[j] of this column lives in lane quad member j/4 (= j4), register j%4 (= jj)
      const int src = __builtin_bit_cast(int, x[jj]);
      int bc;
      switch (j4) {
        case 0: bc = __builtin_amdgcn_update_dpp(0, src, 0x00, 0xf, 0xf, false); break;
        case 1: bc = __builtin_amdgcn_update_dpp(0, src, 0x55, 0xf, 0xf, false); break;
        case 2: bc = __builtin_amdgcn_update_dpp(0, src, 0xaa, 0xf, 0xf, false); break;
        default: bc = __builtin_amdgcn_update_dpp(0, src, 0xff, 0xf, 0xf, false); break;
      }
      const float xj = __builtin_bit_cast(float, bc);
#pragma unroll
      for (int r = 0; r < 4; ++r) x[r] -= a[j4][r][jj] * xj;  // a = 0 unless 4q + r > j
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) Tb[(4 * q + r) * kSS + c] = x[r];
  unsigned h01, l01, h23, l23;
  split2(x[0], x[1], h01, l01);
  split2(x[2], x[3], h23, l23);
  const unsigned hw[4] = {h01, h01 >> 16, h23, h23 >> 16}, lw[4] = {l01, l01 >> 16, l23, l23 >> 16};
  const int pc = perm_col(row0 + c);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int off = tp_off(row0 + 4 * q + r, pc);
    bf.Th[off] = static_cast<u16>(hw[r]);
    bf.Tl[off] = static_cast<u16>(lw[r]);
  }
}

// Scale one transposed block (see producer_blocks) into P and A and write
// them: this lane holds row t = 16 R + l16, columns s = 16 C + 4 g + i.
// B = 0 is the wave's diagonal block; B >= 1 an off-diagonal one whose decay
// factors are in the wave's tables (slot B - 1).
template <int B, int R, int C, bool NORM, bool SO, int K, int VT>
__device__ __forceinline__ void scale_block(ChunkBuf<K, VT>& bf, ProdScratch& ps, int lane, float dh,
                                            const f32x4& qk, const f32x4& kk4) {
  const int g = lane >> 4, l16 = lane & 15;
  const int t = 16 * R + l16;
  f32x4 av, pv;
  if constexpr (B == 0) {
    // diagonal block: masks and two exps per element (both tokens in one block):
    // e^(G_t - G_s) for P and e^(Gx_t - G_s) for A, so that A never divides by
    // alpha_t. With normalisation the column factor r_k(s) rides in the exponent
    // (G_s - log2 r_k(s)) and the row factors in per-row constants; the clamp
    // only matters for the masked entries.
    const float Gt = ps.dG[t], Gxt = ps.dGx[t];
    const f32x4 Gs = lds_f4(&(NORM ? ps.dGk : ps.dG)[16 * C + 4 * g]);
    float ca = ps.dB[t], cq = 1.f, ck = dh;  // beta_t, then r_k(t), r_q(t), d r_k(t)
    if constexpr (NORM) {
      const float rqt = bf.rn[0][t], rkt = bf.rn[1][t];
      ca *= rkt;
      cq = rqt;
      ck = dh * rkt;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s_ = 16 * C + 4 * g + i;
      const float M = exp2_fast(fminf(Gt - Gs[i], NORM ? 64.f : 0.f));    // e^(G_t - G_s) [r_k(s)], s <= t
      const float Mx = exp2_fast(fminf(Gxt - Gs[i], NORM ? 64.f : 0.f));  // e^(Gx_t - G_s) [r_k(s)], s < t
      const float kk = kk4[i];
      av[i] = (s_ < t) ? ca * Mx * kk : 0.f;  // beta_t e^(Gx_t - G_s) k_t.k_s
      pv[i] = (s_ <= t) ? (NORM ? qk[i] * cq - ck * kk : qk[i] - dh * kk) * M : 0.f;
    }
  } else {
    // ta and ts carry r_k(t) and r_k(s) when q and k are normalised
    const float ta = ps.oA[B - 1][t], tp = ps.oP[B - 1][t];
    const f32x4 ts = lds_f4(&ps.oS[B - 1][16 * C + 4 * g]);
    float cq = tp, ck = dh * tp;  // e^(G_t - G_r) [r_q(t)], d e^(G_t - G_r) [r_k(t)]
    if constexpr (NORM) {
      cq *= bf.rn[0][t];
      ck *= bf.rn[1][t];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float kk = kk4[i] * ts[i];
      av[i] = ta * kk;
      pv[i] = qk[i] * ts[i] * cq - kk * ck;
    }
  }
  const int col = perm_col(16 * C + 4 * g);
  if constexpr (!SO) put_split4(bf.Ph, bf.Pl, tp_off(t, col), pv);
  if constexpr (B == 0) *reinterpret_cast<f32x4*>(&ps.Aown[l16 * kSS + 4 * g]) = av;
  if constexpr ((R & 1) != 0 && C == R - 1) *reinterpret_cast<f32x4*>(&ps.Aoff[l16 * kSS + 4 * g]) = av;
  if constexpr (R >= 2 && C < 2) put_split4(bf.Th, bf.Tl, tp_off(t, col), -av);  // -A21
}

// One-way hand-over between two producer waves through an LDS flag that
// holds the index (plus one) of the last chunk whose data is ready.
__device__ __forceinline__ void pair_signal(int* flag, int tag, int lane) {
  if (lane == 0) __hip_atomic_store(flag, tag, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void pair_wait(const int* flag, int tag) {
  while (__hip_atomic_load(flag, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < tag)
    __builtin_amdgcn_s_sleep(1);
}

// T_{D,D-1} = -T_DD A_{D,D-1} T_{D-1,D-1} for odd D. The first product uses
// only this wave's data and runs before waiting for the even neighbour's
// T_{D-1,D-1}. Both are formed transposed: W^T = A^T T_DD^T leaves W^T in the
// layout of a B operand, and (W T_{D-1,D-1})^T = T_{D-1,D-1}^T W^T gives a
// lane row l16 and columns 4 g .. 4 g + 3 of the result, one 8-byte piece.
template <int D, int K, int VT>
__device__ __forceinline__ void offdiag_inverse(ChunkBuf<K, VT>& bf, const ProdScratch& ps,
                                                const ProdScratch& prev, const int* pair_flag, int tag,
                                                int lane) {
  const int g = lane >> 4, l16 = lane & 15;
  f32x4 acol;
#pragma unroll
  for (int j = 0; j < 4; ++j) acol[j] = ps.Aoff[(4 * g + j) * kSS + l16];
  s4 ah, al, th, tl;
  split4(acol, ah, al);
  split4(lds_f4(&ps.Town[l16 * kSS + 4 * g]), th, tl);
  f32x4 wt = {0.f, 0.f, 0.f, 0.f};
  wt = mfma16x16x16(ah, th, wt);
  wt = mfma16x16x16(ah, tl, wt);
  wt = mfma16x16x16(al, th, wt);
  s4 wh, wl;
  split4(wt, wh, wl);
  pair_wait(pair_flag, tag);
  f32x4 pcol;
#pragma unroll
  for (int j = 0; j < 4; ++j) pcol[j] = prev.Town[(4 * g + j) * kSS + l16];
  s4 ph, pl;
  split4(pcol, ph, pl);
  f32x4 r = {0.f, 0.f, 0.f, 0.f};
  r = mfma16x16x16(ph, wh, r);
  r = mfma16x16x16(ph, wl, r);
  r = mfma16x16x16(pl, wh, r);
  put_split4(bf.Th, bf.Tl, tp_off(16 * D + l16, perm_col(16 * (D - 1) + 4 * g)), -r);
}

// One producer's share of the chunk's ten lower-triangular 16x16 blocks
// (row block R, column block C <= R): its diagonal block (D, D) first, then up
// to two more, (R1, C1) and (R2, C2). The shares are balanced so that no wave
// carries more than three blocks next to its diagonal inverse:
//   wave 0: (0,0) (3,0) (3,1)   wave 1: (1,1) (1,0)
//   wave 2: (2,2) (2,0) (2,1)   wave 3: (3,3) (3,2)
// (waves 1 and 3 also form the off-diagonal inverse block afterwards).
// For each block: Q K^T and K K^T on the matrix cores, then A (strictly lower,
// beta_t e^(Gx_t - G_s) k_t.k_s) and P ((q_t.k_s - d k_t.k_s) e^(G_t - G_s), s <= t)
// written as hi / lo bf16. A_DD goes to the wave's scratch for its inverse;
// A_{R,R-1} (odd R) to the scratch for the off-diagonal step; the A blocks
// below the 32x32 diagonal enter T's storage negated (-A21).
template <int D, int NB, int R1, int C1, int R2, int C2, bool NORM, bool SO, int K, int VT>
__device__ __forceinline__ void producer_blocks(ChunkBuf<K, VT>& bf, ProdScratch& ps, const ProdScratch& prev,
                                                int* pair_flag, int chunk_tag, int lane, float dh,
                                                float G, float lg, float be, float rk) {
  constexpr int Rb[3] = {D, R1, R2};
  constexpr int Cb[3] = {D, C1, C2};
  const int g = lane >> 4, l16 = lane & 15;
  // Decay tables (lane = token). Off-diagonal blocks (every s < every t)
  // factor e^(G_t - G_s) = e^(G_t - G_r) e^(G_r - G_s) through the column
  // block's last token r: both factors lie in (0, 1], so no per-element exp.
  ps.dG[lane] = G;
  ps.dB[lane] = be;
  ps.dGx[lane] = G - lg;
  if constexpr (NORM) ps.dGk[lane] = G - __builtin_amdgcn_logf(rk);
#pragma unroll
  for (int b = 1; b < NB; ++b) {
    const float Gr = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, G), 16 * Cb[b] + 15));
    ps.oA[b - 1][lane] = be * exp2_fast(fminf(G - lg - Gr, 0.f)) * rk;  // beta_t e^(Gx_t - G_r) r_k, t > r
    ps.oP[b - 1][lane] = exp2_fast(fminf(G - Gr, 0.f));                 // e^(G_t - G_r), t > r
    ps.oS[b - 1][lane] = exp2_fast(fminf(Gr - G, 0.f)) * rk;            // e^(G_r - G_s) r_k, s <= r
  }
  // Each block is formed transposed, K_C Q_R^T and K_C K_R^T (K K^T is
  // symmetric): the accumulator then gives a lane one row t = 16 R + l16 and
  // four consecutive columns s = 16 C + 4 g + i, i.e. a contiguous 8-byte
  // piece of a row of P, A or T, written without any lane exchange.
  f32x4 aqk[NB], akk[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    aqk[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    akk[b] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int s = 0; s < K / 32; ++s) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const bf16x8 ak = lds8(&bf.Kc[qk_off<K>(16 * Rb[b] + l16, 32 * s + 8 * g)]);
      const bf16x8 bk = lds8(&bf.Kc[qk_off<K>(16 * Cb[b] + l16, 32 * s + 8 * g)]);
      if constexpr (!SO) {  // q k^T only feeds P, which a state-only pass does not form
        const bf16x8 aq = lds8(&bf.Q[qk_off<K>(16 * Rb[b] + l16, 32 * s + 8 * g)]);
        aqk[b] = mfma16x16x32(bk, aq, aqk[b]);
      }
      akk[b] = mfma16x16x32(bk, ak, akk[b]);
    }
  }
  scale_block<0, D, D, NORM, SO>(bf, ps, lane, dh, aqk[0], akk[0]);
  if constexpr ((D & 1) != 0) scale_block<1, R1, C1, NORM, SO>(bf, ps, lane, dh, aqk[1], akk[1]);  // A_{D,D-1}
  // diagonal inverse of this wave's block (reads this wave's own scratch writes)
  invert16(bf, ps.Aown, ps.Town, 16 * D, lane);
  if constexpr ((D & 1) == 0) {
    // T_DD is what the odd neighbour waits for: signal it before the rest.
    pair_signal(pair_flag, chunk_tag, lane);
    if constexpr (NB > 1) scale_block<1, R1, C1, NORM, SO>(bf, ps, lane, dh, aqk[1], akk[1]);
    if constexpr (NB > 2) scale_block<2, R2, C2, NORM, SO>(bf, ps, lane, dh, aqk[2], akk[2]);
  } else {
    static_assert(NB == 2 && R1 == D && C1 == D - 1, "odd waves hold (D, D) and (D, D-1)");
    offdiag_inverse<D>(bf, ps, prev, pair_flag, chunk_tag, lane);
  }
}

// Sum of squares of the eight bf16 values in a 16-byte piece: four bf16-pair
// dot products accumulated in fp32 (each bf16 square is exact in fp32). The
// words go through scalar copies: a bit cast applied directly to a vector
// subscript reads element 0 for every index with this compiler.
__device__ __forceinline__ float sumsq8(const u32x4& w) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const unsigned e[4] = {w.x, w.y, w.z, w.w};
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16x2 p = __builtin_bit_cast(bf16x2, e[i]);
    ss = __builtin_amdgcn_fdot2_f32_bf16(p, p, ss, false);
  }
  return ss;
}

// ---- kernel -------------------------------------------------------------------------------

// The kernel body. PAIR (a state-only pass for the segment-parallel forward,
// K == V): a second group of four consumer wavefronts (waves 8-11) runs the
// same chunks from the identity with v = 0 over K state rows and writes its
// final state to sf2, the segment's K x K map, while waves 0-3 form the
// segment-end state from zero; the producers' work serves both groups.
template <int K, int V, int VT, typename OutT, bool NORM, bool SO, bool PAIR>
__device__ __forceinline__ void chunk_fwd_bf16_body(
    const u16* __restrict__ q, const u16* __restrict__ k, const u16* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta, const float* __restrict__ d,
    const float* s0, const int32_t* __restrict__ cu_seqlens,
    const int32_t* __restrict__ order, int T, int H, int Hk, int N, OutT* o,
    float* sf, unsigned fusion, float* hck, float* sf2) {
  static_assert(VT == 64, "four consumer wavefronts of 16 channels");
  static_assert(!PAIR || (SO && K == V), "the paired pass is state-only, with K == V");
  constexpr int NVT = V / VT, NT = PAIR ? 768 : 512;
  __shared__ SmemV3<K, VT> sm;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wavefront-uniform role
  const int lane = tid & 63, g = lane >> 4, l16 = lane & 15;
  int unit, vt;
  if (!unit_of_block(blockIdx.x, NVT, N * H, unit, vt)) return;
  const int h = unit % H, hk = h / (H / Hk);
  int n = unit / H;
  if (order) n = __builtin_amdgcn_readfirstlane(order[n]);
  int b, t0, t1;
  sequence_range(cu_seqlens, n, T, b, t0, t1);
  // The bounds are the same for every lane (loaded values): keep them, and
  // all address arithmetic derived from them, in scalar registers.
  t0 = __builtin_amdgcn_readfirstlane(t0);
  t1 = __builtin_amdgcn_readfirstlane(t1);
  const float dh = d[h];
  const int nchunks = (t1 - t0 + 63) / 64;

  // Zero both buffers' T / P storage once: the upper blocks (0,1), (2,3) are
  // read by the 32-wide reduction steps and never written.
  for (int e = tid; e < kTP; e += NT) {
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      sm.buf[bb].Th[e] = 0;
      sm.buf[bb].Tl[e] = 0;
      sm.buf[bb].Ph[e] = 0;
      sm.buf[bb].Pl[e] = 0;
    }
  }
  if (tid == 0) {
    sm.prod_bar = 0;
    sm.pair_flag[0] = 0;
    sm.pair_flag[1] = 0;
  }
  __syncthreads();

  if (wave >= 4 && (!PAIR || wave < 8)) {
    // ======================= producers: prepare chunk it in iteration it =======================
    const int p = wave - 4;
    const int ptid = tid - 256;
    constexpr int KP = K / 8, QPT = 64 * KP / 256, VPR = VT / 8, VPT = 64 * VPR / 256;
    u32x4 rq[QPT], rk[QPT], rv[VPT];
    float ra = 1.f, rb = 0.f;
    int epoch = 0;
    // Byte offsets of this thread's 16-byte pieces inside one chunk (row of
    // the chunk times the token stride, plus the column): the same for every
    // chunk, so each load below is one buffer instruction without address
    // arithmetic. Rows past the end of the sequence lie beyond the chunk's
    // buffer range and load as zeros (the padding the chunk algebra needs).
    int qkoff[QPT], voff[VPT];
    // Column (16-byte piece of a row) of this thread's q / k pieces, and the row
    // of its piece j; together a bijection onto the tile's pieces. Each 16-lane
    // group of the 8-byte LDS writes below spans two rows, which keeps the
    // writes conflict-free (measured; one row per group is two-way whatever the
    // swizzle). For K = 128 the two rows' pieces are not on consecutive lanes,
    // which the in-kernel normalisation's row sums need: that instantiation
    // keeps one row per 16 consecutive lanes (two-way writes).
    constexpr bool SPREAD = K == 128 && !NORM;
    const int qk_col = SPREAD ? (ptid & 7) | (((ptid >> 4) & 1) << 3) : ptid % KP;
    auto qk_row = [&](int j) {
      if constexpr (SPREAD) {
        return 16 * j + ((ptid >> 6) & 1) + (((ptid >> 5) & 1) << 1) + (((ptid >> 3) & 1) << 2) + ((ptid >> 7) << 3);
      } else if constexpr (K == 128) {
        return 16 * j + 4 * ((ptid >> 4) & 3) + (ptid >> 6);
      } else {
        const int ph = ptid >> 5, grp = (ptid >> 3) & 3;
        return 32 * j + (ph & 1) * 2 + (ph >> 1) * 8 + (grp & 1) + 4 * (grp >> 1);
      }
    };
#pragma unroll
    for (int j = 0; j < QPT; ++j) qkoff[j] = (qk_row(j) * Hk * K + qk_col * 8) * 2;
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int piece = ptid + j * 256, row = piece / VPR, c8 = piece % VPR;
      voff[j] = (row * H * V + c8 * 8) * 2;
    }
    auto fetch = [&](int c0) {
      const int nrows = min(64, t1 - c0);
      const int64_t tok0 = (static_cast<int64_t>(b) * T + c0) * H + h;      // token c0, value head h
      const int64_t tqk0 = (static_cast<int64_t>(b) * T + c0) * Hk + hk;    // token c0, its q / k head
      const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc(
          uniform_ptr(const_cast<u16*>(q + tqk0 * K)), static_cast<short>(0),
          __builtin_amdgcn_readfirstlane(nrows * Hk * K * 2), kBufferWord3);
      const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
          uniform_ptr(const_cast<u16*>(k + tqk0 * K)), static_cast<short>(0),
          __builtin_amdgcn_readfirstlane(nrows * Hk * K * 2), kBufferWord3);
      const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
          uniform_ptr(const_cast<u16*>(v + tok0 * V + vt * VT)), static_cast<short>(0),
          __builtin_amdgcn_readfirstlane((fusion & kModeZeroV) ? 0 : nrows * H * V * 2), kBufferWord3);
#pragma unroll
      for (int j = 0; j < QPT; ++j) {
        rq[j] = __builtin_amdgcn_raw_buffer_load_b128(qr, qkoff[j], 0, 0);
        rk[j] = __builtin_amdgcn_raw_buffer_load_b128(kr, qkoff[j], 0, 0);
      }
#pragma unroll
      for (int j = 0; j < VPT; ++j) rv[j] = __builtin_amdgcn_raw_buffer_load_b128(vr, voff[j], 0, 0);
      if (ptid < 64) {
        if (ptid < nrows) {
          const int64_t tok = tok0 + static_cast<int64_t>(ptid) * H;
          ra = alpha[tok];
          rb = beta[tok];
        } else {  // padding token: no decay, no write
          ra = 1.f;
          rb = 0.f;
        }
      }
    };
    // LDS offsets of this thread's first q / k pieces (two 8-byte halves in perm32
    // order) and first v piece; 256 is a multiple of the pieces per row, so every
    // later piece keeps the column and the row's swizzle phase
    static_assert(256 % KP == 0 && 256 % VPR == 0, "a thread's pieces share their column");
    const int sq0 = qk_off<K>(qk_row(0), perm_col(qk_col * 8)), sq1 = qk_off<K>(qk_row(0), perm_col(qk_col * 8 + 4));
    const int sv0 = swz<VT>(ptid / VPR, ptid % VPR * 8);
    if (nchunks > 0) fetch(t0);
    for (int it = 0; it <= nchunks; ++it) {
      if (it < nchunks) {
        ChunkBuf<K, VT>& bf = sm.buf[it & 1];
        // Opaque per-iteration copy of the lane index: keeps the compiler from
        // hoisting every lane-dependent LDS address of the four row-block
        // variants out of the loop (which exhausts the registers and spills).
        int olane;
        asm volatile("v_mov_b32 %0, %1" : "=v"(olane) : "v"(lane));
        // Piece j of a thread lies 256 / KP (q, k) or 256 / VPR (v) rows below its
        // piece 0, in the same column and swizzle phase: a fixed offset each.
#pragma unroll
        for (int j = 0; j < QPT; ++j) {
          constexpr int dr = 256 / KP * K;
          *reinterpret_cast<uint2*>(&bf.Q[sq0 + j * dr]) = make_uint2(rq[j].x, rq[j].y);
          *reinterpret_cast<uint2*>(&bf.Q[sq1 + j * dr]) = make_uint2(rq[j].z, rq[j].w);
          *reinterpret_cast<uint2*>(&bf.Kc[sq0 + j * dr]) = make_uint2(rk[j].x, rk[j].y);
          *reinterpret_cast<uint2*>(&bf.Kc[sq1 + j * dr]) = make_uint2(rk[j].z, rk[j].w);
        }
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
          constexpr int dr = 256 / VPR * VT;
          *reinterpret_cast<u32x4*>(&bf.Vv[sv0 + j * dr]) = rv[j];
        }
        const int nrows_c = min(64, t1 - (t0 + it * 64));
        if (ptid < 64) {
          float a_ = ra, b_ = rb;
          if ((fusion & kFuseGateLogits) && ptid < nrows_c) {  // logits -> alpha, beta
            a_ = sigmoid_fast(a_);
            b_ = sigmoid_fast(b_);
          }
          bf.raw_a[ptid] = a_;
          bf.raw_b[ptid] = b_;
        }
        // Normalisation: per-piece sums of squares of q and k here, while the
        // staging registers still hold them ...
        float ss[2 * QPT];  // q pieces, then k pieces
        if constexpr (NORM) {
#pragma unroll
          for (int j = 0; j < QPT; ++j) {
            ss[j] = sumsq8(rq[j]);
            ss[QPT + j] = sumsq8(rk[j]);
          }
        }
        // The staging registers are free again: fetch the next chunk now, so
        // that its loads are in flight during all of this chunk's work (the
        // work below issues no other vector-memory access that would wait on
        // them).
        if (it + 1 < nchunks) fetch(t0 + (it + 1) * 64);
        if constexpr (NORM) {
          // ... then the row sums over the KP consecutive lanes that hold a
          // row's pieces (256 % KP == 0: a thread's pieces all sit at the same
          // position in their rows), scattered so that each lane pair ends with
          // one of the 2 QPT sums, and 1 / sqrt(sum + eps) with the hardware
          // reciprocal square root (about 1 ulp).
          static_assert(2 * QPT == KP / 2, "one sum per lane pair");
          const float tot = group_sums_scatter<KP>(ss, ptid);
          const int idx = (ptid >> 1) & (2 * QPT - 1), j = idx % QPT;
          if ((ptid & 1) == 0)
            bf.rn[idx / QPT][qk_row(j)] = __builtin_amdgcn_rsqf(tot + kL2NormEps);
        }
        producer_sync(&sm.prod_bar, epoch, lane);

        // decays: every producer wave computes all 64 rows (lane = row)
        const float a = bf.raw_a[lane], be = bf.raw_b[lane];
        // Decays in base 2: G (and lg, Gn) hold cumulative log2(alpha), so
        // every decay factor is one v_exp_f32. alpha is clamped to the
        // smallest normal float so that the hardware log stays finite.
        const float lg = __builtin_amdgcn_logf(fmaxf(a, 1.17549435e-38f));
        const float G = wave_scan_dpp(lg);
        const float rql = NORM ? bf.rn[0][lane] : 1.f, rkl = NORM ? bf.rn[1][lane] : 1.f;
        if (p == 0) {
          const float Gn = __shfl(G, 63, kWave);
          const int gp = gate_pos(lane);
          bf.gl[0][gp] = be;
          bf.gl[1][gp] = be * exp2_fast(G - lg) * rkl;
          bf.gl[2][gp] = exp2_fast(G) * rql;
          bf.gl[3][gp] = exp2_fast(Gn - G) * rkl;
          if constexpr (NORM) bf.gl[4][gp] = dh * exp2_fast(G) * rkl;
          if (lane == 63) bf.eGn = exp2_fast(G);
        }
        // Waves 0 / 1 and 2 / 3 form pairs: the even wave hands its diagonal
        // inverse to the odd one through pair_flag[p / 2].
        // The block / inverse chain is the latency-critical part of the
        // producers' work: while it runs, a producer's instruction issues first
        // when both wavefronts of a SIMD are ready (staging and gates run at
        // normal priority so that the consumers keep their share).
        __builtin_amdgcn_s_setprio(2);
        const int tag = it + 1;
        switch (p) {
          case 0: producer_blocks<0, 3, 3, 0, 3, 1, NORM, SO>(bf, sm.ps[0], sm.ps[0], &sm.pair_flag[0], tag, olane, dh, G, lg, be, rkl); break;
          case 1: producer_blocks<1, 2, 1, 0, 0, 0, NORM, SO>(bf, sm.ps[1], sm.ps[0], &sm.pair_flag[0], tag, olane, dh, G, lg, be, rkl); break;
          case 2: producer_blocks<2, 3, 2, 0, 2, 1, NORM, SO>(bf, sm.ps[2], sm.ps[2], &sm.pair_flag[1], tag, olane, dh, G, lg, be, rkl); break;
          default: producer_blocks<3, 2, 3, 2, 0, 0, NORM, SO>(bf, sm.ps[3], sm.ps[2], &sm.pair_flag[1], tag, olane, dh, G, lg, be, rkl); break;
        }
        __builtin_amdgcn_s_setprio(0);
      }
      __syncthreads();
    }
  } else {
    // ======================= consumers: run chunk it-1 in iteration it =======================
    // Group 1 of a paired pass: the identity-start, zero-v run over K state rows.
    const bool grp1 = PAIR && wave >= 8;
    const int cw = PAIR ? (wave & 3) : wave;  // consumer index within the group
    const int vloc = cw * 16 + l16;
    const int vcol = vt * VT + vloc;
    // Byte offsets of this lane's four output rows (4 g + i) inside a 16-row
    // block, channel vcol; H * V elements separate consecutive tokens.
    const int hv = H * V;
    int ovoff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) ovoff[i] = ((4 * g + i) * hv + vcol) * static_cast<int>(sizeof(OutT));
    f32x4 hs[K / 16];
    const int64_t srow = ((static_cast<int64_t>(n) * H + h) * V + vcol) * K;  // (V == K when paired)
#pragma unroll
    for (int kb = 0; kb < K / 16; ++kb) {
      hs[kb] = s0 && !grp1 ? *reinterpret_cast<const f32x4*>(s0 + srow + 16 * kb + 4 * g) : f32x4{0.f, 0.f, 0.f, 0.f};
      if ((fusion & kModeIdentityInit) || grp1) {
#pragma unroll
        for (int i = 0; i < 4; ++i) hs[kb][i] = (16 * kb + 4 * g + i == vcol) ? 1.f : 0.f;
      }
    }

    for (int it = 0; it <= nchunks; ++it) {
      if (it > 0) {
        const int c = it - 1;
        const ChunkBuf<K, VT>& bf = sm.buf[c & 1];
        const int c0 = t0 + c * 64;
        const int nrows = min(64, t1 - c0);
        const int64_t obase = ((static_cast<int64_t>(b) * T + c0) * H + h) * V;  // row c0, head h
        if (hck) {  // keep the chunk's incoming state (for the backward)
          float* dst = hck + ((chunk_slot(cu_seqlens != nullptr, t0, n, c, T) * H + h) * V + vcol) * K + 4 * g;
#pragma unroll
          for (int kb = 0; kb < K / 16; ++kb) *reinterpret_cast<f32x4*>(dst + 16 * kb) = hs[kb];
        }

        // The body is software-pipelined by hand: every stage issues the LDS
        // reads of the next one before its own matrix products, and
        // scheduling barriers keep that order, so the products rarely wait on
        // LDS latency.
        constexpr int NS = K / 32;  // 32-wide reduction steps over the key dimension
        auto kfrag = [&](int r4, int s_) { return lds8(&bf.Kc[qk_off<K>(16 * r4 + l16, 32 * s_ + 8 * g)]); };
        auto qfrag = [&](int r4, int s_) { return lds8(&bf.Q[qk_off<K>(16 * r4 + l16, 32 * s_ + 8 * g)]); };

        bf16x8 hbh[NS], hbl[NS];
#pragma unroll
        for (int s_ = 0; s_ < NS; ++s_) split_pair(hs[2 * s_], hs[2 * s_ + 1], hbh[s_], hbl[s_]);

        // ---- stage A: K h and Q h, in steps of two reduction slices of one row block
        constexpr int NSTEP = 4 * NS / 2;
        bf16x8 fk[2], fq[2];
        fk[0] = kfrag(0, 0);
        fk[1] = kfrag(0, 1);
        if constexpr (!SO) {
          fq[0] = qfrag(0, 0);
          fq[1] = qfrag(0, 1);
        }
        f32x4 KH[4], QH[4];
#pragma unroll
        for (int j = 0; j < NSTEP; ++j) {
          const int r4 = j / (NS / 2), s0 = 2 * (j % (NS / 2));
          bf16x8 nk[2], nq[2];
          if (j + 1 < NSTEP) {
            const int r4n = (j + 1) / (NS / 2), s0n = 2 * ((j + 1) % (NS / 2));
            nk[0] = kfrag(r4n, s0n);
            nk[1] = kfrag(r4n, s0n + 1);
            if constexpr (!SO) {
              nq[0] = qfrag(r4n, s0n);
              nq[1] = qfrag(r4n, s0n + 1);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
          if (s0 == 0) {
            KH[r4] = f32x4{0.f, 0.f, 0.f, 0.f};
            QH[r4] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            KH[r4] = mfma16x16x32(fk[u], hbh[s0 + u], KH[r4]);
            KH[r4] = mfma16x16x32(fk[u], hbl[s0 + u], KH[r4]);
            if constexpr (!SO) {
              QH[r4] = mfma16x16x32(fq[u], hbh[s0 + u], QH[r4]);
              QH[r4] = mfma16x16x32(fq[u], hbl[s0 + u], QH[r4]);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
          if (j + 1 < NSTEP) {
            fk[0] = nk[0];
            fk[1] = nk[1];
            if constexpr (!SO) {
              fq[0] = nq[0];
              fq[1] = nq[1];
            }
          }
        }

        // ---- stage B: R, then Ubar_top = T1 R_top (T1 read before R is formed)
        bf16x8 t1h[2], t1l[2];
#pragma unroll
        for (int r4 = 0; r4 < 2; ++r4) {
          t1h[r4] = lds8(&bf.Th[tp_off(16 * r4 + l16, 8 * g)]);
          t1l[r4] = lds8(&bf.Tl[tp_off(16 * r4 + l16, 8 * g)]);
        }
        f32x4 R[4];
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const f32x4 bt = lds_f4(&bf.gl[0][16 * g + 4 * r4]);
          const f32x4 bx = lds_f4(&bf.gl[1][16 * g + 4 * r4]);
          const f32x4 vv = grp1 ? f32x4{0.f, 0.f, 0.f, 0.f} : v_frag<VT>(bf.Vv, r4, cw * 16, g, l16);
#pragma unroll
          for (int i = 0; i < 4; ++i) R[r4][i] = bt[i] * vv[i] - bx[i] * KH[r4][i];
        }
        // A21 and T2 for stage C
        bf16x8 a2h[2], a2l[2], t2h[2], t2l[2];
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const int row = 32 + 16 * r + l16;
          a2h[r] = lds8(&bf.Th[tp_off(row, 8 * g)]);
          a2l[r] = lds8(&bf.Tl[tp_off(row, 8 * g)]);
          t2h[r] = lds8(&bf.Th[tp_off(row, 32 + 8 * g)]);
          t2l[r] = lds8(&bf.Tl[tp_off(row, 32 + 8 * g)]);
        }
        __builtin_amdgcn_sched_barrier(0);
        bf16x8 rbh, rbl;
        split_pair(R[0], R[1], rbh, rbl);
        f32x4 U[4];
#pragma unroll
        for (int r4 = 0; r4 < 2; ++r4) U[r4] = mma3(t1h[r4], t1l[r4], rbh, rbl, f32x4{0.f, 0.f, 0.f, 0.f});
        bf16x8 ubh0, ubl0;
        split_pair(U[0], U[1], ubh0, ubl0);

        // ---- stage C: Y = R_bot - A21 Ubar_top ; Ubar_bot = T2 Y (P rows 0-31 read meanwhile)
        bf16x8 p0h[2], p0l[2];
        if constexpr (!SO) {
#pragma unroll
          for (int r4 = 0; r4 < 2; ++r4) {
            p0h[r4] = lds8(&bf.Ph[tp_off(16 * r4 + l16, 8 * g)]);
            p0l[r4] = lds8(&bf.Pl[tp_off(16 * r4 + l16, 8 * g)]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        f32x4 Y[2];
#pragma unroll
        for (int r = 0; r < 2; ++r) Y[r] = mma3(a2h[r], a2l[r], ubh0, ubl0, R[2 + r]);
        bf16x8 ybh, ybl;
        split_pair(Y[0], Y[1], ybh, ybl);
        // P rows 32-63 for stage D
        bf16x8 p1h[2][2], p1l[2][2];
        if constexpr (!SO) {
#pragma unroll
          for (int r = 0; r < 2; ++r) {
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
              p1h[r][hf] = lds8(&bf.Ph[tp_off(32 + 16 * r + l16, 32 * hf + 8 * g)]);
              p1l[r][hf] = lds8(&bf.Pl[tp_off(32 + 16 * r + l16, 32 * hf + 8 * g)]);
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int r = 0; r < 2; ++r) U[2 + r] = mma3(t2h[r], t2l[r], ybh, ybl, f32x4{0.f, 0.f, 0.f, 0.f});
        bf16x8 ubh1, ubl1;
        split_pair(U[2], U[3], ubh1, ubl1);

        // ---- stage D: O = e^G (Q h - d K h) + P Ubar, stored straight from the
        // accumulator layout (K^T fragments of the first key block read meanwhile)
        bf16x8 kt0[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) kt0[s2] = kt_frag<K>(bf.Kc, 0, s2, g, l16);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (!SO) {  // a state-only pass forms no output
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const f32x4 eg = lds_f4(&bf.gl[2][16 * g + 4 * r4]);
          f32x4 acc;
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[i] = eg[i] * (QH[r4][i] - dh * KH[r4][i]);
          if constexpr (NORM) {  // e^G r_q (Q h) - d e^G r_k (K h)
            const f32x4 egk = lds_f4(&bf.gl[4][16 * g + 4 * r4]);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = eg[i] * QH[r4][i] - egk[i] * KH[r4][i];
          }
          if (r4 < 2) {
            acc = mma3(p0h[r4], p0l[r4], ubh0, ubl0, acc);
          } else {
            acc = mma3(p1h[r4 - 2][0], p1l[r4 - 2][0], ubh0, ubl0, acc);
            acc = mma3(p1h[r4 - 2][1], p1l[r4 - 2][1], ubh1, ubl1, acc);
          }
          // Stored straight from the accumulator layout: this lane holds rows
          // 16 r4 + 4 g + i of its wavefront's channel l16; the 16 lanes of a
          // row write 32 contiguous bytes and the four consumer waves complete
          // the workgroup's segment of that row. The buffer resource covers
          // only the rows of this 16-row block that lie inside the sequence,
          // so stores to rows past its end are dropped by the range check.
          const int vrows = min(max(nrows - 16 * r4, 0), 16);
          const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
              uniform_ptr(o + obase + static_cast<int64_t>(16 * r4) * hv), static_cast<short>(0),
              __builtin_amdgcn_readfirstlane((fusion & kModeNoOutput) ? 0 : vrows * hv * static_cast<int>(sizeof(OutT))),
              kBufferWord3);
          if constexpr (sizeof(OutT) == 2) {
            const unsigned p01 = __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2){acc[0], acc[1]}, bf16x2));
            const unsigned p23 = __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2){acc[2], acc[3]}, bf16x2));
            __builtin_amdgcn_raw_buffer_store_b16(static_cast<u16>(p01), orsrc, ovoff[0], 0, 0);
            __builtin_amdgcn_raw_buffer_store_b16(static_cast<u16>(p01 >> 16), orsrc, ovoff[1], 0, 0);
            __builtin_amdgcn_raw_buffer_store_b16(static_cast<u16>(p23), orsrc, ovoff[2], 0, 0);
            __builtin_amdgcn_raw_buffer_store_b16(static_cast<u16>(p23 >> 16), orsrc, ovoff[3], 0, 0);
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i]), orsrc, ovoff[i], 0, 0);
          }
        }
        }

        // ---- stage E: h' = e^Gn h + K^T diag(e^(Gn - G)) Ubar, K^T fragments
        // double-buffered by key block
        bf16x8 ush[2], usl[2];
        {
          f32x4 Us[4];
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const f32x4 en = lds_f4(&bf.gl[3][16 * g + 4 * r4]);
#pragma unroll
            for (int i = 0; i < 4; ++i) Us[r4][i] = U[r4][i] * en[i];
          }
          split_pair(Us[0], Us[1], ush[0], usl[0]);
          split_pair(Us[2], Us[3], ush[1], usl[1]);
        }
        const float eGn = bf.eGn;
        bf16x8 ktc[2] = {kt0[0], kt0[1]};
#pragma unroll
        for (int kb = 0; kb < K / 16; ++kb) {
          bf16x8 ktn[2];
          if (kb + 1 < K / 16) {
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) ktn[s2] = kt_frag<K>(bf.Kc, kb + 1, s2, g, l16);
          }
          __builtin_amdgcn_sched_barrier(0);
          hs[kb] *= eGn;
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            hs[kb] = mfma16x16x32(ktc[s2], ush[s2], hs[kb]);
            hs[kb] = mfma16x16x32(ktc[s2], usl[s2], hs[kb]);
          }
          __builtin_amdgcn_sched_barrier(0);
          if (kb + 1 < K / 16) {
            ktc[0] = ktn[0];
            ktc[1] = ktn[1];
          }
        }
      }
      __syncthreads();
    }
    float* const dst = grp1 ? sf2 : sf;
    if (dst) {
#pragma unroll
      for (int kb = 0; kb < K / 16; ++kb) *reinterpret_cast<f32x4*>(dst + srow + 16 * kb + 4 * g) = hs[kb];
    }
  }
}

template <int K, int V, int VT, typename OutT, bool NORM, bool SO>
__global__ __launch_bounds__(512) void chunk_fwd_bf16_kernel(
    const u16* __restrict__ q, const u16* __restrict__ k, const u16* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta, const float* __restrict__ d,
    const float* s0, const int32_t* __restrict__ cu_seqlens,
    const int32_t* __restrict__ order, int T, int H, int Hk, int N, OutT* o,
    float* sf, unsigned fusion, float* hck) {
  chunk_fwd_bf16_body<K, V, VT, OutT, NORM, SO, false>(q, k, v, alpha, beta, d, s0, cu_seqlens, order, T, H, Hk, N,
                                                        o, sf, fusion, hck, nullptr);
}

// State-only pass of the segment-parallel forward that forms both the
// segment-end states (sf) and the segment maps (sf2) in one launch.
template <int K, int VT, bool NORM>
__global__ __launch_bounds__(768) void chunk_fwd_bf16_pair_kernel(
    const u16* __restrict__ q, const u16* __restrict__ k, const u16* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta, const float* __restrict__ d,
    const int32_t* __restrict__ cu_seqlens, int T, int H, int Hk, int N, float* sf, unsigned fusion,
    float* sf2) {
  chunk_fwd_bf16_body<K, K, VT, u16, NORM, true, true>(q, k, v, alpha, beta, d, nullptr, cu_seqlens, nullptr, T, H,
                                                       Hk, N, nullptr, sf, fusion, nullptr, sf2);
}

template <int K, int V, typename OutT, bool NORM, bool SO>
static hipError_t launch_bf16_t(const FwdArgs& a, hipStream_t st) {
  constexpr int VT = 64, NVT = V / VT;
  const int units = a.N * a.H;
  chunk_fwd_bf16_kernel<K, V, VT, OutT, NORM, SO><<<xcd_grid(units, NVT), 512, 0, st>>>(
      static_cast<const u16*>(a.q), static_cast<const u16*>(a.k), static_cast<const u16*>(a.v), a.alpha,
      a.beta, a.d, a.s0, a.cu_seqlens, a.order, a.T, a.H, a.Hk, a.N, static_cast<OutT*>(a.o), a.sf, a.fusion, a.hck);
  return hipGetLastError();
}

template <int K, bool NORM>
static hipError_t launch_pair_t(const FwdArgs& a, float* sf2, hipStream_t st) {
  constexpr int VT = 64, NVT = K / VT;
  chunk_fwd_bf16_pair_kernel<K, VT, NORM><<<xcd_grid(a.N * a.H, NVT), 768, 0, st>>>(
      static_cast<const u16*>(a.q), static_cast<const u16*>(a.k), static_cast<const u16*>(a.v), a.alpha, a.beta,
      a.d, a.cu_seqlens, a.T, a.H, a.Hk, a.N, a.sf, a.fusion, sf2);
  return hipGetLastError();
}

template <int K, int V, bool NORM>
static hipError_t launch_bf16_n(const FwdArgs& a, hipStream_t st) {
  // a pass without output (state maps, checkpoints) runs the state-only instantiation
  if (a.fusion & kModeNoOutput) return launch_bf16_t<K, V, u16, NORM, true>(a, st);
  if (a.out_dtype == COMBA_BF16) return launch_bf16_t<K, V, u16, NORM, false>(a, st);
  return launch_bf16_t<K, V, float, NORM, false>(a, st);
}

template <int K, int V>
static hipError_t launch_bf16_kv(const FwdArgs& a, hipStream_t st) {
  if (a.fusion & kFuseQkL2Norm) return launch_bf16_n<K, V, true>(a, st);
  return launch_bf16_n<K, V, false>(a, st);
}

hipError_t launch_chunk_bf16_pair(const FwdArgs& a, float* sf2, hipStream_t st) {
  if (a.K != a.V || (a.K != 64 && a.K != 128)) return hipErrorInvalidValue;
  const bool norm = (a.fusion & kFuseQkL2Norm) != 0;
  if (a.K == 128) return norm ? launch_pair_t<128, true>(a, sf2, st) : launch_pair_t<128, false>(a, sf2, st);
  return norm ? launch_pair_t<64, true>(a, sf2, st) : launch_pair_t<64, false>(a, sf2, st);
}

hipError_t launch_chunk_bf16(const FwdArgs& a, hipStream_t st) {
  if (a.K == 128 && a.V == 128) return launch_bf16_kv<128, 128>(a, st);
  if (a.K == 128 && a.V == 64) return launch_bf16_kv<128, 64>(a, st);
  if (a.K == 64 && a.V == 128) return launch_bf16_kv<64, 128>(a, st);
  return launch_bf16_kv<64, 64>(a, st);
}

}  // namespace comba
