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
//   dlog(alpha_t) = -dGx_t + sum_{s >= t} (dG_s + dGx_s),   dalpha_t = dlog(alpha_t) / alpha_t,
// evaluated in the equivalent form without cancelling terms (grad_scalars), so
// that alpha_t near zero keeps dalpha_t accurate.
// An fp64 prototype of exactly these formulas matches the reverse-mode oracle
// of the token recurrence to 1e-15.
//
// Launches after a forward pass that stores every chunk's incoming state (the
// chunk kernels' checkpoint option):
//   chunk_bwd_prep_kernel  one workgroup per (chunk, head), all chunks at once:
//                          Tinv, P (their 16 x 16 blocks on or below the
//                          diagonal), k_t.k_s (fp32 inputs) and the decay
//                          gates of the chunk, stored;
//   chunk_bwd_dh_kernel    reverse scan over chunks, one workgroup per
//   (_bf16_kernel)         (sequence, head, 32 (fp32) or 64 (bf16) value
//                          channels), next chunk prefetched into registers:
//                          stores each chunk's outgoing-state gradient dh,
//                          writes dS_0;
//   chunk_bwd_grad_kernel  one workgroup per (chunk, head): every per-token
//                          gradient and a partial of dd;
//   dd_reduce_kernel       dd per head, summed over chunks in a fixed order.
// For fp32 inputs the scan and the gradient kernel form their products on the
// fp32 matrix cores (16 x 16 x 4 tiles, exact fp32 operands read from
// row-major LDS buffers; a transposed operand only swaps the fragment's
// indices). For bf16 inputs both run on the bf16 matrix cores with every fp32
// operand split into hi + lo bf16, and the prep kernel forms its scores on
// them; for fp32 inputs the prep kernel's scores use the vector units. The
// prep kernel's inverse takes its diagonal blocks by substitution on the
// vector units and its off-diagonal blocks on the fp32 matrix cores.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstddef>
#include <type_traits>

#include "bf16_tiles.h"
#include "chunk_common.h"
#include "launch.h"

namespace comba {

namespace {

constexpr int kDhVT = 32;  // value channels per workgroup of the reverse scan
// Stored gates of a chunk: the first seven rows of ChunkGates (G, Gx, beta,
// bEGx, EG, EGnG, alpha with 1 on padded rows), read back as one block.
constexpr int kGateWords = 7 * 64;
static_assert(offsetof(ChunkGates, raw_a) == 6 * 64 * sizeof(float), "gate rows in order");
constexpr int kLdT = 68;   // row stride of 64-wide fp32 tiles (16-byte aligned rows)

template <typename InT>
__device__ __forceinline__ float ld(const InT* p, int64_t i) {
  return Elem<InT>::load(p, i);
}

__device__ __forceinline__ f32x4 ld4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ void st4(float* p, f32x4 x) { *reinterpret_cast<f32x4*>(p) = x; }
__device__ __forceinline__ float hsum(f32x4 x) { return (x[0] + x[1]) + (x[2] + x[3]); }

// Tinv and P are lower triangular: the prep kernel stores only their 16x16
// blocks on or below the diagonal (the rest of the 64x64 buffers is never
// written), and the readers load those blocks and zero the others.
__device__ __forceinline__ bool tri_block_live(int row, int col) { return (col >> 4) <= (row >> 4); }
__device__ __forceinline__ f32x4 ld4_lower(const float* m, int row, int c4) {
  return tri_block_live(row, c4) ? ld4(m + row * 64 + c4) : f32x4{0.f, 0.f, 0.f, 0.f};
}

// ---- row loads through buffer resources ---------------------------------------------------
// A chunk's rows are read with unconditional 16- or 8-byte buffer loads whose
// resource ends after the chunk's last valid row: loads past it return zeros,
// the padding the chunk algebra needs. The loaded words stay raw in registers
// until they are written to LDS, so a load issued one chunk (or tile) ahead is
// waited for only there.

template <typename T>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const T* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(const_cast<T*>(base)), static_cast<short>(0),
                                           __builtin_amdgcn_readfirstlane(static_cast<int>(bytes)), kBufferWord3);
}

// Four consecutive elements: 8 bytes of bf16 or 16 bytes of fp32.
template <typename InT>
struct Piece4 {
  typedef typename std::conditional<sizeof(InT) == 2, u32x2, u32x4>::type type;
};

template <typename InT>
__device__ __forceinline__ typename Piece4<InT>::type load4(__amdgpu_buffer_rsrc_t r, int byte_off) {
  if constexpr (sizeof(InT) == 2) return __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, 0);
  else return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
}

__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
}

// The four floats of a Piece4. Words go through scalar copies: a bit cast of
// a vector subscript reads element 0 for every index with this compiler.
__device__ __forceinline__ f32x4 unpack4(const u32x2& w) {
  const unsigned e0 = w.x, e1 = w.y;
  return f32x4{__uint_as_float(e0 << 16), __uint_as_float(e0 & 0xffff0000u), __uint_as_float(e1 << 16),
               __uint_as_float(e1 & 0xffff0000u)};
}
__device__ __forceinline__ f32x4 unpack4(const u32x4& w) {
  const unsigned e0 = w.x, e1 = w.y, e2 = w.z, e3 = w.w;
  return f32x4{__uint_as_float(e0), __uint_as_float(e1), __uint_as_float(e2), __uint_as_float(e3)};
}

__device__ __forceinline__ float to_f32(u16 b) { return bf16_bits_to_float(b); }
__device__ __forceinline__ float to_f32(float x) { return x; }

// The floats of a 16-byte piece: eight bf16 (lo = elements 0-3, hi = 4-7) or
// four fp32 (lo only).
template <typename InT>
__device__ __forceinline__ void unpack16(const u32x4& w, f32x4& lo, f32x4& hi) {
  if constexpr (sizeof(InT) == 2) {
    lo = unpack4(u32x2{w.x, w.y});
    hi = unpack4(u32x2{w.z, w.w});
  } else {
    lo = unpack4(w);
    hi = lo;
  }
}

// q and k rows of a chunk, one thread's share: QP 16-byte pieces of each, the
// piece p = tid + j NT covering row p / (K / EB), columns EB (p % (K / EB)) ..
template <int K, int NT, typename InT>
struct RowPieces {
  static constexpr int EB = 16 / static_cast<int>(sizeof(InT));  // elements per piece
  static constexpr int QP = 64 * K / EB / NT;
  static_assert(QP >= 1 && QP * EB * NT == 64 * K, "whole pieces per thread");
  u32x4 q[QP], k[QP];

  __device__ __forceinline__ void load(const InT* qg, const InT* kg, int64_t tok0, int H, int nrows, int tid) {
    const int64_t bytes = static_cast<int64_t>(nrows) * H * K * sizeof(InT);
    const __amdgpu_buffer_rsrc_t qr = rows_rsrc(qg + tok0 * K, bytes), kr = rows_rsrc(kg + tok0 * K, bytes);
#pragma unroll
    for (int j = 0; j < QP; ++j) {
      const int p = tid + j * NT, row = p / (K / EB), col = EB * (p % (K / EB));
      const int off = (row * H * K + col) * static_cast<int>(sizeof(InT));
      q[j] = load16(qr, off);
      k[j] = load16(kr, off);
    }
  }
  // bf16 q and k tiles of K per row (swz<K>), keys of each 32-block in perm32 order
  __device__ __forceinline__ void store_bf16(u16* Qc, u16* Kc, int tid) const {
    static_assert(EB == 8, "bf16 pieces");
#pragma unroll
    for (int j = 0; j < QP; ++j) {
      const int p = tid + j * NT, row = p / (K / EB), col = EB * (p % (K / EB));
      const int p0 = swz<K>(row, perm_col(col)), p1 = swz<K>(row, perm_col(col + 4));
      *reinterpret_cast<u32x2*>(Qc + p0) = u32x2{q[j].x, q[j].y};
      *reinterpret_cast<u32x2*>(Qc + p1) = u32x2{q[j].z, q[j].w};
      *reinterpret_cast<u32x2*>(Kc + p0) = u32x2{k[j].x, k[j].y};
      *reinterpret_cast<u32x2*>(Kc + p1) = u32x2{k[j].z, k[j].w};
    }
  }
  // Kc[row][c] = k, Qt[row][c] = q - d k (fp32 rows of stride LD)
  template <int LD>
  __device__ __forceinline__ void store(float* Qt, float* Kc, float dh, int tid) const {
#pragma unroll
    for (int j = 0; j < QP; ++j) {
      const int p = tid + j * NT, row = p / (K / EB), col = EB * (p % (K / EB));
      f32x4 q0, q1, k0, k1;
      unpack16<InT>(q[j], q0, q1);
      unpack16<InT>(k[j], k0, k1);
      st4(Kc + row * LD + col, k0);
      st4(Qt + row * LD + col, q0 - dh * k0);
      if constexpr (EB == 8) {
        st4(Kc + row * LD + col + 4, k1);
        st4(Qt + row * LD + col + 4, q1 - dh * k1);
      }
    }
  }
};

// The chunk of a slot (see chunk_slot). Returns false for a slot between packed sequences.
__device__ __forceinline__ bool slot_chunk(const int32_t* cu_seqlens, int64_t slot, int T, int N, int& n, int& c,
                                           int& b, int& t0, int& t1) {
  if (cu_seqlens) {
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
  return c >= 0 && t0 + 64 * c < t1;
}

__device__ __forceinline__ void stage_gates(ChunkGates& gt, const float* alpha, const float* beta, int64_t tok0,
                                            int H, int nrows, int tid) {
  if (tid < 64) {
    gt.raw_a[tid] = tid < nrows ? alpha[tok0 + static_cast<int64_t>(tid) * H] : 1.f;
    gt.raw_b[tid] = tid < nrows ? beta[tok0 + static_cast<int64_t>(tid) * H] : 0.f;
  }
}

// D += A (16 x 4) B (4 x 16) in fp32 on the matrix cores. Lane l supplies
// A[l % 16][l / 16] and B[l / 16][l % 16]; D holds rows 4 (l / 16) + i of
// column (l % 16).
__device__ __forceinline__ f32x4 mma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Tinv = (I + A)^-1 for the prep kernel: the diagonal 16x16 blocks by
// column-wise forward substitution as in unit_lower_inverse64, the
// off-diagonal levels on the fp32 matrix cores (exact fp32 products). Block
// (i, j) of level L = i - j goes to wavefront j (3, 2, 1 blocks):
//   Y = sum_{j <= m < i} A_im T_mj  (4 L products over four columns of A),
//   T_ij = -T_ii Y,
// where Y passes from the accumulator layout to the operand layout through the
// wavefront's own 256 floats of Ys (one wavefront's LDS accesses complete in
// order). Called by all 256 threads; ends with a barrier.
__device__ __forceinline__ void unit_lower_inverse64_mfma(const float* Am, float* Tm, float* Ys, int tid) {
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
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, c = lane & 15, g = lane >> 4;
#pragma unroll
  for (int L = 1; L <= 3; ++L) {
    if (wave < 4 - L) {
      const int j = wave, i = j + L;
      f32x4 y{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int mm = 0; mm < L; ++mm) {
        const int m = j + mm;
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4)
          y = mma4(Am[(16 * i + c) * kLdF + 16 * m + 4 * s4 + g], Tm[(16 * m + 4 * s4 + g) * kLdF + 16 * j + c], y);
      }
      float* ys = Ys + 256 * wave;
#pragma unroll
      for (int r = 0; r < 4; ++r) ys[(4 * g + r) * 16 + c] = y[r];
      __builtin_amdgcn_wave_barrier();
      f32x4 t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4)
        t = mma4(Tm[(16 * i + c) * kLdF + 16 * i + 4 * s4 + g], ys[(4 * s4 + g) * 16 + c], t);
#pragma unroll
      for (int r = 0; r < 4; ++r) Tm[(16 * i + 4 * g + r) * kLdF + 16 * j + c] = -t[r];
    }
    __syncthreads();
  }
}

// ---- prep: Tinv, P and k_t.k_s of every chunk -------------------------------------------

template <int K>
struct alignas(16) SmemPrepValu {
  float QtT[K][kLdT];  // q~ transposed: [key channel][token]
  float KT[K][kLdT];
  float Am[64 * kLdF];
  float Tm[64 * kLdF];
  float Ys[768];
  ChunkGates gt;
};

template <int K>
struct alignas(16) SmemPrepMfma {
  union {
    struct {
      float Am[64 * kLdF];
      float Tm[64 * kLdF];
    };
    struct {  // q and k rows for the score products, read before A is formed
      u16 Qc[64 * K];
      u16 Kc[64 * K];
    };
  };
  float Ys[768];
  ChunkGates gt;
};

// A (to LDS, for the inverse), P and, for the fp32 gradient kernel, k_t.k_s
// (to the per-chunk buffers) of one entry. Hardware exp (about 2 ulp).
template <bool kStoreKK>
__device__ __forceinline__ void prep_entry(const ChunkGates& gt, int t, int s, float kk, float qtk, float* Am,
                                           float* Pg, float* KKg) {
  Am[t * kLdF + s] = s < t ? gt.beta[t] * decay_Gx(gt, t, s) * kk : 0.f;
  if (tri_block_live(t, s)) Pg[t * 64 + s] = s <= t ? qtk * decay_G(gt, t, s) : 0.f;
  if constexpr (kStoreKK) KKg[t * 64 + s] = kk;
}

// Scores of NB of the ten 16x16 blocks (R_b, C_b), C_b <= R_b, of a chunk for
// bf16 q and k: k_t.k_s and q_t.k_s on the matrix cores. Lane l supplies row
// (l % 16) of a block and 8 keys of each 32-block (the same keys for both
// operands) from the q / k tiles; the accumulator holds rows 4 (l / 16) + i of
// column (l % 16).
template <int NB, int R0, int C0, int R1, int C1, int R2, int C2, int K>
__device__ __forceinline__ void prep_score_blocks(const u16* Qc, const u16* Kc, int lane, f32x4* akk, f32x4* aqk) {
  constexpr int Rb[3] = {R0, R1, R2}, Cb[3] = {C0, C1, C2};
  const int l16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int b = 0; b < NB; ++b) akk[b] = aqk[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < K / 32; ++j) {
    const int kofs = 32 * j + 8 * g;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const bf16x8 ak = lds8(&Kc[swz<K>(16 * Rb[b] + l16, kofs)]), aq = lds8(&Qc[swz<K>(16 * Rb[b] + l16, kofs)]);
      const bf16x8 bk = lds8(&Kc[swz<K>(16 * Cb[b] + l16, kofs)]);
      akk[b] = mfma16x16x32(ak, bk, akk[b]);
      aqk[b] = mfma16x16x32(aq, bk, aqk[b]);
    }
  }
}

// A (to LDS) and P (to the chunk's buffer) of the same blocks. Diagonal blocks
// take each decay directly; in a block below the diagonal every s <= r < t
// for r = 16 C + 15, its last column, so the decays factor into a row part
// e^(G_t - G_r) (or e^(Gx_t - G_r)) and a column part e^(G_r - G_s), each at
// most 1: nine exponentials per lane instead of 32.
template <int NB, int R0, int C0, int R1, int C1, int R2, int C2>
__device__ __forceinline__ void prep_score_entries(const ChunkGates& gt, int lane, float dh, const f32x4* akk,
                                                   const f32x4* aqk, float* Am, float* Pg) {
  constexpr int Rb[3] = {R0, R1, R2}, Cb[3] = {C0, C1, C2};
  const int l16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int s_ = 16 * Cb[b] + l16;
    if (Rb[b] == Cb[b]) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        prep_entry<false>(gt, 16 * Rb[b] + 4 * g + i, s_, akk[b][i], aqk[b][i] - dh * akk[b][i], Am, Pg, nullptr);
    } else {
      const int r = 16 * Cb[b] + 15;
      const float cs = expf(static_cast<float>(gt.Gd[r] - gt.Gd[s_]));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * Rb[b] + 4 * g + i;
        const float eg = expf(static_cast<float>(gt.Gd[t] - gt.Gd[r]));
        const float ex = expf(static_cast<float>(gt.Gxd[t] - gt.Gd[r]));
        Am[t * kLdF + s_] = gt.beta[t] * (ex * cs) * akk[b][i];
        Pg[t * 64 + s_] = (aqk[b][i] - dh * akk[b][i]) * (eg * cs);
      }
    }
  }
}

template <int K, typename InT>
__global__ __launch_bounds__(256, sizeof(InT) == 2 ? 4 : 1) void chunk_bwd_prep_kernel(
    const InT* __restrict__ q, const InT* __restrict__ k, const float* __restrict__ alpha,
    const float* __restrict__ beta, const float* __restrict__ d, const int32_t* __restrict__ cu_seqlens, int T,
    int H, int N, int64_t nslots, float* __restrict__ Tg, float* __restrict__ Pg, float* __restrict__ KKg,
    float* __restrict__ Gg) {
  constexpr int NT = 256;
  constexpr bool kMfma = sizeof(InT) == 2;  // bf16 q / k: exact matrix-core operands
  using Smem = typename std::conditional<kMfma, SmemPrepMfma<K>, SmemPrepValu<K>>::type;
  __shared__ Smem sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = blockIdx.x % H;
  const int64_t slot = blockIdx.x / H;
  if (slot >= nslots) return;
  int n, c, b, t0, t1;
  if (!slot_chunk(cu_seqlens, slot, T, N, n, c, b, t0, t1)) return;
  const int c0 = t0 + 64 * c, nrows = min(64, t1 - c0);
  const int64_t tok0 = (static_cast<int64_t>(b) * T + c0) * H + h;
  const float dh = d[h];
  const int64_t mb = (slot * H + h) * 64 * 64;
  if constexpr (kMfma) {
    // q and k rows in flight while the gates are staged and formed
    RowPieces<K, NT, u16> rqk;
    rqk.load(reinterpret_cast<const u16*>(q), reinterpret_cast<const u16*>(k), tok0, H, nrows, tid);
    stage_gates(sm.gt, alpha, beta, tok0, H, nrows, tid);
    rqk.store_bf16(sm.Qc, sm.Kc, tid);
  } else {
    for (int e = tid; e < 64 * K; e += NT) {
      const int row = e / K, cc = e % K;
      float kv = 0.f, qv = 0.f;
      if (row < nrows) {
        const int64_t off = (tok0 + static_cast<int64_t>(row) * H) * K + cc;
        kv = ld(k, off);
        qv = ld(q, off);
      }
      sm.KT[cc][row] = kv;
      sm.QtT[cc][row] = qv - dh * kv;
    }
    stage_gates(sm.gt, alpha, beta, tok0, H, nrows, tid);
  }
  __syncthreads();
  if (wave == 0) chunk_gates(sm.gt, lane, nrows);
  __syncthreads();
  // the gates, for the scan and the gradient kernel
  if (tid < kGateWords / 4) st4(Gg + (slot * H + h) * kGateWords + 4 * tid, ld4(&sm.gt.G[0] + 4 * tid));
  if constexpr (kMfma) {
    // The ten blocks on or below the diagonal in balanced sets, one diagonal
    // block per wavefront (the blocks above it are zero and never formed).
    f32x4 akk[3], aqk[3];
    switch (wave) {
      case 0: prep_score_blocks<3, 0, 0, 3, 0, 2, 1, K>(sm.Qc, sm.Kc, lane, akk, aqk); break;
      case 1: prep_score_blocks<3, 1, 1, 1, 0, 3, 2, K>(sm.Qc, sm.Kc, lane, akk, aqk); break;
      case 2: prep_score_blocks<2, 2, 2, 2, 0, 0, 0, K>(sm.Qc, sm.Kc, lane, akk, aqk); break;
      default: prep_score_blocks<2, 3, 3, 3, 1, 0, 0, K>(sm.Qc, sm.Kc, lane, akk, aqk); break;
    }
    __syncthreads();  // the q / k tiles share A's space
    switch (wave) {
      case 0: prep_score_entries<3, 0, 0, 3, 0, 2, 1>(sm.gt, lane, dh, akk, aqk, sm.Am, Pg + mb); break;
      case 1: prep_score_entries<3, 1, 1, 1, 0, 3, 2>(sm.gt, lane, dh, akk, aqk, sm.Am, Pg + mb); break;
      case 2: prep_score_entries<2, 2, 2, 2, 0, 0, 0>(sm.gt, lane, dh, akk, aqk, sm.Am, Pg + mb); break;
      default: prep_score_entries<2, 3, 3, 3, 1, 0, 0>(sm.gt, lane, dh, akk, aqk, sm.Am, Pg + mb); break;
    }
  } else {
    // 4 x 4 block of (t, s) per thread: k_t.k_s and q~_t.k_s
    const int tb = 4 * (tid >> 4), sb = 4 * (tid & 15);
    f32x4 kk[4], qk[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) kk[i] = qk[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int cc = 0; cc < K; ++cc) {
      const f32x4 kt = ld4(&sm.KT[cc][tb]), ks = ld4(&sm.KT[cc][sb]), qt = ld4(&sm.QtT[cc][tb]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        kk[i] += kt[i] * ks;
        qk[i] += qt[i] * ks;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) prep_entry<true>(sm.gt, tb + i, sb + j, kk[i][j], qk[i][j], sm.Am, Pg + mb, KKg + mb);
  }
  __syncthreads();
  unit_lower_inverse64_mfma(sm.Am, sm.Tm, sm.Ys, tid);
  for (int e = 4 * tid; e < 64 * 64; e += 4 * NT) {  // four entries of a row per thread
    const int t = e >> 6, s_ = e & 63;
    if (tri_block_live(t, s_)) {
      f32x4 x = ld4(&sm.Tm[t * kLdF + s_]);
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = s_ + i <= t ? x[i] : 0.f;
      st4(Tg + mb + e, x);
    }
  }
}

// ---- reverse scan of dh --------------------------------------------------------------------

template <int K>
struct alignas(16) SmemDh {
  float Qt[64][K + 4];
  float Kc[64][K + 4];
  float Tm[64][kLdT];
  float Pm[64][kLdT];
  float dh[K][kDhVT + 4];
  float dO[64][kDhVT + 4];
  float dU[64][kDhVT + 4];  // dUbar
  float dR[64][kDhVT + 4];
  ChunkGates gt;
};

template <int K, int V, typename InT>
__global__ __launch_bounds__(512) void chunk_bwd_dh_kernel(
    const InT* __restrict__ q, const InT* __restrict__ k, const float* __restrict__ d, const InT* __restrict__ dO,
    const int32_t* __restrict__ cu_seqlens, int T, int H, int N, const float* __restrict__ Tg,
    const float* __restrict__ Pg, const float* __restrict__ Gg, const float* __restrict__ dsf,
    float* __restrict__ dhck, float* __restrict__ ds0);

// ---- per-chunk gradients ------------------------------------------------------------------


constexpr int kGrVT = 16;  // value channels per tile of the gradient kernel
constexpr int kLdV = kGrVT + 4;

template <int K>
struct alignas(16) SmemGrad {
  float Qt[64][K + 4];
  float Kc[64][K + 4];
  float Tm[64][kLdT];  // Tinv, then dP (.) M
  float Pm[64][kLdT];  // P, then dP (.) P
  union {
    struct {
      float S[kGrVT][K + 4];   // state tile, [channel][key]
      float dS[kGrVT][K + 4];  // outgoing-state gradient tile
      float dO[64][kLdV];      // [token][channel]
      float R[64][kLdV];
      float U[64][kLdV];       // Ubar
      float dU[64][kLdV];      // dUbar, then dR
    } t;
    struct {
      float W[64][kLdT];  // dA (.) E
      float X[64][kLdT];  // W (.) k_t.k_s
    } p;
  } u;
  ChunkGates gt;
  float vec[12][64];
  float red[16];
};

// Per-token scalars of a chunk, run by one wavefront (lane = row). vec rows:
// 1 sum dR.(v - e^Gx K h), 2 sum (K h).dR, 3 sum (K dh).Ubar, 5 row sums of
// W (.) k_t.k_s, 8 + 9 the two halves of (q~ h).dO, 10 and 11 the rectangle
// sums R_P(t) = sum_{s>=t, r<t} (dP (.) P)[s][r] and R_A(t) = sum_{s>t, r<t}
// (dA (.) A)[s][r]; red[0..7] partial <h, dh>, red[8..15] partial dd.
//
// The gradient of log alpha_t is a reverse cumulative sum of dG + dGx over the
// chunk (see the formulas above), but the row and column sums in it cancel
// wherever both indices are >= t, and the t2 terms against dGn. Written
// without those cancelling parts, every remaining term carries the factor
// alpha_t, so a tiny alpha_t leaves no catastrophic cancellation:
//   dlog_t = sum_{s>=t} e^G_s (q~ h)_s.dO_s + R_P(t) + R_A(t) + e^Gn <h, dh>
//            + sum_{s<t} e^(Gn - G_s) (K dh)_s.Ubar_s - sum_{s>t} b1_s (K h)_s.dR_s
// (exclusive sums formed directly, never as an inclusive sum minus its term).
__device__ __forceinline__ void grad_scalars(const ChunkGates& gt, const float (*vec)[64], const float* red, int lane,
                                             int nrows, int64_t tok0, int H, float* dalpha, float* dbeta,
                                             float* dd_out) {
  const int t = lane;
  float hd = 0.f;
  for (int w = 0; w < 8; ++w) hd += red[w];
  const float x1 = gt.EG[t] * (vec[8][t] + vec[9][t]);
  const float t2 = gt.EGnG[t] * vec[3][t];
  const float x3 = gt.bEGx[t] * vec[2][t];
  // sum_{s>=t} x1, sum_{s>t} x3 and sum_{s<t} t2 by DPP scans; the exclusive
  // sums are the inclusive ones moved by one lane (the end lane reads zero).
  // Every cross-lane read runs in all 64 lanes.
  const float suf1 = wave_suffix_scan_dpp(x1);
  const float suf3 = wave_from_higher(wave_suffix_scan_dpp(x3));
  const float pre2 = wave_from_lower(wave_scan_dpp(t2));
  const float dlog = suf1 + vec[10][t] + vec[11][t] + gt.EG[63] * hd + pre2 - suf3;
  if (t < nrows) {
    const int64_t off = tok0 + static_cast<int64_t>(t) * H;
    dbeta[off] = vec[5][t] + vec[1][t];
    dalpha[off] = dlog / gt.raw_a[t];
  }
  if (t == 0) {
    float s2 = 0.f;
    for (int w = 0; w < 8; ++w) s2 += red[8 + w];
    *dd_out = s2;
  }
}

// Value of the lane D places before this one in its group of four (DPP
// quad_perm [0,0,1,2] or [0,1,0,1]); lanes at the start of the group read
// their own value.
template <int D>
__device__ __forceinline__ float quad_up(float x) {
  constexpr int ctrl = D == 1 ? 0x90 : 0x44;
  static_assert(D == 1 || D == 2, "shift by one or two lanes");
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), ctrl, 0xf, 0xf, false));
}

// The rectangle sums of grad_scalars from two 64 x 64 fp32 products in LDS
// (row stride kLdT): X = dP (.) P and Z = W (.) k_t.k_s, whose rows scaled by
// beta_s give Y = dA (.) A. Two passes over all 512 threads of the workgroup,
// with a workgroup barrier between them:
//   rect_row_prefix: row s of X (threads 0-255) or of Y (256-511) becomes its
//     exclusive prefix sum_{r<t}; four neighbouring lanes take 16 columns each
//     and add the running sums of the lanes before them; the Z lanes also
//     write the plain row sum of Z (vec row 5, for dbeta);
//   rect_column_sums: R_P(t) = sum_{s>=t} X'[s][t], R_A(t) = sum_{s>t} Y'[s][t],
//     four neighbouring lanes per column taking the rows s = 4 m + part.
__device__ __forceinline__ void rect_row_prefix(float (*X)[kLdT], float (*Z)[kLdT], const float* beta,
                                                float (*vec)[64], int tid) {
  const bool isz = tid >= 256;
  const int row = (tid >> 2) & 63, part = tid & 3;
  float* p = (isz ? Z[row] : X[row]) + 16 * part;
  const float b = isz ? beta[row] : 1.f;
  f32x4 x[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) x[j] = ld4(p + 4 * j);
  f32x4 pre[4];
  float acc = 0.f, raw = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pre[j][i] = acc;
      acc += b * x[j][i];
      raw += x[j][i];
    }
  // running sums of the lanes holding the columns before this lane's
  float incl = acc;
  const float u1 = quad_up<1>(incl);
  if (part >= 1) incl += u1;
  const float u2 = quad_up<2>(incl);
  if (part >= 2) incl += u2;
  const float u3 = quad_up<1>(incl);
  const float before = part >= 1 ? u3 : 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) st4(p + 4 * j, pre[j] + before);
  raw += dpp_flip<0>(raw);
  raw += dpp_flip<1>(raw);
  if (isz && part == 0) vec[5][row] = raw;
}
__device__ __forceinline__ void rect_column_sums(const float (*X)[kLdT], const float (*Y)[kLdT], float (*vec)[64],
                                                 int tid) {
  const bool isy = tid >= 256;
  const int t = (tid >> 2) & 63, part = tid & 3;
  const float (*A)[kLdT] = isy ? Y : X;
  const int first = isy ? t + 1 : t;  // rows s >= first
  float acc = 0.f;
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    const int s_ = 4 * m + part;
    const float a = A[s_][t];
    acc += s_ >= first ? a : 0.f;
  }
  acc += dpp_flip<0>(acc);
  acc += dpp_flip<1>(acc);
  if (part == 0) vec[isy ? 11 : 10][t] = acc;
}

// Gradients of one (chunk, head). Wavefront w owns token block tb = w % 4
// (rows 16 tb ..) and, with half hw = w / 4, the 16 x 16 blocks (tb, key
// block KBW hw + c) of the 64 x K accumulators and (tb, 2 hw + c) of the
// 64 x 64 ones. Per value tile, the hw = 0 waves form K h, R, Ubar and dR of
// their token block and the hw = 1 waves K dh and dUbar; then every wave
// accumulates its blocks of dO h^T, Ubar dh^T, dR h^T, dR Ubar^T, dO Ubar^T.
template <int K, int V, typename InT>
__global__ __launch_bounds__(512) void chunk_bwd_grad_kernel(
    const InT* __restrict__ q, const InT* __restrict__ k, const InT* __restrict__ v, const float* __restrict__ d,
    const InT* __restrict__ dO, const int32_t* __restrict__ cu_seqlens, int T, int H, int N, int64_t nslots,
    const float* __restrict__ hck, const float* __restrict__ dhck, const float* __restrict__ Tg,
    const float* __restrict__ Pg, const float* __restrict__ KKg, const float* __restrict__ Gg,
    float* __restrict__ dq, float* __restrict__ dk,
    float* __restrict__ dv, float* __restrict__ dalpha, float* __restrict__ dbeta, float* __restrict__ dd_part) {
  constexpr int NT = 512, VT = kGrVT, NTILE = V / VT, LQ = K + 4, KB = K / 16, KBW = KB / 2;
  __shared__ SmemGrad<K> sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = blockIdx.x % H;
  const int64_t slot = blockIdx.x / H;
  if (slot >= nslots) return;
  int n, c, b, t0, t1;
  if (!slot_chunk(cu_seqlens, slot, T, N, n, c, b, t0, t1)) {
    if (tid == 0) dd_part[slot * H + h] = 0.f;
    return;
  }
  const int c0 = t0 + 64 * c, nrows = min(64, t1 - c0);
  const int64_t tok0 = (static_cast<int64_t>(b) * T + c0) * H + h;
  const float dh_ = d[h];
  const float* hsrc = hck + (slot * H + h) * V * K;
  const float* dhsrc = dhck + (slot * H + h) * V * K;
  const int64_t mb = (slot * H + h) * 64 * 64;

  const int l16 = lane & 15, l4 = lane >> 4;
  const int tb = wave & 3, hw = wave >> 2;
  const int ta = 16 * tb + l16;  // token row this lane supplies to A operands

  // Every load of the chunk's operands is issued before the first wait: q and
  // k rows, Tinv and P, the gates the prep kernel stored, the k_t.k_s entries
  // of the post phase, and the first value tile (below).
  constexpr int MPT = 64 * 16 / NT;
  RowPieces<K, NT, InT> rqk;
  rqk.load(q, k, tok0, H, nrows, tid);
  f32x4 rt[MPT], rp[MPT];
#pragma unroll
  for (int j = 0; j < MPT; ++j) {
    const int e = tid + j * NT, row = e >> 4, c4 = 4 * (e & 15);
    rt[j] = ld4_lower(Tg + mb, row, c4);
    rp[j] = ld4_lower(Pg + mb, row, c4);
  }
  f32x4 rg{};
  if (tid < kGateWords / 4) rg = ld4(Gg + (slot * H + h) * kGateWords + 4 * tid);
  float kkv[2][4];  // k_t.k_s of this lane's entries of the blocks (tb, 2 hw + cb)
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int i = 0; i < 4; ++i) kkv[cb][i] = KKg[mb + (16 * tb + 4 * l4 + i) * 64 + 16 * (2 * hw + cb) + l16];

  // Value tiles, loaded one tile ahead: the state and state-gradient rows
  // (one 16-byte piece each per thread), a four-channel piece of dO (threads
  // below 256) and, in the hw = 0 waves, v at this lane's rows (clamped; rows
  // past the end are replaced by zero where used).
  constexpr int SPC = VT * K / 4;  // state pieces per tile
  static_assert(SPC <= NT && 64 * VT / 4 <= NT, "at most one piece of each per thread");
  const int srow_ = tid / (K / 4), scol = 4 * (tid % (K / 4));
  const int orow = tid / (VT / 4), ocol = 4 * (tid % (VT / 4));
  const __amdgpu_buffer_rsrc_t orsrc = rows_rsrc(dO + tok0 * V, static_cast<int64_t>(nrows) * H * V * sizeof(InT));
  f32x4 pS{}, pdS{};
  typename Piece4<InT>::type pO{};
  InT pv[4];
  auto fetch_tile = [&](int jt) {
    const int v0 = jt * VT;
    if (tid < SPC) {
      pS = ld4(hsrc + static_cast<int64_t>(v0 + srow_) * K + scol);
      pdS = ld4(dhsrc + static_cast<int64_t>(v0 + srow_) * K + scol);
    }
    if (tid < 64 * VT / 4) pO = load4<InT>(orsrc, (orow * H * V + v0 + ocol) * static_cast<int>(sizeof(InT)));
    if (hw == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = min(16 * tb + 4 * l4 + i, nrows - 1);
        pv[i] = v[(tok0 + static_cast<int64_t>(t) * H) * V + v0 + l16];
      }
    }
  };
  fetch_tile(0);

  rqk.template store<LQ>(&sm.Qt[0][0], &sm.Kc[0][0], dh_, tid);
#pragma unroll
  for (int j = 0; j < MPT; ++j) {
    const int e = tid + j * NT, row = e >> 4, c4 = 4 * (e & 15);
    st4(&sm.Tm[row][c4], rt[j]);
    st4(&sm.Pm[row][c4], rp[j]);
  }
  if (tid < kGateWords / 4) st4(&sm.gt.G[0] + 4 * tid, rg);
  __syncthreads();
  f32x4 accQ[KBW], accK[KBW], accA[2], accP[2];
#pragma unroll
  for (int i = 0; i < KBW; ++i) accQ[i] = accK[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 2; ++i) accA[i] = accP[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  // per-lane sums over the tile channels, for the accumulator rows 16 tb + 4 l4 + i
  float sbR[4] = {0.f, 0.f, 0.f, 0.f}, sKhdR[4] = {0.f, 0.f, 0.f, 0.f}, st2[4] = {0.f, 0.f, 0.f, 0.f};
  float shdh = 0.f;

  for (int jt = 0; jt < NTILE; ++jt) {
    const int v0 = jt * VT;
    __syncthreads();
    if (tid < SPC) {
      st4(&sm.u.t.S[srow_][scol], pS);
      st4(&sm.u.t.dS[srow_][scol], pdS);
      shdh += hsum(pS * pdS);
    }
    if (tid < 64 * VT / 4) st4(&sm.u.t.dO[orow][ocol], unpack4(pO));
    float vv[4] = {0.f, 0.f, 0.f, 0.f};
    if (hw == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) vv[i] = 16 * tb + 4 * l4 + i < nrows ? to_f32(pv[i]) : 0.f;
    }
    if (jt + 1 < NTILE) fetch_tile(jt + 1);  // in flight during this tile's work
    __syncthreads();
    // K h (hw = 0) or K dh (hw = 1) for token block tb; B[k][v] = X[v][k]
    f32x4 kx{0.f, 0.f, 0.f, 0.f};
    {
      const float(*X)[K + 4] = hw == 0 ? sm.u.t.S : sm.u.t.dS;
#pragma unroll 8
      for (int j = 0; j < K / 4; ++j) kx = mma4(sm.Kc[ta][4 * j + l4], X[l16][4 * j + l4], kx);
    }
    if (hw == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * tb + 4 * l4 + i;
        sm.u.t.R[t][l16] = sm.gt.beta[t] * vv[i] - sm.gt.bEGx[t] * kx[i];
      }
    }
    __syncthreads();
    if (hw == 0) {
      // Ubar = Tinv R (Tinv is zero above the diagonal)
      f32x4 u{0.f, 0.f, 0.f, 0.f};
      for (int j = 0; j < 4 * (tb + 1); ++j) u = mma4(sm.Tm[ta][4 * j + l4], sm.u.t.R[4 * j + l4][l16], u);
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.u.t.U[16 * tb + 4 * l4 + i][l16] = u[i];
    } else {
      // dUbar = P^T dO + diag(e^(Gn - G)) K dh; A[t][t'] = P[t'][t], zero for t' < t
      f32x4 du;
#pragma unroll
      for (int i = 0; i < 4; ++i) du[i] = sm.gt.EGnG[16 * tb + 4 * l4 + i] * kx[i];
      for (int j = 4 * tb; j < 16; ++j) du = mma4(sm.Pm[4 * j + l4][ta], sm.u.t.dO[4 * j + l4][l16], du);
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.u.t.dU[16 * tb + 4 * l4 + i][l16] = du[i];
    }
    __syncthreads();
    f32x4 dr{0.f, 0.f, 0.f, 0.f};
    if (hw == 0) {
      // dR = Tinv^T dUbar
      for (int j = 4 * tb; j < 16; ++j) dr = mma4(sm.Tm[4 * j + l4][ta], sm.u.t.dU[4 * j + l4][l16], dr);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) st2[i] += kx[i] * sm.u.t.U[16 * tb + 4 * l4 + i][l16];
    }
    __syncthreads();
    if (hw == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * tb + 4 * l4 + i;
        sm.u.t.dU[t][l16] = dr[i];
        if (t < nrows) dv[(tok0 + static_cast<int64_t>(t) * H) * V + v0 + l16] = sm.gt.beta[t] * dr[i];
        sbR[i] += dr[i] * (vv[i] - expf(sm.gt.Gx[t]) * kx[i]);
        sKhdR[i] += kx[i] * dr[i];
      }
    }
    __syncthreads();
    // accumulators over the tile's channels (reduction index 4 j + l4)
#pragma unroll
    for (int j = 0; j < VT / 4; ++j) {
      const int vc = 4 * j + l4;
      const float aO = sm.u.t.dO[ta][vc];
      const float aR = sm.u.t.dU[ta][vc];  // dR
      const float aU = sm.gt.EGnG[ta] * sm.u.t.U[ta][vc];
      const float aRb = -sm.gt.bEGx[ta] * aR;
#pragma unroll
      for (int cb = 0; cb < KBW; ++cb) {
        const int kcol = 16 * (KBW * hw + cb) + l16;
        const float bS = sm.u.t.S[vc][kcol], bdS = sm.u.t.dS[vc][kcol];
        accQ[cb] = mma4(aO, bS, accQ[cb]);
        accK[cb] = mma4(aU, bdS, accK[cb]);
        accK[cb] = mma4(aRb, bS, accK[cb]);
      }
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const float bU = sm.u.t.U[16 * (2 * hw + cb) + l16][vc];  // B[v][s] = Ubar[s][v]
        accA[cb] = mma4(-aR, bU, accA[cb]);
        accP[cb] = mma4(aO, bU, accP[cb]);
      }
    }
  }
  __syncthreads();

  // sums over channels: reduce over the 16 lanes of a row group
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) {
      sbR[i] += __shfl_xor(sbR[i], m, kWave);
      sKhdR[i] += __shfl_xor(sKhdR[i], m, kWave);
      st2[i] += __shfl_xor(st2[i], m, kWave);
    }
  }
  if (l16 == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * tb + 4 * l4 + i;
      if (hw == 0) {
        sm.vec[1][t] = sbR[i];
        sm.vec[2][t] = sKhdR[i];
      } else {
        sm.vec[3][t] = st2[i];
      }
    }
  }
  // sum over channels of (Qt h)_t . dO_t = sum over keys of Qt_t . (dO h^T)_t, per wave half
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = 16 * tb + 4 * l4 + i;
    float x = 0.f;
#pragma unroll
    for (int cb = 0; cb < KBW; ++cb) x += sm.Qt[t][16 * (KBW * hw + cb) + l16] * accQ[cb][i];
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) x += __shfl_xor(x, m, kWave);
    if (l16 == 0) sm.vec[8 + hw][t] = x;
  }
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) shdh += __shfl_xor(shdh, m, kWave);
  if (lane == 0) sm.red[wave] = shdh;
  // masks and elementwise products of the 64 x 64 blocks (tb, 2 hw + cb)
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * tb + 4 * l4 + i, s_ = 16 * (2 * hw + cb) + l16;
      const float M = s_ <= t ? expf(fminf(sm.gt.G[t] - sm.gt.G[s_], 0.f)) : 0.f;
      const float E = s_ < t ? expf(fminf(sm.gt.Gx[t] - sm.gt.G[s_], 0.f)) : 0.f;
      const float dpv = s_ <= t ? accP[cb][i] : 0.f, dav = s_ < t ? accA[cb][i] : 0.f;
      const float w = dav * E;
      sm.Pm[t][s_] = dpv * sm.Pm[t][s_];  // dP (.) P
      sm.Tm[t][s_] = dpv * M;             // dP (.) M
      sm.u.p.W[t][s_] = w;
      sm.u.p.X[t][s_] = w * kkv[cb][i];
    }
  }
  __syncthreads();
  // first pass of the rectangle sums (dP (.) P in Pm, W (.) k_t.k_s in X)
  rect_row_prefix(sm.Pm, sm.u.p.X, sm.gt.beta, sm.vec, tid);
  // dq, dk of the blocks (tb, KBW hw + cb)
  f32x4 xq[KBW], xk[KBW];
#pragma unroll
  for (int cb = 0; cb < KBW; ++cb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) xq[cb][i] = sm.gt.EG[16 * tb + 4 * l4 + i] * accQ[cb][i];
    xk[cb] = accK[cb];
  }
  const float bta = sm.gt.beta[ta];
  for (int j = 0; j < 4 * (tb + 1); ++j) {  // columns s <= t: (dP (.) M) K and diag(beta) W K
    const int sr = 4 * j + l4;
    const float a1 = sm.Tm[ta][sr], a2 = bta * sm.u.p.W[ta][sr];
#pragma unroll
    for (int cb = 0; cb < KBW; ++cb) {
      const float bK = sm.Kc[sr][16 * (KBW * hw + cb) + l16];
      xq[cb] = mma4(a1, bK, xq[cb]);
      xk[cb] = mma4(a2, bK, xk[cb]);
    }
  }
  for (int j = 4 * tb; j < 16; ++j) {  // rows t' >= t: (dP (.) M)^T Qt and W^T diag(beta) K
    const int tr2 = 4 * j + l4;
    const float a1 = sm.Tm[tr2][ta], a2 = sm.u.p.W[tr2][ta], bb = sm.gt.beta[tr2];
#pragma unroll
    for (int cb = 0; cb < KBW; ++cb) {
      const int kc = 16 * (KBW * hw + cb) + l16;
      xk[cb] = mma4(a1, sm.Qt[tr2][kc], xk[cb]);
      xk[cb] = mma4(a2, bb * sm.Kc[tr2][kc], xk[cb]);
    }
  }
  float ddp = 0.f;
#pragma unroll
  for (int cb = 0; cb < KBW; ++cb) {
    const int kc = 16 * (KBW * hw + cb) + l16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * tb + 4 * l4 + i;
      xk[cb][i] -= dh_ * xq[cb][i];
      ddp -= xq[cb][i] * sm.Kc[t][kc];
      if (t < nrows) {
        const int64_t off = (tok0 + static_cast<int64_t>(t) * H) * K + kc;
        dq[off] = xq[cb][i];
        dk[off] = xk[cb][i];
      }
    }
  }
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) ddp += __shfl_xor(ddp, m, kWave);
  __syncthreads();
  if (lane == 0) sm.red[8 + wave] = ddp;
  rect_column_sums(sm.Pm, sm.u.p.X, sm.vec, tid);
  __syncthreads();
  if (wave == 0) grad_scalars(sm.gt, sm.vec, sm.red, lane, nrows, tok0, H, dalpha, dbeta, dd_part + slot * H + h);
}

// Reverse scan of dh on fp32 matrix-core tiles. Wavefront w owns channel
// block vb = w / 4 and token block tb of dUbar and dR, and the blocks
// (KBD tb + c, vb) of dh, with tb = w % 4 for vb = 0 and 3 - w % 4 for vb = 1:
// the two wavefronts of a SIMD (w and w + 4) then hold triangle rows of
// complementary length, 16 - 4 tb blocks each for P^T dO and Tinv^T dUbar.
template <int K, int V, typename InT>
__global__ __launch_bounds__(512) void chunk_bwd_dh_kernel(
    const InT* __restrict__ q, const InT* __restrict__ k, const float* __restrict__ d, const InT* __restrict__ dO,
    const int32_t* __restrict__ cu_seqlens, int T, int H, int N, const float* __restrict__ Tg,
    const float* __restrict__ Pg, const float* __restrict__ Gg, const float* __restrict__ dsf,
    float* __restrict__ dhck, float* __restrict__ ds0) {
  constexpr int NT = 512, VT = kDhVT, NVT = V / VT, KBD = K / 64;
  constexpr int MPT = 64 * 16 / NT;  // 16-byte pieces of Tinv and P per thread
  static_assert(VT == 32, "two 16-channel blocks per workgroup");
  static_assert(64 * VT / 4 == NT, "one four-element piece of dO per thread");
  __shared__ SmemDh<K> sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int unit, vt;
  if (!unit_of_block(blockIdx.x, NVT, N * H, unit, vt)) return;
  const int h = unit % H, n = unit / H;
  int b, t0, t1;
  sequence_range(cu_seqlens, n, T, b, t0, t1);
  const float dh_ = d[h];
  const int nch = (t1 - t0 + 63) / 64;
  const bool packed = cu_seqlens != nullptr;
  const int64_t srow = (static_cast<int64_t>(n) * H + h) * V + vt * VT;  // state row of channel 0 of the tile
  const int l16 = lane & 15, l4 = lane >> 4;
  const int vb = wave >> 2, tb = vb == 0 ? (wave & 3) : 3 - (wave & 3);
  const int ta = 16 * tb + l16, vc = 16 * vb + l16;

  // The next chunk's operands, loaded one chunk ahead into registers (raw
  // words; rows past the end of the sequence load as zeros), and its gates as
  // the prep kernel stored them.
  RowPieces<K, NT, InT> rqk;
  typename Piece4<InT>::type ro;
  f32x4 rg{};
  f32x4 rt[MPT], rp[MPT];
  const int orow = tid / (VT / 4), ocol = 4 * (tid % (VT / 4));  // this thread's piece of dO
  auto fetch = [&](int ci) {
    const int c0 = t0 + 64 * ci, nrows = min(64, t1 - c0);
    const int64_t tok0 = (static_cast<int64_t>(b) * T + c0) * H + h;
    const int64_t mb = (chunk_slot(packed, t0, n, ci, T) * H + h) * 64 * 64;
    rqk.load(q, k, tok0, H, nrows, tid);
    const __amdgpu_buffer_rsrc_t orsrc =
        rows_rsrc(dO + tok0 * V, static_cast<int64_t>(nrows) * H * V * sizeof(InT));
    ro = load4<InT>(orsrc, (orow * H * V + vt * VT + ocol) * static_cast<int>(sizeof(InT)));
#pragma unroll
    for (int j = 0; j < MPT; ++j) {
      const int e = tid + j * NT, row = e >> 4, c4 = 4 * (e & 15);
      rt[j] = ld4_lower(Tg + mb, row, c4);
      rp[j] = ld4_lower(Pg + mb, row, c4);
    }
    if (tid < kGateWords / 4) rg = ld4(Gg + (chunk_slot(packed, t0, n, ci, T) * H + h) * kGateWords + 4 * tid);
  };

  {
    // dh of the last chunk = dL/dS_final ([channel][key] in memory, [key][channel] here)
    constexpr int FP = K * VT / 4 / NT;
    static_assert(FP * 4 * NT == K * VT, "whole pieces per thread");
    f32x4 x[FP];
#pragma unroll
    for (int j = 0; j < FP; ++j) {
      const int e = tid + j * NT, cc = e / (K / 4), k4 = 4 * (e % (K / 4));
      x[j] = dsf ? ld4(dsf + (srow + cc) * K + k4) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int j = 0; j < FP; ++j) {
      const int e = tid + j * NT, cc = e / (K / 4), k4 = 4 * (e % (K / 4));
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.dh[k4 + i][cc] = x[j][i];
    }
  }
  if (nch > 0) fetch(nch - 1);
  for (int ci = nch - 1; ci >= 0; --ci) {
    const int64_t slot = chunk_slot(packed, t0, n, ci, T);
    __syncthreads();
    rqk.template store<K + 4>(&sm.Qt[0][0], &sm.Kc[0][0], dh_, tid);
    st4(&sm.dO[orow][ocol], unpack4(ro));
#pragma unroll
    for (int j = 0; j < MPT; ++j) {
      const int e = tid + j * NT, row = e >> 4, c4 = 4 * (e & 15);
      st4(&sm.Tm[row][c4], rt[j]);
      st4(&sm.Pm[row][c4], rp[j]);
    }
    if (tid < kGateWords / 4) st4(&sm.gt.G[0] + 4 * tid, rg);
    // the gradient of this chunk's outgoing state, for the gradient kernel ([channel][key])
    {
      float* dst = dhck + (slot * H + h) * V * K + static_cast<int64_t>(vt) * VT * K;
      for (int e = tid; e < VT * K / 4; e += NT) {
        const int cc = e / (K / 4), k4 = 4 * (e % (K / 4));
        f32x4 x;
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = sm.dh[k4 + i][cc];
        st4(dst + static_cast<int64_t>(cc) * K + k4, x);
      }
    }
    __syncthreads();
    if (ci > 0) fetch(ci - 1);  // in flight during this chunk's work
    // dUbar = P^T dO + diag(e^(Gn - G)) K dh   (block tb, vb); A[t][t'] = P[t'][t]
    {
      f32x4 kd{0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
      for (int j = 0; j < K / 4; ++j) kd = mma4(sm.Kc[ta][4 * j + l4], sm.dh[4 * j + l4][vc], kd);
      f32x4 du;
#pragma unroll
      for (int i = 0; i < 4; ++i) du[i] = sm.gt.EGnG[16 * tb + 4 * l4 + i] * kd[i];
      for (int j = 4 * tb; j < 16; ++j) du = mma4(sm.Pm[4 * j + l4][ta], sm.dO[4 * j + l4][vc], du);
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.dU[16 * tb + 4 * l4 + i][vc] = du[i];
    }
    __syncthreads();
    // dR = Tinv^T dUbar
    f32x4 dr{0.f, 0.f, 0.f, 0.f};
    for (int j = 4 * tb; j < 16; ++j) dr = mma4(sm.Tm[4 * j + l4][ta], sm.dU[4 * j + l4][vc], dr);
#pragma unroll
    for (int i = 0; i < 4; ++i) sm.dR[16 * tb + 4 * l4 + i][vc] = dr[i];
    __syncthreads();
    // dh_in = e^Gn dh + Qt^T diag(e^G) dO - K^T diag(b1) dR   (blocks (KBD tb + c, vb)); A[k][t] = X[t][k]
    const float eGn = sm.gt.EG[63];
    f32x4 acc[KBD];
#pragma unroll
    for (int cb = 0; cb < KBD; ++cb) {
      const int kb = KBD * tb + cb;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[cb][i] = eGn * sm.dh[16 * kb + 4 * l4 + i][vc];
    }
#pragma unroll 4
    for (int j = 0; j < 16; ++j) {
      const int tr2 = 4 * j + l4;
      const float bO = sm.gt.EG[tr2] * sm.dO[tr2][vc], bR = -sm.gt.bEGx[tr2] * sm.dR[tr2][vc];
#pragma unroll
      for (int cb = 0; cb < KBD; ++cb) {
        const int kc = 16 * (KBD * tb + cb) + l16;
        acc[cb] = mma4(sm.Qt[tr2][kc], bO, acc[cb]);
        acc[cb] = mma4(sm.Kc[tr2][kc], bR, acc[cb]);
      }
    }
    __syncthreads();
#pragma unroll
    for (int cb = 0; cb < KBD; ++cb) {
      const int kb = KBD * tb + cb;
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.dh[16 * kb + 4 * l4 + i][vc] = acc[cb][i];
    }
  }
  __syncthreads();
  if (ds0) {
    for (int e = tid; e < K * VT; e += NT) {
      const int kk = e % K, cc = e / K;
      ds0[(srow + cc) * K + kk] = sm.dh[kk][cc];
    }
  }
}

// ---- reverse scan of dh on bf16 matrix cores (bf16 q, k, dO) ----------------------------

constexpr int kDhbVT = 64;  // value channels per workgroup of the bf16 reverse scan

// One chunk of the scan in LDS. Exact bf16 operands: q, k (token rows, keys
// of each 32-block in perm32 order) and dO (token rows). Split into hi / lo
// bf16: P and Tinv ([t'][t] as the prep kernel stores them), and the
// right-hand operands dUbar, X = diag(e^G) dO, Z = -d X - diag(b1) dR and dh,
// stored by channel with the reduction axis (tokens or keys) in perm32 order.
// ---- reverse scan on bf16 matrix cores, producer / consumer form -------------------------

// One chunk's shared operands of the reverse scan, double-buffered between
// the producer and the consumer wavefronts: q and k rows ([token][key], keys
// of each 32-block in perm32 order), Tinv and P split hi / lo ([t][s]), dO
// ([token][channel]) and the three gate rows the consumers read, by token.
template <int K>
struct alignas(16) DhChunkBuf {
  u16 Qc[64 * K], Kc[64 * K];
  u16 Th[64 * 64], Tl[64 * 64], Ph[64 * 64], Pl[64 * 64];
  u16 dO[64 * kDhbVT];
  float b1[64], eg[64], en[64];  // beta e^Gx, e^G, e^(Gn - G): rows 3-5 of the stored gates
};

// Reverse scan of dh for bf16 inputs, 64 value channels per workgroup, in the
// forward's two roles one chunk apart. Producers (wavefronts 4-7) stage chunk
// c - 1 (q, k, Tinv, P, dO, gates; loads issued a chunk ahead) while the
// consumers (wavefronts 0-3, 16 channels each) run chunk c; one barrier per
// chunk hands a buffer over. A consumer keeps dh (keys x its 16 channels) in
// fp32 registers for the whole sequence and needs no other wavefront's
// results, so the chain of a chunk has no barrier inside:
//   dUbar = diag(e^(Gn - G)) K dh + P^T dO   (K dh over its own channels)
//   dR    = Tinv^T dUbar,  X = diag(e^G) dO,  Z = -d X - diag(b1) dR
//   dh   <- e^Gn dh + q^T X + k^T Z
// with every fp32 operand split into hi + lo bf16 as in the forward.
template <int K, int V>
__global__ __launch_bounds__(512) void chunk_bwd_dh_pc_kernel(
    const u16* __restrict__ q, const u16* __restrict__ k, const float* __restrict__ d, const u16* __restrict__ dO,
    const int32_t* __restrict__ cu_seqlens, int T, int H, int N, const float* __restrict__ Tg,
    const float* __restrict__ Pg, const float* __restrict__ Gg, const float* __restrict__ dsf,
    float* __restrict__ dhck, float* __restrict__ ds0) {
  constexpr int VT = kDhbVT, NVT = V / VT, NS = K / 32, KB = K / 16;
  static_assert(VT == 64, "four consumer wavefronts of 16 channels");
  __shared__ DhChunkBuf<K> buf[2];
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int unit, vt;
  if (!unit_of_block(blockIdx.x, NVT, N * H, unit, vt)) return;
  const int h = unit % H, n = unit / H;
  int b, t0, t1;
  sequence_range(cu_seqlens, n, T, b, t0, t1);
  const int nch = (t1 - t0 + 63) / 64;
  const bool packed = cu_seqlens != nullptr;

  if (wave >= 4) {
    // ======================= producers: stage chunk nch - 1 - it in iteration it =======================
    const int ptid = tid - 256;
    constexpr int MPT = 64 * 16 / 256;  // 16-byte pieces of a 64 x 64 fp32 matrix per thread
    RowPieces<K, 256, u16> rqk;
    f32x4 rt[MPT], rp[MPT], rg{};
    u32x4 ro[2];
    const int orow = ptid / (VT / 8), ocol = 8 * (ptid % (VT / 8));  // dO pieces: rows orow, orow + 32
    auto fetch = [&](int ci) {
      const int c0 = t0 + 64 * ci, nrows = min(64, t1 - c0);
      const int64_t tok0 = (static_cast<int64_t>(b) * T + c0) * H + h;
      const int64_t sl = chunk_slot(packed, t0, n, ci, T) * H + h;
      rqk.load(q, k, tok0, H, nrows, ptid);
      const __amdgpu_buffer_rsrc_t orsrc = rows_rsrc(dO + tok0 * V, static_cast<int64_t>(nrows) * H * V * 2);
#pragma unroll
      for (int j = 0; j < 2; ++j) ro[j] = load16(orsrc, ((orow + 32 * j) * H * V + vt * VT + ocol) * 2);
#pragma unroll
      for (int j = 0; j < MPT; ++j) {
        const int e = ptid + j * 256, row = e >> 4, c4 = 4 * (e & 15);
        rt[j] = ld4_lower(Tg + sl * 64 * 64, row, c4);
        rp[j] = ld4_lower(Pg + sl * 64 * 64, row, c4);
      }
      if (ptid < 48) rg = ld4(Gg + sl * kGateWords + 3 * 64 + 4 * ptid);
    };
    if (nch > 0) fetch(nch - 1);
    for (int it = 0; it <= nch; ++it) {
      if (it < nch) {
        DhChunkBuf<K>& bf = buf[it & 1];
        rqk.store_bf16(bf.Qc, bf.Kc, ptid);
#pragma unroll
        for (int j = 0; j < 2; ++j) *reinterpret_cast<u32x4*>(&bf.dO[swz<VT>(orow + 32 * j, ocol)]) = ro[j];
#pragma unroll
        for (int j = 0; j < MPT; ++j) {
          const int e = ptid + j * 256, row = e >> 4, c4 = 4 * (e & 15);
          put_split4(bf.Th, bf.Tl, swz<64>(row, c4), rt[j]);
          put_split4(bf.Ph, bf.Pl, swz<64>(row, c4), rp[j]);
        }
        if (ptid < 48) {
          const int r = ptid >> 4;
          st4((r == 0 ? bf.b1 : r == 1 ? bf.eg : bf.en) + 4 * (ptid & 15), rg);
        }
        if (it + 1 < nch) fetch(nch - 2 - it);  // in flight during the next chunk's staging wait
      }
      __syncthreads();
    }
    return;
  }

  // ======================= consumers: chunk nch - it in iteration it =======================
  const int cw = wave;
  const int cpos = 16 * cw + 4 * (l16 & 3);  // dO tile position of this lane's channel quad
  const int64_t crow = (static_cast<int64_t>(n) * H + h) * V + vt * VT + 16 * cw + l16;  // state row
  const float dd_ = d[h];
  f32x4 dh[KB];  // dh[key 16 kb + 4 g + i][channel]
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
    dh[kb] = dsf ? ld4(dsf + crow * K + 16 * kb + 4 * g) : f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it <= nch; ++it) {
    if (it > 0) {
      const int ci = nch - it;
      const DhChunkBuf<K>& bf = buf[(it - 1) & 1];
      // this chunk's outgoing-state gradient, fp32 [channel][key], for the gradient pass
      float* dst = dhck + ((chunk_slot(packed, t0, n, ci, T) * H + h) * V + vt * VT + 16 * cw + l16) * K;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) st4(dst + 16 * kb + 4 * g, dh[kb]);
      bf16x8 hb[NS], lb[NS];
#pragma unroll
      for (int s_ = 0; s_ < NS; ++s_) split_pair(dh[2 * s_], dh[2 * s_ + 1], hb[s_], lb[s_]);
      // dUbar = diag(e^(Gn - G)) K dh + P^T dO (P[t'][t] = 0 for t' < t)
      f32x4 du[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        f32x4 kd{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s_ = 0; s_ < NS; ++s_) {
          const bf16x8 a = lds8(&bf.Kc[swz<K>(16 * r + l16, 32 * s_ + 8 * g)]);
          kd = mfma16x16x32(a, hb[s_], kd);
          kd = mfma16x16x32(a, lb[s_], kd);
        }
        du[r] = ld4(&bf.en[16 * r + 4 * g]) * kd;
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          if (s2 == 0 && r >= 2) continue;
          const bf16x8 o = tr_frag<VT>(bf.dO, 32 * s2, cpos, g, l16);
          const int pos = 16 * r + 4 * (l16 & 3);
          du[r] = mfma16x16x32(tr_frag<64>(bf.Ph, 32 * s2, pos, g, l16), o, du[r]);
          du[r] = mfma16x16x32(tr_frag<64>(bf.Pl, 32 * s2, pos, g, l16), o, du[r]);
        }
      }
      // dR = Tinv^T dUbar (Tinv[t'][t] = 0 for t' < t); X = diag(e^G) dO; Z = -d X - diag(b1) dR
      bf16x8 uh[2], ul[2];
      split_pair(du[0], du[1], uh[0], ul[0]);
      split_pair(du[2], du[3], uh[1], ul[1]);
      f32x4 X[4], Z[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        f32x4 dr{0.f, 0.f, 0.f, 0.f};
        const int pos = 16 * r + 4 * (l16 & 3);
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          if (s2 == 0 && r >= 2) continue;
          dr = mma3(tr_frag<64>(bf.Th, 32 * s2, pos, g, l16), tr_frag<64>(bf.Tl, 32 * s2, pos, g, l16), uh[s2], ul[s2],
                    dr);
        }
        X[r] = ld4(&bf.eg[16 * r + 4 * g]) * tr4<VT>(bf.dO, 16 * r, cpos, g, l16);
        Z[r] = -dd_ * X[r] - ld4(&bf.b1[16 * r + 4 * g]) * dr;
      }
      bf16x8 xh[2], xl[2], zh[2], zl[2];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        split_pair(X[2 * s2], X[2 * s2 + 1], xh[s2], xl[s2]);
        split_pair(Z[2 * s2], Z[2 * s2 + 1], zh[s2], zl[s2]);
      }
      // dh <- e^Gn dh + q^T X + k^T Z
      const float eGn = bf.eg[63];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        f32x4 acc = eGn * dh[kb];
        const int pos = perm_col(16 * kb + 4 * (l16 & 3));
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const bf16x8 aq = tr_frag<K>(bf.Qc, 32 * s2, pos, g, l16), ak = tr_frag<K>(bf.Kc, 32 * s2, pos, g, l16);
          acc = mfma16x16x32(aq, xh[s2], acc);
          acc = mfma16x16x32(aq, xl[s2], acc);
          acc = mfma16x16x32(ak, zh[s2], acc);
          acc = mfma16x16x32(ak, zl[s2], acc);
        }
        dh[kb] = acc;
      }
    }
    __syncthreads();
  }
  if (ds0) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) st4(ds0 + crow * K + 16 * kb + 4 * g, dh[kb]);
  }
}

// ---- per-chunk gradients on bf16 matrix cores (bf16 q, k, v, dO) -------------------------

constexpr int kGbVT = 32;  // value channels per tile of the bf16 gradient kernel

// LDS of the bf16 gradient kernel. Exact bf16: q, k ([token][key], keys in
// perm32 order), dO ([token][channel], perm32) and v ([token][channel]). Split
// hi / lo: Tinv and P ([t][s], s in perm32 order), the state and
// state-gradient tiles ([channel][key], perm32) and R, Ubar, dUbar, dR
// ([channel][token], perm32); after the value tiles, dP (.) M and beta W as
// [s][t] (t in perm32 order), and dP (.) P and W (.) k_t.k_s in fp32.
template <int K>
struct alignas(16) SmemGradB {
  u16 Qc[64 * K], Kc[64 * K];
  u16 Th[64 * 64], Tl[64 * 64], Ph[64 * 64], Pl[64 * 64];
  union {
    struct {
      u16 hh[kGbVT * K], hl[kGbVT * K], dhh[kGbVT * K], dhl[kGbVT * K];
      u16 dO[64 * kGbVT], Vt[64 * kGbVT];
      u16 Rh[kGbVT * 64], Rl[kGbVT * 64], Uh[kGbVT * 64], Ul[kGbVT * 64];
      u16 dUh[kGbVT * 64], dUl[kGbVT * 64], dRh[kGbVT * 64], dRl[kGbVT * 64];
    } t;
    struct {
      u16 dPMh[64 * 64], dPMl[64 * 64], WBh[64 * 64], WBl[64 * 64];
      float dPP[64][kLdT];  // dP (.) P
      float Z[64][kLdT];    // W (.) k_t.k_s
    } p;
  } u;
  ChunkGates gt;
  float vec[12][64];
  float red[16];
};

// Gradients of one (chunk, head) for bf16 inputs: the products of
// chunk_bwd_grad_kernel on 16x16x32 bf16 matrix cores, every fp32 operand
// split into hi + lo bf16 (exact operands enter once), over value tiles of 32
// channels. Wavefront w owns token block tb = w % 4 and half hw = w / 4: per
// tile the hw = 0 wavefronts form K h, R, Ubar and dR of their token block
// and the hw = 1 wavefronts K dh and dUbar (both channel blocks), then every
// wavefront accumulates its blocks (tb, KBW hw + c) of dO h^T, Ubar dh^T and
// dR h^T and (tb, 2 hw + c) of dR Ubar^T and dO Ubar^T. The row scales
// e^(Gn - G) and b1 of Ubar dh^T and dR h^T apply after the channel sums.
template <int K, int V>
__global__ __launch_bounds__(512) void chunk_bwd_grad_bf16_kernel(
    const u16* __restrict__ q, const u16* __restrict__ k, const u16* __restrict__ v, const float* __restrict__ d,
    const u16* __restrict__ dO, const int32_t* __restrict__ cu_seqlens, int T, int H, int N, int64_t nslots,
    const float* __restrict__ hck, const float* __restrict__ dhck, const float* __restrict__ Tg,
    const float* __restrict__ Pg, const float* __restrict__ Gg, float* __restrict__ dq, float* __restrict__ dk,
    float* __restrict__ dv, float* __restrict__ dalpha, float* __restrict__ dbeta, float* __restrict__ dd_part) {
  constexpr int NT = 512, VT = kGbVT, NTILE = V / VT, KB = K / 16, KBW = KB / 2;
  constexpr int HP = VT * K / 4 / NT;  // 16-byte pieces of a state tile per thread
  constexpr int MPT = 64 * 16 / NT;
  static_assert(HP >= 1 && HP * 4 * NT == VT * K && 64 * VT / 4 == NT, "whole pieces per thread");
  __shared__ SmemGradB<K> sm;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = blockIdx.x % H;
  const int64_t slot = blockIdx.x / H;
  if (slot >= nslots) return;
  int n, c, b, t0, t1;
  if (!slot_chunk(cu_seqlens, slot, T, N, n, c, b, t0, t1)) {
    if (tid == 0) dd_part[slot * H + h] = 0.f;
    return;
  }
  const int c0 = t0 + 64 * c, nrows = min(64, t1 - c0);
  const int64_t tok0 = (static_cast<int64_t>(b) * T + c0) * H + h;
  const float dd_ = d[h];
  const float* hsrc = hck + (slot * H + h) * V * K;
  const float* dhsrc = dhck + (slot * H + h) * V * K;
  const int64_t mb = (slot * H + h) * 64 * 64;
  const int tb = wave & 3, hw = wave >> 2;
  const int pt = perm_col(16 * tb + 4 * (l16 & 3));  // tile position of this lane's token quad (block tb)

  // every load of the chunk's operands before the first wait
  RowPieces<K, NT, u16> rqk;
  rqk.load(q, k, tok0, H, nrows, tid);
  f32x4 rt[MPT], rp[MPT];
#pragma unroll
  for (int j = 0; j < MPT; ++j) {
    const int e = tid + j * NT, row = e >> 4, c4 = 4 * (e & 15);
    rt[j] = ld4_lower(Tg + mb, row, c4);
    rp[j] = ld4_lower(Pg + mb, row, c4);
  }
  f32x4 rg{};
  if (tid < kGateWords / 4) rg = ld4(Gg + (slot * H + h) * kGateWords + 4 * tid);
  // value tiles, one tile ahead: state rows, state-gradient rows, dO and v pieces
  const int orow = tid / (VT / 4), ocol = 4 * (tid % (VT / 4));
  const __amdgpu_buffer_rsrc_t orsrc = rows_rsrc(dO + tok0 * V, static_cast<int64_t>(nrows) * H * V * 2);
  const __amdgpu_buffer_rsrc_t vrsrc = rows_rsrc(v + tok0 * V, static_cast<int64_t>(nrows) * H * V * 2);
  f32x4 pS[HP], pdS[HP];
  u32x2 pO, pV;
  // fp32 gradient rows of the chunk; stores to rows past its end fall outside
  // the resource and are dropped
  const __amdgpu_buffer_rsrc_t dvrsrc = rows_rsrc(dv + tok0 * V, static_cast<int64_t>(nrows) * H * V * 4);
  // in three parts, spread over a tile's stages: issued together, the loads
  // of all eight wavefronts queue in the CU's memory unit and hold up the
  // wavefronts behind them
  auto fetch_h = [&](int jt) {
#pragma unroll
    for (int j = 0; j < HP; ++j) {
      const int e = tid + j * NT, row = e / (K / 4), k4 = 4 * (e % (K / 4));
      pS[j] = ld4(hsrc + static_cast<int64_t>(jt * VT + row) * K + k4);
    }
  };
  auto fetch_dh = [&](int jt) {
#pragma unroll
    for (int j = 0; j < HP; ++j) {
      const int e = tid + j * NT, row = e / (K / 4), k4 = 4 * (e % (K / 4));
      pdS[j] = ld4(dhsrc + static_cast<int64_t>(jt * VT + row) * K + k4);
    }
  };
  auto fetch_ov = [&](int jt) {
    const int off = (orow * H * V + jt * VT + ocol) * 2;
    pO = __builtin_amdgcn_raw_buffer_load_b64(orsrc, off, 0, 0);
    pV = __builtin_amdgcn_raw_buffer_load_b64(vrsrc, off, 0, 0);
  };
  fetch_h(0);
  fetch_dh(0);
  fetch_ov(0);

  rqk.store_bf16(sm.Qc, sm.Kc, tid);
#pragma unroll
  for (int j = 0; j < MPT; ++j) {
    const int e = tid + j * NT, row = e >> 4, c4 = 4 * (e & 15);
    put_split4(sm.Th, sm.Tl, swz<64>(row, perm_col(c4)), rt[j]);
    put_split4(sm.Ph, sm.Pl, swz<64>(row, perm_col(c4)), rp[j]);
  }
  if (tid < kGateWords / 4) st4(&sm.gt.G[0] + 4 * tid, rg);

  f32x4 accQ[KBW], accUd[KBW], accRh[KBW], accA[2], accP[2];
#pragma unroll
  for (int i = 0; i < KBW; ++i) accQ[i] = accUd[i] = accRh[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 2; ++i) accA[i] = accP[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  // per-lane sums over channels, for the rows 16 tb + 4 g + i
  f32x4 sbR{0.f, 0.f, 0.f, 0.f}, sKhdR{0.f, 0.f, 0.f, 0.f}, st2{0.f, 0.f, 0.f, 0.f};
  float shdh = 0.f;

  f32x4 eGx;  // e^Gx of this lane's four token rows
  for (int jt = 0; jt < NTILE; ++jt) {
    const int v0 = jt * VT;
    __syncthreads();
    if (jt == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) eGx[i] = __expf(sm.gt.Gx[16 * tb + 4 * g + i]);
    }
#pragma unroll
    for (int j = 0; j < HP; ++j) {
      const int e = tid + j * NT, row = e / (K / 4), k4 = 4 * (e % (K / 4));
      put_split4(sm.u.t.hh, sm.u.t.hl, swz<K>(row, perm_col(k4)), pS[j]);
      put_split4(sm.u.t.dhh, sm.u.t.dhl, swz<K>(row, perm_col(k4)), pdS[j]);
      shdh += hsum(pS[j] * pdS[j]);
    }
    *reinterpret_cast<u32x2*>(&sm.u.t.dO[swz<VT>(orow, perm_col(ocol))]) = pO;
    *reinterpret_cast<u32x2*>(&sm.u.t.Vt[swz<VT>(orow, ocol)]) = pV;
    __syncthreads();
    if (jt + 1 < NTILE) fetch_h(jt + 1);  // in flight during this tile's work
    // Opaque per-tile copies of the lane coordinates: the LDS addresses below
    // are then formed inside the loop instead of being hoisted out of it,
    // which exhausts the registers.
    int olane;
    asm volatile("v_mov_b32 %0, %1" : "=v"(olane) : "v"(lane));
    const int g = olane >> 4, l16 = olane & 15;
    const int pt = perm_col(16 * tb + 4 * (l16 & 3));

    // K h (hw = 0) or K dh (hw = 1) of the blocks (tb, cb), cb = 0, 1
    f32x4 kx[2];
    {
      const u16* xh = hw == 0 ? sm.u.t.hh : sm.u.t.dhh;
      const u16* xl = hw == 0 ? sm.u.t.hl : sm.u.t.dhl;
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) kx[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s_ = 0; s_ < K / 32; ++s_) {
        const bf16x8 a = lds8(&sm.Kc[swz<K>(16 * tb + l16, 32 * s_ + 8 * g)]);
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          const int off = swz<K>(16 * cb + l16, 32 * s_ + 8 * g);
          kx[cb] = mfma16x16x32(a, lds8(xh + off), kx[cb]);
          kx[cb] = mfma16x16x32(a, lds8(xl + off), kx[cb]);
        }
      }
    }
    f32x4 vv[2];
    const f32x4 bt = ld4(&sm.gt.beta[16 * tb + 4 * g]), b1 = ld4(&sm.gt.bEGx[16 * tb + 4 * g]);
    if (hw == 0) {  // R = diag(beta) V - diag(b1) K h
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        vv[cb] = tr4<VT>(sm.u.t.Vt, 16 * tb, 16 * cb + 4 * (l16 & 3), g, l16);
        put_split4(sm.u.t.Rh, sm.u.t.Rl, swz<64>(16 * cb + l16, perm_col(16 * tb + 4 * g)), bt * vv[cb] - b1 * kx[cb]);
      }
    }
    __syncthreads();
    if (jt + 1 < NTILE) fetch_dh(jt + 1);
    if (hw == 0) {  // Ubar = Tinv R (Tinv[t][s] = 0 for s > t)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        f32x4 u{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s_ = 0; s_ < 2; ++s_) {
          if (s_ == 1 && tb < 2) continue;
          const int ao = swz<64>(16 * tb + l16, 32 * s_ + 8 * g), bo = swz<64>(16 * cb + l16, 32 * s_ + 8 * g);
          u = mma3(lds8(&sm.Th[ao]), lds8(&sm.Tl[ao]), lds8(&sm.u.t.Rh[bo]), lds8(&sm.u.t.Rl[bo]), u);
        }
        put_split4(sm.u.t.Uh, sm.u.t.Ul, swz<64>(16 * cb + l16, perm_col(16 * tb + 4 * g)), u);
      }
    } else {  // dUbar = diag(e^(Gn - G)) K dh + P^T dO (P[t'][t] = 0 for t' < t)
      const f32x4 en = ld4(&sm.gt.EGnG[16 * tb + 4 * g]);
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        f32x4 du = en * kx[cb];
#pragma unroll
        for (int s_ = 0; s_ < 2; ++s_) {
          if (s_ == 0 && tb >= 2) continue;
          const bf16x8 o = tr_frag<VT>(sm.u.t.dO, 32 * s_, perm_col(16 * cb + 4 * (l16 & 3)), g, l16);
          du = mfma16x16x32(tr_frag<64>(sm.Ph, 32 * s_, pt, g, l16), o, du);
          du = mfma16x16x32(tr_frag<64>(sm.Pl, 32 * s_, pt, g, l16), o, du);
        }
        put_split4(sm.u.t.dUh, sm.u.t.dUl, swz<64>(16 * cb + l16, perm_col(16 * tb + 4 * g)), du);
      }
    }
    __syncthreads();
    if (jt + 1 < NTILE) fetch_ov(jt + 1);
    if (hw == 0) {  // dR = Tinv^T dUbar, dv = beta dR, and the channel sums of dR
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        f32x4 dr{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s_ = 0; s_ < 2; ++s_) {
          if (s_ == 0 && tb >= 2) continue;
          const int bo = swz<64>(16 * cb + l16, 32 * s_ + 8 * g);
          dr = mma3(tr_frag<64>(sm.Th, 32 * s_, pt, g, l16), tr_frag<64>(sm.Tl, 32 * s_, pt, g, l16),
                    lds8(&sm.u.t.dUh[bo]), lds8(&sm.u.t.dUl[bo]), dr);
        }
        put_split4(sm.u.t.dRh, sm.u.t.dRl, swz<64>(16 * cb + l16, perm_col(16 * tb + 4 * g)), dr);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(bt[i] * dr[i]), dvrsrc,
                                                ((16 * tb + 4 * g + i) * H * V + v0 + 16 * cb + l16) * 4, 0, 0);
        sbR += dr * (vv[cb] - eGx * kx[cb]);
        sKhdR += kx[cb] * dr;
      }
    } else {  // (K dh) . Ubar over the channels
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const int off = swz<64>(16 * cb + l16, perm_col(16 * tb + 4 * g));
        const f32x4 u = unpack4(*reinterpret_cast<const u32x2*>(&sm.u.t.Uh[off])) +
                        unpack4(*reinterpret_cast<const u32x2*>(&sm.u.t.Ul[off]));
        st2 += kx[cb] * u;
      }
    }
    __syncthreads();
    // accumulators over the tile's 32 channels
    {
      const bf16x8 aO = lds8(&sm.u.t.dO[swz<VT>(16 * tb + l16, 8 * g)]);
      const bf16x8 aUh = tr_frag<64>(sm.u.t.Uh, 0, pt, g, l16), aUl = tr_frag<64>(sm.u.t.Ul, 0, pt, g, l16);
      const bf16x8 aRh = tr_frag<64>(sm.u.t.dRh, 0, pt, g, l16), aRl = tr_frag<64>(sm.u.t.dRl, 0, pt, g, l16);
#pragma unroll
      for (int cc = 0; cc < KBW; ++cc) {
        const int pk = perm_col(16 * (KBW * hw + cc) + 4 * (l16 & 3));
        const bf16x8 bh = tr_frag<K>(sm.u.t.hh, 0, pk, g, l16), bl = tr_frag<K>(sm.u.t.hl, 0, pk, g, l16);
        const bf16x8 dh_h = tr_frag<K>(sm.u.t.dhh, 0, pk, g, l16), dh_l = tr_frag<K>(sm.u.t.dhl, 0, pk, g, l16);
        accQ[cc] = mfma16x16x32(aO, bh, accQ[cc]);
        accQ[cc] = mfma16x16x32(aO, bl, accQ[cc]);
        accUd[cc] = mma3(aUh, aUl, dh_h, dh_l, accUd[cc]);
        accRh[cc] = mma3(aRh, aRl, bh, bl, accRh[cc]);
      }
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        if (2 * hw + cc > tb) continue;  // blocks above the diagonal are masked to zero
        const int ps = perm_col(16 * (2 * hw + cc) + 4 * (l16 & 3));
        const bf16x8 uh = tr_frag<64>(sm.u.t.Uh, 0, ps, g, l16), ul = tr_frag<64>(sm.u.t.Ul, 0, ps, g, l16);
        accA[cc] = mma3(aRh, aRl, uh, ul, accA[cc]);  // dR Ubar^T (dA is its negative)
        accP[cc] = mfma16x16x32(aO, uh, accP[cc]);
        accP[cc] = mfma16x16x32(aO, ul, accP[cc]);
      }
    }
  }
  __syncthreads();

  // q~_t . (dO h^T)_t summed over this wave's keys; q~ = q - d k from the bf16 tiles
  f32x4 kv[KBW];
  f32x4 x{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int cc = 0; cc < KBW; ++cc) {
    const int pk = perm_col(16 * (KBW * hw + cc) + 4 * (l16 & 3));
    kv[cc] = tr4<K>(sm.Kc, 16 * tb, pk, g, l16);
    x += (tr4<K>(sm.Qc, 16 * tb, pk, g, l16) - dd_ * kv[cc]) * accQ[cc];
  }
  // Sums over the 16 lanes (channels or keys) of each row group, eight per
  // wavefront in one DPP reduce-scatter: value j ends in lanes 2 j, 2 j + 1 of
  // the group. hw = 0: sbR, sKhdR, then x alone; hw = 1: st2 and x.
  {
    float v8[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v8[i] = hw == 0 ? sbR[i] : st2[i];
      v8[4 + i] = hw == 0 ? sKhdR[i] : x[i];
    }
    const float sum = group_sums_scatter<16>(v8, lane);
    const int j = l16 >> 1;
    if ((l16 & 1) == 0) sm.vec[hw == 0 ? 1 + (j >> 2) : (j < 4 ? 3 : 9)][16 * tb + 4 * g + (j & 3)] = sum;
    if (hw == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) v8[i] = x[i];
      halve_dpp<3, 2>(v8, lane);
      halve_dpp<2, 1>(v8, lane);
      const float r = v8[0] + dpp_flip<1>(v8[0]);
      const float sx = r + dpp_flip<0>(r);  // value (l16 >> 2) of x
      if ((l16 & 3) == 0) sm.vec[8][16 * tb + 4 * g + (l16 >> 2)] = sx;
    }
  }
  shdh = wave_sum(shdh);
  if (lane == 0) sm.red[wave] = shdh;
  // k_t.k_s of the blocks (tb, 2 hw + cc) from the exact bf16 k tile
  f32x4 kkv[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int s_ = 0; s_ < K / 32; ++s_) {
    const bf16x8 a = lds8(&sm.Kc[swz<K>(16 * tb + l16, 32 * s_ + 8 * g)]);
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
      kkv[cc] = mfma16x16x32(a, lds8(&sm.Kc[swz<K>(16 * (2 * hw + cc) + l16, 32 * s_ + 8 * g)]), kkv[cc]);
  }
  // masks and elementwise products of the 64 x 64 blocks (tb, 2 hw + cc):
  // dP (.) M and beta W as hi / lo bf16 for the products below, dP (.) P and
  // W (.) k_t.k_s in fp32 for the rectangle sums
  const f32x4 Gt = ld4(&sm.gt.G[16 * tb + 4 * g]), Gxt = ld4(&sm.gt.Gx[16 * tb + 4 * g]);
  const f32x4 btt = ld4(&sm.gt.beta[16 * tb + 4 * g]);
#pragma unroll
  for (int cc = 0; cc < 2; ++cc) {
    const int s_ = 16 * (2 * hw + cc) + l16;
    // P[t][s] from its hi / lo parts (about 16 significant bits)
    const int ps = perm_col(16 * (2 * hw + cc) + 4 * (l16 & 3));
    const f32x4 pv = tr4<64>(sm.Ph, 16 * tb, ps, g, l16) + tr4<64>(sm.Pl, 16 * tb, ps, g, l16);
    const float Gs = sm.gt.G[s_];
    f32x4 dpm, wb;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * tb + 4 * g + i;
      const float M = s_ <= t ? __expf(fminf(Gt[i] - Gs, 0.f)) : 0.f;
      const float E = s_ < t ? __expf(fminf(Gxt[i] - Gs, 0.f)) : 0.f;
      const float dpv = s_ <= t ? accP[cc][i] : 0.f, dav = s_ < t ? -accA[cc][i] : 0.f;
      const float w = dav * E;
      sm.u.p.dPP[t][s_] = dpv * pv[i];
      sm.u.p.Z[t][s_] = w * kkv[cc][i];
      dpm[i] = dpv * M;
      wb[i] = btt[i] * w;
    }
    const int off = swz<64>(s_, perm_col(16 * tb + 4 * g));
    put_split4(sm.u.p.dPMh, sm.u.p.dPMl, off, dpm);
    put_split4(sm.u.p.WBh, sm.u.p.WBl, off, wb);
  }
  __syncthreads();
  // first pass of the rectangle sums (threads 0-127; the products below do not read these tiles)
  rect_row_prefix(sm.u.p.dPP, sm.u.p.Z, sm.gt.beta, sm.vec, tid);
  // dq, dk of the blocks (tb, KBW hw + cc):
  //   dq = diag(e^G) dO h^T + (dP (.) M) K
  //   dk = diag(e^(Gn - G)) Ubar dh^T - diag(b1) dR h^T + diag(beta) W K + (dP (.) M)^T q
  //        + W^T diag(beta) K - d (dP (.) M)^T k - d dq
  const f32x4 eg = ld4(&sm.gt.EG[16 * tb + 4 * g]), en = ld4(&sm.gt.EGnG[16 * tb + 4 * g]);
  const f32x4 b1 = ld4(&sm.gt.bEGx[16 * tb + 4 * g]);
  f32x4 xq[KBW], xk[KBW], xd[KBW];
#pragma unroll
  for (int cc = 0; cc < KBW; ++cc) {
    xq[cc] = eg * accQ[cc];
    xk[cc] = en * accUd[cc] - b1 * accRh[cc];
    xd[cc] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // dq first, so that its stores drain while the dk products run
#pragma unroll
  for (int s_ = 0; s_ < 2; ++s_) {
    if (s_ == 1 && tb < 2) continue;  // columns s <= t
    const bf16x8 mh = tr_frag<64>(sm.u.p.dPMh, 32 * s_, pt, g, l16), ml = tr_frag<64>(sm.u.p.dPMl, 32 * s_, pt, g, l16);
#pragma unroll
    for (int cc = 0; cc < KBW; ++cc) {
      const bf16x8 bk = tr_frag<K>(sm.Kc, 32 * s_, perm_col(16 * (KBW * hw + cc) + 4 * (l16 & 3)), g, l16);
      xq[cc] = mfma16x16x32(mh, bk, xq[cc]);
      xq[cc] = mfma16x16x32(ml, bk, xq[cc]);
    }
  }
  float ddp = 0.f;
  const __amdgpu_buffer_rsrc_t dqrsrc = rows_rsrc(dq + tok0 * K, static_cast<int64_t>(nrows) * H * K * 4);
  const __amdgpu_buffer_rsrc_t dkrsrc = rows_rsrc(dk + tok0 * K, static_cast<int64_t>(nrows) * H * K * 4);
#pragma unroll
  for (int cc = 0; cc < KBW; ++cc) {
    ddp -= hsum(xq[cc] * kv[cc]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(xq[cc][i]), dqrsrc,
                                            ((16 * tb + 4 * g + i) * H * K + 16 * (KBW * hw + cc) + l16) * 4, 0, 0);
  }
#pragma unroll
  for (int s_ = 0; s_ < 2; ++s_) {
    if (s_ == 1 && tb < 2) continue;  // columns s <= t
    const bf16x8 wh = tr_frag<64>(sm.u.p.WBh, 32 * s_, pt, g, l16), wl = tr_frag<64>(sm.u.p.WBl, 32 * s_, pt, g, l16);
#pragma unroll
    for (int cc = 0; cc < KBW; ++cc) {
      const bf16x8 bk = tr_frag<K>(sm.Kc, 32 * s_, perm_col(16 * (KBW * hw + cc) + 4 * (l16 & 3)), g, l16);
      xk[cc] = mfma16x16x32(wh, bk, xk[cc]);
      xk[cc] = mfma16x16x32(wl, bk, xk[cc]);
    }
  }
#pragma unroll
  for (int s_ = 0; s_ < 2; ++s_) {
    if (s_ == 0 && tb >= 2) continue;  // rows t' >= t
    const int ao = swz<64>(16 * tb + l16, 32 * s_ + 8 * g);
    const bf16x8 mh = lds8(&sm.u.p.dPMh[ao]), ml = lds8(&sm.u.p.dPMl[ao]);
    const bf16x8 wh = lds8(&sm.u.p.WBh[ao]), wl = lds8(&sm.u.p.WBl[ao]);
#pragma unroll
    for (int cc = 0; cc < KBW; ++cc) {
      const int pk = perm_col(16 * (KBW * hw + cc) + 4 * (l16 & 3));
      const bf16x8 bq = tr_frag<K>(sm.Qc, 32 * s_, pk, g, l16), bk = tr_frag<K>(sm.Kc, 32 * s_, pk, g, l16);
      xk[cc] = mfma16x16x32(mh, bq, xk[cc]);
      xk[cc] = mfma16x16x32(ml, bq, xk[cc]);
      xk[cc] = mfma16x16x32(wh, bk, xk[cc]);
      xk[cc] = mfma16x16x32(wl, bk, xk[cc]);
      xd[cc] = mfma16x16x32(mh, bk, xd[cc]);
      xd[cc] = mfma16x16x32(ml, bk, xd[cc]);
    }
  }
#pragma unroll
  for (int cc = 0; cc < KBW; ++cc) {
    xk[cc] -= dd_ * (xd[cc] + xq[cc]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(xk[cc][i]), dkrsrc,
                                            ((16 * tb + 4 * g + i) * H * K + 16 * (KBW * hw + cc) + l16) * 4, 0, 0);
  }
  ddp = wave_sum(ddp);
  __syncthreads();
  if (lane == 0) sm.red[8 + wave] = ddp;
  rect_column_sums(sm.u.p.dPP, sm.u.p.Z, sm.vec, tid);
  __syncthreads();
  if (wave == 0) grad_scalars(sm.gt, sm.vec, sm.red, lane, nrows, tok0, H, dalpha, dbeta, dd_part + slot * H + h);
}

// dd per head: one 64-thread block per head sums the chunks in a fixed order
// (strided partial sums, then a fixed butterfly).
__global__ __launch_bounds__(64) void dd_reduce_kernel(const float* __restrict__ dd_part, int64_t nslots, int H,
                                                       float* __restrict__ dd) {
  const int h = blockIdx.x, lane = threadIdx.x;
  float s = 0.f;
  for (int64_t i = lane; i < nslots; i += 64) s += dd_part[i * H + h];
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) s += __shfl_xor(s, m, kWave);
  if (lane == 0) dd[h] = s;
}

template <int K, int V, typename InT>
hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t st) {
  const bool packed = a.cu_seqlens != nullptr;
  const int64_t nslots = chunk_slots(packed, a.B, a.T, a.N);
  const unsigned grid = static_cast<unsigned>(nslots * a.H);
  chunk_bwd_prep_kernel<K, InT><<<grid, 256, 0, st>>>(
      static_cast<const InT*>(a.q), static_cast<const InT*>(a.k), a.alpha, a.beta, a.d, a.cu_seqlens, a.T, a.H, a.N,
      nslots, a.Tg, a.Pg, a.KKg, a.Gg);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if constexpr (sizeof(InT) == 2) {
    chunk_bwd_dh_pc_kernel<K, V><<<xcd_grid(a.N * a.H, V / kDhbVT), 512, 0, st>>>(
        static_cast<const u16*>(a.q), static_cast<const u16*>(a.k), a.d, static_cast<const u16*>(a.dO),
        a.cu_seqlens, a.T, a.H, a.N, a.Tg, a.Pg, a.Gg, a.dsf, a.dhck, a.ds0);
  } else {
    chunk_bwd_dh_kernel<K, V, InT><<<xcd_grid(a.N * a.H, V / kDhVT), 512, 0, st>>>(
        static_cast<const InT*>(a.q), static_cast<const InT*>(a.k), a.d, static_cast<const InT*>(a.dO),
        a.cu_seqlens, a.T, a.H, a.N, a.Tg, a.Pg, a.Gg, a.dsf, a.dhck, a.ds0);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if constexpr (sizeof(InT) == 2) {
    chunk_bwd_grad_bf16_kernel<K, V><<<grid, 512, 0, st>>>(
        static_cast<const u16*>(a.q), static_cast<const u16*>(a.k), static_cast<const u16*>(a.v), a.d,
        static_cast<const u16*>(a.dO), a.cu_seqlens, a.T, a.H, a.N, nslots, a.hck, a.dhck, a.Tg, a.Pg, a.Gg,
        a.dq, a.dk, a.dv, a.dalpha, a.dbeta, a.dd_part);
  } else {
    chunk_bwd_grad_kernel<K, V, InT><<<grid, 512, 0, st>>>(
        static_cast<const InT*>(a.q), static_cast<const InT*>(a.k), static_cast<const InT*>(a.v), a.d,
        static_cast<const InT*>(a.dO), a.cu_seqlens, a.T, a.H, a.N, nslots, a.hck, a.dhck, a.Tg, a.Pg, a.KKg, a.Gg,
        a.dq, a.dk, a.dv, a.dalpha, a.dbeta, a.dd_part);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  dd_reduce_kernel<<<a.H, 64, 0, st>>>(a.dd_part, nslots, a.H, a.dd);
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
