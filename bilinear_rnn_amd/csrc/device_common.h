// Device helpers shared by the Comba kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace comba {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16;

constexpr int kChunk = 64;      // tokens per chunk
constexpr int kWave = 64;       // CDNA wavefront width

__device__ __forceinline__ float bf16_bits_to_float(u16 b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even (hardware v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ __bf16 to_bf16(float x) { return static_cast<__bf16>(x); }

__device__ __forceinline__ u16 float_to_bf16_bits(float x) {
  __bf16 b = to_bf16(x);
  return __builtin_bit_cast(u16, b);
}

// Input-side fusion flags (the COMBA_FUSE_* values of comba.h).
constexpr unsigned kFuseGateLogits = 1u, kFuseQkL2Norm = 2u;
constexpr float kL2NormEps = 1e-6f;  // x / sqrt(sum x^2 + eps)

// sigmoid(x) = 1 / (1 + e^-x) without overflow: e^-|x| is at most 1, and the
// two branches are the two algebraic forms of the same value.
__device__ __forceinline__ float sigmoid_stable(float x) {
  const float e = expf(-fabsf(x));
  return x >= 0.f ? 1.f / (1.f + e) : e / (1.f + e);
}

// x ~= hi + lo with hi = bf16(x), lo = bf16(x - hi): about 16 significant bits.
__device__ __forceinline__ void split_bf16(float x, __bf16& hi, __bf16& lo) {
  hi = to_bf16(x);
  lo = to_bf16(x - static_cast<float>(hi));
}

// D = A(16x32) * B(32x16) + C on the matrix cores, bf16 inputs, fp32 accumulate.
// Lane l holds A row (l % 16), B column (l % 16), 8 reduction elements each
// (the same 8 positions of the reduction axis in A and B), and D rows
// 4 * (l / 16) + 0..3 of column (l % 16).
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Column order used for matrix-core operands in LDS. Within each group of 32
// reduction indices, index p is stored at position perm32(p) so that the
// 8 values a lane needs are contiguous: lane group g (= lane / 16) covers
// p = 4g..4g+3 and p = 16+4g..16+4g+3, which is exactly the set of rows an
// fp32 accumulator pair (rows 16*m + 4g + i, m = 0, 1) holds in one lane.
__host__ __device__ constexpr int perm32(int p) {
  return p < 16 ? 8 * (p >> 2) + (p & 3) : 8 * ((p - 16) >> 2) + 4 + (p & 3);
}
__host__ __device__ constexpr int perm_col(int c) { return (c & ~31) | perm32(c & 31); }

// x summed over the 16 lanes of each DPP row, result in all 16 lanes:
// swap neighbours, swap pairs, mirror the 8-lane halves, mirror the row.
__device__ __forceinline__ float row16_sum(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xb1, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4e, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x141, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x140, 0xf, 0xf, false));
  return x;
}

// x summed over the wavefront, the same value in every lane: the sums of the
// four DPP rows, then those four read lane by lane.
__device__ __forceinline__ float wave_sum(float x) {
  x = row16_sum(x);
  auto at = [&](int l) { return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l)); };
  return (at(0) + at(16)) + (at(32) + at(48));
}

// Value of the lane whose position in the group differs in bit B (the lane
// mirrored within its 16, 8 or 4 lanes, or its neighbour): DPP row_mirror,
// row_half_mirror, quad_perm [2,3,0,1], quad_perm [1,0,3,2].
template <int B>
__device__ __forceinline__ float dpp_flip(float x) {
  constexpr int ctrl = B == 3 ? 0x140 : B == 2 ? 0x141 : B == 1 ? 0x4e : 0xb1;
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), ctrl, 0xf, 0xf, false));
}

// One reduce-scatter step over lane bit B: lanes with the bit clear keep the
// lower N of their 2N partial sums, lanes with it set the upper N, and each
// adds the partner lane's copy of the half it keeps.
template <int B, int N>
__device__ __forceinline__ void halve_dpp(float* v, int lane) {
  const bool hi = (lane >> B) & 1;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const float keep = hi ? v[i + N] : v[i], send = hi ? v[i] : v[i + N];
    v[i] = keep + dpp_flip<B>(send);
  }
}

// Sums each of L values v[0 .. L/2 - 1] over its group of L consecutive lanes
// (L = 16 or 8). Returns in every lane one complete sum: that of value
// (lane >> 1) & (L/2 - 1), the same in both lanes of a pair.
template <int L>
__device__ __forceinline__ float group_sums_scatter(float* v, int lane) {
  if constexpr (L == 16) {
    halve_dpp<3, 4>(v, lane);
    halve_dpp<2, 2>(v, lane);
    halve_dpp<1, 1>(v, lane);
  } else {
    static_assert(L == 8, "groups of 16 or 8 lanes");
    halve_dpp<2, 2>(v, lane);
    halve_dpp<1, 1>(v, lane);
  }
  return v[0] + dpp_flip<0>(v[0]);
}

// x += (x moved by the DPP control CTRL); lanes without a source add 0.
#define COMBA_DPP_ADD(x, CTRL, ROWMASK, BOUND)                                                        \
  (x) += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, (x)), CTRL, \
                                                               ROWMASK, 0xf, BOUND))

// Wavefront inclusive prefix sum: shifts by 1, 2, 4, 8 inside each row of 16
// lanes, then the last lane of row 0 / 2 into rows 1 / 3, then lane 31 into
// rows 2 and 3.
__device__ __forceinline__ float wave_scan_dpp(float x) {
  COMBA_DPP_ADD(x, 0x111, 0xf, true);  // row_shr:1
  COMBA_DPP_ADD(x, 0x112, 0xf, true);  // row_shr:2
  COMBA_DPP_ADD(x, 0x114, 0xf, true);  // row_shr:4
  COMBA_DPP_ADD(x, 0x118, 0xf, true);  // row_shr:8
  COMBA_DPP_ADD(x, 0x142, 0xa, false); // row_bcast:15 into rows 1, 3
  COMBA_DPP_ADD(x, 0x143, 0xc, false); // row_bcast:31 into rows 2, 3
  return x;
}

// Wavefront inclusive suffix sum (lane t: the sum over lanes t .. 63): shifts
// by 1, 2, 4, 8 towards lane 0 inside each row of 16 lanes, then the totals of
// the rows above (read from their first lanes) added.
__device__ __forceinline__ float wave_suffix_scan_dpp(float x) {
  COMBA_DPP_ADD(x, 0x101, 0xf, true);  // row_shl:1
  COMBA_DPP_ADD(x, 0x102, 0xf, true);  // row_shl:2
  COMBA_DPP_ADD(x, 0x104, 0xf, true);  // row_shl:4
  COMBA_DPP_ADD(x, 0x108, 0xf, true);  // row_shl:8
  auto at = [&](int l) { return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l)); };
  const float r3 = at(48), r23 = at(32) + r3, r123 = at(16) + r23;
  const int row = static_cast<int>(__lane_id()) >> 4;
  return x + (row == 0 ? r123 : row == 1 ? r23 : row == 2 ? r3 : 0.f);
}

// Value of the next lower (wave_shr:1) or next higher (wave_shl:1) lane of the
// wavefront; lane 0, respectively lane 63, reads 0.
__device__ __forceinline__ float wave_from_lower(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x138, 0xf, 0xf, true));
}
__device__ __forceinline__ float wave_from_higher(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x130, 0xf, 0xf, true));
}

// Wavefront-wide inclusive prefix sum in double.
__device__ __forceinline__ double wave_inclusive_scan_f64(double x, int lane) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    double y = __shfl_up(x, off, kWave);
    if (lane >= off) x += y;
  }
  return x;
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ static float load(const float* p, int64_t i) { return p[i]; }
  __device__ static void store(float* p, int64_t i, float x) { p[i] = x; }
};
template <> struct Elem<u16> {
  __device__ static float load(const u16* p, int64_t i) { return bf16_bits_to_float(p[i]); }
  __device__ static void store(u16* p, int64_t i, float x) { p[i] = float_to_bf16_bits(x); }
};

// Token range [t0, t1) and batch row of sequence n. Garbage cu_seqlens is
// clamped to [0, T] so that no access leaves the tensors.
__device__ __forceinline__ void sequence_range(const int32_t* cu_seqlens, int n, int T,
                                               int& b, int& t0, int& t1) {
  if (cu_seqlens) {
    b = 0;
    int a = cu_seqlens[n], e = cu_seqlens[n + 1];
    a = a < 0 ? 0 : (a > T ? T : a);
    e = e < a ? a : (e > T ? T : e);
    t0 = a;
    t1 = e;
  } else {
    b = n;
    t0 = 0;
    t1 = T;
  }
}

}  // namespace comba
