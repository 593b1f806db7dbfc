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

// Wavefront-wide inclusive prefix sum.
__device__ __forceinline__ float wave_inclusive_scan(float x, int lane) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    float y = __shfl_up(x, off, kWave);
    if (lane >= off) x += y;
  }
  return x;
}

// The same in double.
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
