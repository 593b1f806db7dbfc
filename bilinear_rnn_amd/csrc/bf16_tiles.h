// bf16 tiles in LDS and matrix-core operands built from them (gfx950 / CDNA4),
// shared by the chunk forward and the chunk backward.
//
// Precision scheme: an fp32 operand x enters a bf16 product as hi = bf16(x)
// and lo = bf16(x - hi), about 16 significant bits; the products hi*hi +
// hi*lo + lo*hi (or hi + lo against an exact bf16 operand) accumulate in fp32.
//
// Fragment orders of a 16x16x32 bf16 MFMA (lane l, g = l / 16, l16 = l % 16):
// the lane supplies row l16 of A and column l16 of B with eight reduction
// indices, the same eight on both sides; the accumulator holds rows 4 g + i
// of column l16. Two orders of the eight indices of a 32-block are used:
//   - "row" fragments read 8 consecutive positions 8 g .. 8 g + 7 of a tile row
//     whose 32-blocks are stored in perm32 order (device_common.h): logical
//     indices {4 g .. 4 g + 3, 16 + 4 g .. 16 + 4 g + 3};
//   - "transposed" fragments read the same logical indices down the rows of a
//     row-major tile with the transposing LDS read (ds_read_b64_tr_b16).
// Either kind can therefore pair with the other.
#pragma once

#include "device_common.h"

namespace comba {

typedef short s4 __attribute__((ext_vector_type(4)));
typedef short s8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s4 lds_s4;

// Third descriptor word of a raw buffer resource on gfx9-family parts
// (32-bit data format, no swizzle): with stride 0, an access at or beyond
// num_records bytes is dropped (stores) or returns zero (loads).
constexpr int kBufferWord3 = 0x00020000;

// A wave-uniform pointer held in scalar registers (the value of lane 0): a
// buffer resource built from it needs no per-lane waterfall loop.
template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
  return reinterpret_cast<T*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Row-major tile of L bf16 per row: 16-byte chunk c of row r is stored at
// chunk c ^ s(r). For L = 64 and 32, s(r) = r mod L/8. For L = 128 (one row per
// 256 bytes) s maps row bits 0, 1, 2 to chunk bits {1}, {2}, {0, 3}: measured
// with the LDS bank-conflict counter on gfx950, the 16-byte fragment reads of 16
// consecutive rows are conflict-free with either, and the transposing reads of
// four consecutive rows at four consecutive 8-byte pieces are two-way with this
// one against four-way with r mod 16.
template <int L>
__device__ __forceinline__ int swz(int row, int pos) {
  constexpr int mask = L / 8 - 1;
  const int s = L == 128 ? ((row & 3) << 1) ^ (9 * ((row >> 2) & 1)) : row & mask;
  return row * L + (((pos >> 3) ^ s) << 3) + (pos & 7);
}

__device__ __forceinline__ bf16x8 lds8(const u16* p) { return *reinterpret_cast<const bf16x8*>(p); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// hi / lo bf16 split of two floats, packed: hi = round-to-nearest bf16 pair
// (one v_cvt_pk_bf16_f32), its exact fp32 values by shift and mask, lo = the
// rounded remainders (a second conversion). Three VALU instructions per value.
__device__ __forceinline__ void split2(float x0, float x1, unsigned& hi, unsigned& lo) {
  const bf16x2 h = __builtin_convertvector((f32x2){x0, x1}, bf16x2);
  hi = __builtin_bit_cast(unsigned, h);
  const float h0 = __uint_as_float(hi << 16), h1 = __uint_as_float(hi & 0xffff0000u);
  const bf16x2 l = __builtin_convertvector((f32x2){x0 - h0, x1 - h1}, bf16x2);
  lo = __builtin_bit_cast(unsigned, l);
}

// Eight values (m0 then m1) as an MFMA operand pair.
__device__ __forceinline__ void split_pair(const f32x4& m0, const f32x4& m1, bf16x8& hi, bf16x8& lo) {
  unsigned h0, h1, h2, h3, l0, l1, l2, l3;
  split2(m0[0], m0[1], h0, l0);
  split2(m0[2], m0[3], h1, l1);
  split2(m1[0], m1[1], h2, l2);
  split2(m1[2], m1[3], h3, l3);
  hi = __builtin_bit_cast(bf16x8, (u32x4){h0, h1, h2, h3});
  lo = __builtin_bit_cast(bf16x8, (u32x4){l0, l1, l2, l3});
}

__device__ __forceinline__ void split4(const f32x4& x, s4& hi, s4& lo) {
  unsigned h0, h1, l0, l1;
  split2(x[0], x[1], h0, l0);
  split2(x[2], x[3], h1, l1);
  hi = __builtin_bit_cast(s4, (u32x2){h0, h1});
  lo = __builtin_bit_cast(s4, (u32x2){l0, l1});
}

// Split four fp32 values into hi / lo bf16 and write them as two 8-byte stores.
__device__ __forceinline__ void put_split4(u16* hi, u16* lo, int off, const f32x4& x) {
  unsigned h0, h1, l0, l1;
  split2(x[0], x[1], h0, l0);
  split2(x[2], x[3], h1, l1);
  *reinterpret_cast<u32x2*>(hi + off) = (u32x2){h0, h1};
  *reinterpret_cast<u32x2*>(lo + off) = (u32x2){l0, l1};
}

// hi + lo * (a*b + c) style triple product accumulate with both operands split.
__device__ __forceinline__ f32x4 mma3(const bf16x8& ah, const bf16x8& al, const bf16x8& bh, const bf16x8& bl,
                                      f32x4 acc) {
  acc = mfma16x16x32(ah, bh, acc);
  acc = mfma16x16x32(ah, bl, acc);
  acc = mfma16x16x32(al, bh, acc);
  return acc;
}

// Transposed fragment: this lane's index is a column of a row-major tile of L
// bf16 per row (swz<L> layout), its eight reduction indices are the rows
// row32 + {4 g .. 4 g + 3, 16 + 4 g .. 16 + 4 g + 3}. pos is the tile
// position of the four consecutive columns 4 (l16 % 4) .. + 3 of the lane's
// 16-column block (col0 + 4 (l16 % 4) in natural order, perm_col of it in
// perm32 order).
template <int L>
__device__ __forceinline__ bf16x8 tr_frag(const u16* tile, int row32, int pos, int g, int l16) {
  const int row0 = row32 + 4 * g + (l16 >> 2);
  const s4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(tile + swz<L>(row0, pos)));
  const s4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(tile + swz<L>(row0 + 16, pos)));
  // Whole-vector reinterpretation: element-wise short -> __bf16 casts of the
  // transposed-read result are folded into a splat of element 0 by this compiler.
  const s8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, both);
}

// Four values in accumulator order: the rows row16 + 4 g + i, i = 0..3, of
// this lane's column of a row-major tile of L bf16 per row, as floats; pos as
// for tr_frag.
template <int L>
__device__ __forceinline__ f32x4 tr4(const u16* tile, int row16, int pos, int g, int l16) {
  const int row = row16 + 4 * g + (l16 >> 2);
  const s4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(tile + swz<L>(row, pos)));
  const uint2 w = __builtin_bit_cast(uint2, x);  // whole-vector reinterpretation (see tr_frag)
  return f32x4{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u), __uint_as_float(w.y << 16),
               __uint_as_float(w.y & 0xffff0000u)};
}

}  // namespace comba
