// Kernel launchers behind the C ABI. Arguments are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace comba {

// Library-internal modes of the chunk kernels, in FwdArgs::fusion above the
// COMBA_FUSE_* bits (callers can never set them), used by the segment-parallel
// forward: v read as zeros, no output written, initial state the identity
// (then V == K).
constexpr unsigned kModeZeroV = 1u << 16, kModeNoOutput = 1u << 17, kModeIdentityInit = 1u << 18;

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* alpha;
  const float* beta;
  const float* d;
  const float* s0;            // may be null
  const int32_t* cu_seqlens;  // may be null
  const int32_t* order;       // longest-first sequence order, may be null
  int N, B, T, H, K, V;
  int Hk;                     // q / k heads (H % Hk == 0): value head h reads q / k head h / (H / Hk)
  int in_dtype, out_dtype;    // COMBA_BF16 / COMBA_FP32
  void* o;
  float* sf;                  // may be null
  unsigned fusion;            // COMBA_FUSE_* flags | kMode* bits
  float* hck = nullptr;       // incoming state of every chunk, [slots, H, V, K] (backward); may be null
};

// Index of chunk c of sequence n (first token t0) in per-chunk buffers: n * ceil(T / 64) + c
// for fixed-length batches; t0 / 64 + n + c for packed ones (unique because sequence starts
// increase), fewer than T / 64 + N + 1 slots in all.
__host__ __device__ inline int64_t chunk_slot(bool packed, int t0, int n, int c, int T) {
  return packed ? static_cast<int64_t>(t0 / 64) + n + c : static_cast<int64_t>(n) * ((T + 63) / 64) + c;
}
__host__ __device__ inline int64_t chunk_slots(bool packed, int B, int T, int N) {
  return packed ? static_cast<int64_t>(T / 64) + N + 1 : static_cast<int64_t>(B) * ((T + 63) / 64);
}

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* alpha;
  const float* beta;
  const float* d;
  const void* dO;             // dL/do, in_dtype, [B, T, H, V]
  const int32_t* cu_seqlens;  // may be null
  int N, B, T, H, K, V;
  int in_dtype;               // COMBA_BF16 / COMBA_FP32
  const float* dsf;           // dL/dS_final [N, H, V, K], may be null
  float* hck;                 // chunk incoming states [slots, H, V, K] (from the forward pass)
  float* dhck;                // chunk outgoing-state gradients [slots, H, V, K]
  float* dd_part;             // [slots, H]
  float* Tg;                  // per chunk and head: Tinv, P and (fp32 inputs) k_t.k_s, fp32 64 x 64 each
  float* Pg;
  float* KKg;                 // written and read for fp32 inputs only
  float* Gg;                  // per chunk and head: the chunk's decay gates, fp32 7 x 64 (see ChunkGates)
  float* dq;                  // [B, T, H, K] fp32
  float* dk;
  float* dv;                  // [B, T, H, V] fp32
  float* dalpha;              // [B, T, H] fp32
  float* dbeta;
  float* dd;                  // [H] fp32
  float* ds0;                 // [N, H, V, K] fp32, may be null
};

hipError_t launch_recurrent(const FwdArgs& a, hipStream_t st);
hipError_t launch_chunk_bwd(const BwdArgs& a, hipStream_t st);
hipError_t launch_chunk_bf16(const FwdArgs& a, hipStream_t st);
// State-only pass over bf16 inputs (K == V) that writes the final states from
// a.s0 == null to a.sf and, from the identity with v = 0, the K x K maps to sf2.
hipError_t launch_chunk_bf16_pair(const FwdArgs& a, float* sf2, hipStream_t st);
hipError_t launch_chunk_fp32(const FwdArgs& a, hipStream_t st);
hipError_t launch_varlen_order(const int32_t* cu_seqlens, int N, int32_t* order, hipStream_t st);
hipError_t launch_check_inputs(const float* alpha, int64_t n_alpha, const int32_t* cu_seqlens, int N, int T,
                               uint32_t* flags, hipStream_t st);
hipError_t launch_segment_bounds(int B, int T, int L, int S, int32_t* cu, hipStream_t st);
hipError_t launch_segment_scan(const float* s0, const float* bst, const float* phi, float* X, float* sf, int B,
                               int H, int K, int V, int S, hipStream_t st);

// Grid for work units of NVT tiles each, dealt round-robin over the 8 XCDs so
// that the tiles of one unit run on the same XCD (and share its L2).
inline int xcd_grid(int units, int nvt) { return ((units + 7) / 8) * 8 * nvt; }

}  // namespace comba
