// C ABI entry points (declared in include/comba.h): host-side validation,
// workspace carving and kernel launches on the caller's stream.
#include <atomic>
#include <climits>
#include <cstdio>
#include <mutex>
#include <string>

#include "comba.h"
#include "launch.h"
#include "measure.h"

#define COMBA_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local std::string g_last_error;

// Above this many packed sequences the longest-first order (quadratic in N)
// is skipped and sequences run in their given order.
constexpr int kMaxOrderedSeqs = 16384;

}  // namespace

// Device scratch of comba_chunk_fwd_noalloc: the longest-first order of up to
// kMaxOrderedSeqs packed sequences (64 KiB). Each GPU holds its own copy until
// the process ends, and every call on that GPU shares it. In host code this
// name is only a stand-in for the symbol: kernels and copies take the address
// that hipGetSymbolAddress returns for the device (scratch_on below).
__device__ __align__(256) int32_t scratch[kMaxOrderedSeqs];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int32_t*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

int32_t fail(int32_t code, const char* what) {
  g_last_error = what;
  return code;
}

size_t align_up(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

bool supported_dim(int32_t x) { return x == 64 || x == 128; }

// Common argument checks; fills a with everything but the workspace.
int32_t check_args(const void* q, const void* k, const void* v, const float* alpha, const float* beta,
                   const float* d, const float* s0, const int32_t* cu, int32_t num_seqs, int32_t B,
                   int32_t T, int32_t H, int32_t Hk, int32_t K, int32_t V, int32_t in_dtype, int32_t out_dtype,
                   void* o, float* sf, comba::FwdArgs& a) {
  if (!q || !k || !v || !alpha || !beta || !d || !o)
    return fail(COMBA_ERR_INVALID_ARG, "q, k, v, alpha, beta, d and o must be non-NULL");
  if ((in_dtype != COMBA_BF16 && in_dtype != COMBA_FP32) || (out_dtype != COMBA_BF16 && out_dtype != COMBA_FP32))
    return fail(COMBA_ERR_INVALID_ARG, "in_dtype and out_dtype must be COMBA_BF16 or COMBA_FP32");
  if (B < 1 || H < 1 || K < 1 || V < 1)
    return fail(COMBA_ERR_INVALID_ARG, "B, H, K and V must be >= 1");
  if (Hk < 1 || H % Hk != 0)
    return fail(COMBA_ERR_INVALID_ARG, "num_qk_heads must be >= 1 and divide H");
  if (cu) {
    if (B != 1) return fail(COMBA_ERR_INVALID_ARG, "cu_seqlens requires B == 1");
    if (num_seqs < 1) return fail(COMBA_ERR_INVALID_ARG, "cu_seqlens requires num_seqs >= 1");
    if (T < 0) return fail(COMBA_ERR_INVALID_ARG, "T must be >= 0");
  } else if (T < 1) {
    return fail(COMBA_ERR_INVALID_ARG, "T must be >= 1 without cu_seqlens");
  }
  if (!supported_dim(K) || !supported_dim(V))
    return fail(COMBA_ERR_UNSUPPORTED, "only K, V in {64, 128} are implemented");
  const int64_t N = cu ? num_seqs : B;
  if (N * H * 2 > INT_MAX / 16)
    return fail(COMBA_ERR_UNSUPPORTED, "too many (sequence, head) pairs for one launch");
  // Byte offsets inside one 64-token chunk, 64 * H * max(K, V) * 4 with fp32
  // rows, are 32-bit in the kernels.
  if (static_cast<int64_t>(H) * (K > V ? K : V) > (1 << 22))
    return fail(COMBA_ERR_UNSUPPORTED, "H * max(K, V) above 2^22 (chunk byte offsets must fit 31 bits)");
  if (s0 && sf && s0 != sf) {
    const char* s0b = reinterpret_cast<const char*>(s0);
    const char* sfb = reinterpret_cast<const char*>(sf);
    const int64_t bytes = N * H * V * K * 4;
    if (s0b < sfb + bytes && sfb < s0b + bytes)
      return fail(COMBA_ERR_INVALID_ARG, "final_state partially overlaps initial_state");
  }
  a = comba::FwdArgs{q, k, v, alpha, beta, d, s0, cu, nullptr, static_cast<int>(N), B, T, H, K, V, Hk,
                     in_dtype, out_dtype, o, sf, 0u};
  return COMBA_OK;
}

int32_t launched(hipError_t e) {
  if (e != hipSuccess) {
    g_last_error = std::string("HIP launch failed: ") + hipGetErrorString(e);
    return COMBA_ERR_HIP;
  }
  g_last_error.clear();
  return COMBA_OK;
}

}  // namespace

COMBA_API int32_t comba_abi_version(void) { return COMBA_ABI_VERSION; }

COMBA_API const char* comba_status_string(int32_t status) {
  switch (status) {
    case COMBA_OK: return "COMBA_OK";
    case COMBA_ERR_INVALID_ARG: return "COMBA_ERR_INVALID_ARG";
    case COMBA_ERR_UNSUPPORTED: return "COMBA_ERR_UNSUPPORTED";
    case COMBA_ERR_WORKSPACE: return "COMBA_ERR_WORKSPACE";
    case COMBA_ERR_HIP: return "COMBA_ERR_HIP";
    default: return "COMBA_ERR_UNKNOWN";
  }
}

COMBA_API const char* comba_last_error(void) { return g_last_error.c_str(); }

COMBA_API size_t comba_chunk_fwd_workspace_size(int32_t B, int32_t T, int32_t H, int32_t K, int32_t V,
                                                int32_t num_seqs, int32_t in_dtype) {
  (void)B; (void)T; (void)H; (void)K; (void)V; (void)in_dtype;
  if (num_seqs > 0 && num_seqs <= kMaxOrderedSeqs) return align_up(sizeof(int32_t) * num_seqs);
  return 0;
}

namespace {

constexpr uint32_t kKnownFusion = COMBA_FUSE_GATE_LOGITS | COMBA_FUSE_QK_L2NORM;

int32_t chunk_fwd_impl(const void* q, const void* k, const void* v, const float* alpha, const float* beta,
                       const float* d, const float* initial_state, const int32_t* cu_seqlens, int32_t num_seqs,
                       int32_t B, int32_t T, int32_t H, int32_t Hk, int32_t K, int32_t V, int32_t in_dtype,
                       int32_t out_dtype, void* o, float* final_state, void* workspace, size_t workspace_bytes,
                       uint32_t fusion, void* stream, float* chunk_states = nullptr) {
  if (fusion & ~kKnownFusion) return fail(COMBA_ERR_INVALID_ARG, "unknown bits in fusion");
  comba::FwdArgs a;
  int32_t rc = check_args(q, k, v, alpha, beta, d, initial_state, cu_seqlens, num_seqs, B, T, H, Hk, K, V,
                          in_dtype, out_dtype, o, final_state, a);
  if (rc != COMBA_OK) return rc;
  a.fusion = fusion;
  a.hck = chunk_states;
  const size_t need = comba_chunk_fwd_workspace_size(B, T, H, K, V, cu_seqlens ? num_seqs : 0, in_dtype);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(COMBA_ERR_WORKSPACE, "workspace is NULL or smaller than comba_chunk_fwd_workspace_size()");
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (cu_seqlens && need > 0) {
    int32_t* order = static_cast<int32_t*>(workspace);
    rc = launched(comba::launch_varlen_order(cu_seqlens, a.N, order, st));
    if (rc != COMBA_OK) return rc;
    a.order = order;
  }
  if (in_dtype == COMBA_BF16) return launched(comba::launch_chunk_bf16(a, st));
  return launched(comba::launch_chunk_fp32(a, st));
}

int32_t recurrent_impl(const void* q, const void* k, const void* v, const float* alpha, const float* beta,
                       const float* d, const float* initial_state, const int32_t* cu_seqlens, int32_t num_seqs,
                       int32_t B, int32_t T, int32_t H, int32_t Hk, int32_t K, int32_t V, int32_t in_dtype,
                       int32_t out_dtype, void* o, float* final_state, uint32_t fusion, void* stream) {
  if (fusion & ~kKnownFusion) return fail(COMBA_ERR_INVALID_ARG, "unknown bits in fusion");
  comba::FwdArgs a;
  int32_t rc = check_args(q, k, v, alpha, beta, d, initial_state, cu_seqlens, num_seqs, B, T, H, Hk, K, V,
                          in_dtype, out_dtype, o, final_state, a);
  if (rc != COMBA_OK) return rc;
  a.fusion = fusion;
  return launched(comba::launch_recurrent(a, static_cast<hipStream_t>(stream)));
}

}  // namespace

COMBA_API int32_t comba_chunk_fwd(const void* q, const void* k, const void* v, const float* alpha,
                                  const float* beta, const float* d, const float* initial_state,
                                  const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T,
                                  int32_t H, int32_t K, int32_t V, int32_t in_dtype, int32_t out_dtype,
                                  void* o, float* final_state, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  return chunk_fwd_impl(q, k, v, alpha, beta, d, initial_state, cu_seqlens, num_seqs, B, T, H, H, K, V, in_dtype,
                        out_dtype, o, final_state, workspace, workspace_bytes, 0u, stream);
}

COMBA_API int32_t comba_chunk_fwd_fused(const void* q, const void* k, const void* v, const float* alpha,
                                        const float* beta, const float* d, const float* initial_state,
                                        const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T,
                                        int32_t H, int32_t K, int32_t V, int32_t in_dtype, int32_t out_dtype,
                                        void* o, float* final_state, void* workspace, size_t workspace_bytes,
                                        uint32_t fusion, void* stream) {
  return chunk_fwd_impl(q, k, v, alpha, beta, d, initial_state, cu_seqlens, num_seqs, B, T, H, H, K, V, in_dtype,
                        out_dtype, o, final_state, workspace, workspace_bytes, fusion, stream);
}

COMBA_API int32_t comba_chunk_fwd_ex(const void* q, const void* k, const void* v, const float* alpha,
                                     const float* beta, const float* d, const float* initial_state,
                                     const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T, int32_t H,
                                     int32_t num_qk_heads, int32_t K, int32_t V, int32_t in_dtype,
                                     int32_t out_dtype, void* o, float* final_state, void* workspace,
                                     size_t workspace_bytes, uint32_t fusion, void* stream) {
  return chunk_fwd_impl(q, k, v, alpha, beta, d, initial_state, cu_seqlens, num_seqs, B, T, H, num_qk_heads, K, V,
                        in_dtype, out_dtype, o, final_state, workspace, workspace_bytes, fusion, stream);
}

namespace {

// Device address of `scratch` on the GPU that runs `stream` (the current
// device for the null stream): looked up once per device with that device
// current, then kept.
int32_t scratch_on(void* stream, int32_t** out) {
  int dev = -1;
  hipError_t e;
  if (stream) {
    hipDevice_t d = -1;
    e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &d);
    dev = static_cast<int>(d);
  } else {
    e = hipGetDevice(&dev);
  }
  if (e != hipSuccess) return fail(COMBA_ERR_HIP, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(COMBA_ERR_UNSUPPORTED, "device ordinal beyond 63");
  int32_t* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
      int cur = -1;
      e = hipGetDevice(&cur);
      if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
      void* addr = nullptr;
      if (e == hipSuccess) e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
      if (cur >= 0 && cur != dev) {
        const hipError_t e2 = hipSetDevice(cur);
        if (e == hipSuccess) e = e2;
      }
      if (e != hipSuccess || !addr)
        return fail(COMBA_ERR_HIP, e != hipSuccess ? hipGetErrorString(e) : "no device address for the scratch array");
      p = static_cast<int32_t*>(addr);
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return COMBA_OK;
}

}  // namespace

COMBA_API int32_t comba_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const float* alpha,
                                          const float* beta, const float* d, const float* initial_state,
                                          const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T,
                                          int32_t H, int32_t K, int32_t V, int32_t in_dtype, int32_t out_dtype,
                                          void* o, float* final_state, void* stream) {
  comba::FwdArgs a;  // host-side checks first, so that bad arguments never reach the device lookup
  int32_t rc = check_args(q, k, v, alpha, beta, d, initial_state, cu_seqlens, num_seqs, B, T, H, H, K, V,
                          in_dtype, out_dtype, o, final_state, a);
  if (rc != COMBA_OK) return rc;
  int32_t* order = nullptr;
  size_t order_bytes = 0;
  if (cu_seqlens) {
    if (num_seqs > kMaxOrderedSeqs)
      return fail(COMBA_ERR_UNSUPPORTED,
                  "comba_chunk_fwd_noalloc takes at most 16384 packed sequences (its device scratch holds the "
                  "order of 16384); use comba_chunk_fwd with a workspace");
    rc = scratch_on(stream, &order);
    if (rc != COMBA_OK) return rc;
    order_bytes = sizeof(int32_t) * kMaxOrderedSeqs;
  }
  return chunk_fwd_impl(q, k, v, alpha, beta, d, initial_state, cu_seqlens, num_seqs, B, T, H, H, K, V, in_dtype,
                        out_dtype, o, final_state, order, order_bytes, 0u, stream);
}

COMBA_API size_t comba_chunk_states_size(int32_t B, int32_t T, int32_t H, int32_t K, int32_t V,
                                         int32_t num_seqs) {
  if (B < 1 || T < 0 || H < 1 || K < 1 || V < 1 || num_seqs < 0) return 0;
  const bool packed = num_seqs > 0;
  return static_cast<size_t>(comba::chunk_slots(packed, B, T, packed ? num_seqs : B)) * H * V * K * 4;
}

COMBA_API int32_t comba_chunk_fwd_keep_states(const void* q, const void* k, const void* v, const float* alpha,
                                              const float* beta, const float* d, const float* initial_state,
                                              const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T,
                                              int32_t H, int32_t K, int32_t V, int32_t in_dtype,
                                              int32_t out_dtype, void* o, float* final_state, void* workspace,
                                              size_t workspace_bytes, float* chunk_states,
                                              size_t chunk_states_bytes, void* stream) {
  if (!chunk_states) return fail(COMBA_ERR_INVALID_ARG, "chunk_states must be non-NULL");
  const size_t need = comba_chunk_states_size(B, T, H, K, V, cu_seqlens ? num_seqs : 0);
  if (chunk_states_bytes < need)
    return fail(COMBA_ERR_WORKSPACE, "chunk_states is smaller than comba_chunk_states_size()");
  return chunk_fwd_impl(q, k, v, alpha, beta, d, initial_state, cu_seqlens, num_seqs, B, T, H, H, K, V, in_dtype,
                        out_dtype, o, final_state, workspace, workspace_bytes, 0u, stream, chunk_states);
}

COMBA_API int32_t comba_recurrent_step(const void* q, const void* k, const void* v, const float* alpha,
                                       const float* beta, const float* d, const float* initial_state,
                                       const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T,
                                       int32_t H, int32_t K, int32_t V, int32_t in_dtype,
                                       int32_t out_dtype, void* o, float* final_state, void* stream) {
  return recurrent_impl(q, k, v, alpha, beta, d, initial_state, cu_seqlens, num_seqs, B, T, H, H, K, V, in_dtype,
                        out_dtype, o, final_state, 0u, stream);
}

COMBA_API int32_t comba_recurrent_step_fused(const void* q, const void* k, const void* v, const float* alpha,
                                             const float* beta, const float* d, const float* initial_state,
                                             const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T,
                                             int32_t H, int32_t K, int32_t V, int32_t in_dtype,
                                             int32_t out_dtype, void* o, float* final_state, uint32_t fusion,
                                             void* stream) {
  return recurrent_impl(q, k, v, alpha, beta, d, initial_state, cu_seqlens, num_seqs, B, T, H, H, K, V, in_dtype,
                        out_dtype, o, final_state, fusion, stream);
}

COMBA_API int32_t comba_recurrent_step_ex(const void* q, const void* k, const void* v, const float* alpha,
                                          const float* beta, const float* d, const float* initial_state,
                                          const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T,
                                          int32_t H, int32_t num_qk_heads, int32_t K, int32_t V, int32_t in_dtype,
                                          int32_t out_dtype, void* o, float* final_state, uint32_t fusion,
                                          void* stream) {
  return recurrent_impl(q, k, v, alpha, beta, d, initial_state, cu_seqlens, num_seqs, B, T, H, num_qk_heads, K, V,
                        in_dtype, out_dtype, o, final_state, fusion, stream);
}

namespace {

// Workgroups that fill the chip once (one chunk-kernel workgroup per CU).
constexpr int kTargetWorkgroups = 256;
// Automatic segments are at least this many tokens long.
constexpr int kMinAutoSegment = 512;

struct SegPlan {
  int S;  // segments per sequence (1: no segmentation)
  int L;  // tokens per segment (a multiple of 64)
};

SegPlan plan_segments(int32_t B, int32_t T, int32_t H, int32_t V, int32_t num_segments) {
  const int chunks = (T + 63) / 64;
  int S = num_segments;
  if (S <= 0) {
    const int64_t units = static_cast<int64_t>(B) * H * ((V + 63) / 64);
    const int64_t fill = units >= kTargetWorkgroups ? 1 : kTargetWorkgroups / units;
    S = static_cast<int>(fill < T / kMinAutoSegment ? fill : T / kMinAutoSegment);
  }
  if (S > chunks) S = chunks;
  if (S < 1) S = 1;
  const int L = ((chunks + S - 1) / S) * 64;
  return SegPlan{(T + L - 1) / L, L};
}

struct SegWorkspace {
  size_t cu, bst, phi, x, total;
};

SegWorkspace seg_workspace(int64_t NS, int32_t H, int32_t K, int32_t V) {
  SegWorkspace w;
  w.cu = 0;
  w.bst = align_up(sizeof(int32_t) * (NS + 1));
  w.phi = w.bst + align_up(static_cast<size_t>(NS) * H * V * K * 4);
  w.x = w.phi + align_up(static_cast<size_t>(NS) * H * K * K * 4);
  w.total = w.x + align_up(static_cast<size_t>(NS) * H * V * K * 4);
  return w;
}

}  // namespace

COMBA_API size_t comba_chunk_fwd_segmented_workspace_size(int32_t B, int32_t T, int32_t H, int32_t K, int32_t V,
                                                          int32_t num_segments) {
  if (B < 1 || T < 1 || H < 1 || K < 1 || V < 1) return 0;
  const SegPlan p = plan_segments(B, T, H, V, num_segments);
  if (p.S <= 1) return 0;
  return seg_workspace(static_cast<int64_t>(B) * p.S, H, K, V).total;
}

COMBA_API int32_t comba_chunk_fwd_segmented(const void* q, const void* k, const void* v, const float* alpha,
                                            const float* beta, const float* d, const float* initial_state,
                                            int32_t B, int32_t T, int32_t H, int32_t num_qk_heads, int32_t K,
                                            int32_t V,
                                            int32_t in_dtype, int32_t out_dtype, void* o, float* final_state,
                                            int32_t num_segments, void* workspace, size_t workspace_bytes,
                                            uint32_t fusion, void* stream) {
  if (fusion & ~kKnownFusion) return fail(COMBA_ERR_INVALID_ARG, "unknown bits in fusion");
  if (num_segments < 0) return fail(COMBA_ERR_INVALID_ARG, "num_segments must be >= 0 (0: automatic)");
  comba::FwdArgs a;
  int32_t rc = check_args(q, k, v, alpha, beta, d, initial_state, nullptr, 0, B, T, H, num_qk_heads, K, V,
                          in_dtype, out_dtype, o, final_state, a);
  if (rc != COMBA_OK) return rc;
  if (static_cast<int64_t>(B) * T > INT_MAX)
    return fail(COMBA_ERR_UNSUPPORTED, "B * T above 2^31 - 1 tokens");
  const SegPlan p = plan_segments(B, T, H, V, num_segments);
  if (p.S <= 1)
    return chunk_fwd_impl(q, k, v, alpha, beta, d, initial_state, nullptr, 0, B, T, H, num_qk_heads, K, V, in_dtype,
                          out_dtype, o, final_state, nullptr, 0, fusion, stream);
  const int NS = B * p.S;
  if (static_cast<int64_t>(NS) * H * 2 > INT_MAX / 16)
    return fail(COMBA_ERR_UNSUPPORTED, "too many (segment, head) pairs for one launch");
  const SegWorkspace w = seg_workspace(NS, H, K, V);
  if (!workspace || workspace_bytes < w.total)
    return fail(COMBA_ERR_WORKSPACE,
                "workspace is NULL or smaller than comba_chunk_fwd_segmented_workspace_size()");
  char* ws = static_cast<char*>(workspace);
  int32_t* cu = reinterpret_cast<int32_t*>(ws + w.cu);
  float* bst = reinterpret_cast<float*>(ws + w.bst);
  float* phi = reinterpret_cast<float*>(ws + w.phi);
  float* X = reinterpret_cast<float*>(ws + w.x);
  hipStream_t st = static_cast<hipStream_t>(stream);
  auto launch = [&](const comba::FwdArgs& x) {
    return in_dtype == COMBA_BF16 ? comba::launch_chunk_bf16(x, st) : comba::launch_chunk_fp32(x, st);
  };
  rc = launched(comba::launch_segment_bounds(B, T, p.L, p.S, cu, st));
  if (rc != COMBA_OK) return rc;
  // every segment as a packed sequence of one long row of B T tokens
  comba::FwdArgs seg = a;
  seg.cu_seqlens = cu;
  seg.order = nullptr;
  seg.N = NS;
  seg.B = 1;
  seg.T = B * T;
  seg.fusion = fusion;
  // b_j: final states from zero states, no output
  comba::FwdArgs p1 = seg;
  p1.s0 = nullptr;
  p1.sf = bst;
  p1.fusion = fusion | comba::kModeNoOutput;
  if (in_dtype == COMBA_BF16 && K == V) {
    // one launch forms both: the producers' work serves the b_j and Phi_j consumers
    rc = launched(comba::launch_chunk_bf16_pair(p1, phi, st));
    if (rc != COMBA_OK) return rc;
  } else {
    rc = launched(launch(p1));
    if (rc != COMBA_OK) return rc;
    // Phi_j: v = 0 from the identity, a K x K state
    comba::FwdArgs p2 = p1;
    p2.V = K;
    p2.sf = phi;
    p2.fusion = fusion | comba::kModeNoOutput | comba::kModeZeroV | comba::kModeIdentityInit;
    rc = launched(launch(p2));
    if (rc != COMBA_OK) return rc;
  }
  // X_{j+1} = X_j Phi_j + b_j; the last one is the final state
  rc = launched(comba::launch_segment_scan(initial_state, bst, phi, X, final_state, B, H, K, V, p.S, st));
  if (rc != COMBA_OK) return rc;
  // outputs: every segment from its true initial state
  comba::FwdArgs p3 = seg;
  p3.s0 = X;
  p3.sf = nullptr;
  return launched(launch(p3));
}

namespace {

// Backward workspace. The recomputed chunk states come last: the variant that
// takes them from the forward needs everything before them (`cached`).
struct BwdWorkspace {
  size_t dhck, tm, pm, kk, gt, dd, hck, cached, total;
};

BwdWorkspace bwd_workspace(int64_t nslots, int32_t H, int32_t K, int32_t V) {
  BwdWorkspace w;
  const size_t state = align_up(static_cast<size_t>(nslots) * H * V * K * 4);
  const size_t mat = align_up(static_cast<size_t>(nslots) * H * 64 * 64 * 4);
  w.dhck = 0;
  w.tm = state;
  w.pm = w.tm + mat;
  w.kk = w.pm + mat;
  w.gt = w.kk + mat;
  w.dd = w.gt + align_up(static_cast<size_t>(nslots) * H * 7 * 64 * 4);
  w.hck = w.dd + align_up(static_cast<size_t>(nslots) * H * 4);
  w.cached = w.hck;
  w.total = w.hck + state;
  return w;
}

}  // namespace

COMBA_API size_t comba_chunk_bwd_workspace_size(int32_t B, int32_t T, int32_t H, int32_t K, int32_t V,
                                                int32_t num_seqs) {
  if (B < 1 || T < 0 || H < 1 || K < 1 || V < 1) return 0;
  const bool packed = num_seqs > 0;
  return bwd_workspace(comba::chunk_slots(packed, B, T, packed ? num_seqs : B), H, K, V).total;
}

namespace {

int32_t chunk_bwd_impl(const void* q, const void* k, const void* v, const float* alpha, const float* beta,
                       const float* d, const float* initial_state, const int32_t* cu_seqlens, int32_t num_seqs,
                       int32_t B, int32_t T, int32_t H, int32_t K, int32_t V, int32_t in_dtype, const void* d_o,
                       const float* d_final_state, float* dq, float* dk, float* dv, float* dalpha, float* dbeta,
                       float* dd, float* d_initial_state, const float* chunk_states, size_t chunk_states_bytes,
                       void* workspace, size_t workspace_bytes, void* stream) {
  if (!d_o || !dq || !dk || !dv || !dalpha || !dbeta || !dd)
    return fail(COMBA_ERR_INVALID_ARG, "d_o, dq, dk, dv, dalpha, dbeta and dd must be non-NULL");
  comba::FwdArgs a;
  int32_t rc = check_args(q, k, v, alpha, beta, d, initial_state, cu_seqlens, num_seqs, B, T, H, H, K, V, in_dtype,
                          in_dtype, const_cast<void*>(d_o), nullptr, a);
  if (rc != COMBA_OK) return rc;
  const bool packed = cu_seqlens != nullptr;
  const int64_t nslots = comba::chunk_slots(packed, B, T, a.N);
  if (nslots * H > INT_MAX) return fail(COMBA_ERR_UNSUPPORTED, "too many (chunk, head) pairs for one launch");
  const BwdWorkspace w = bwd_workspace(nslots, H, K, V);
  const bool cached = chunk_states != nullptr;
  if (cached && chunk_states_bytes < static_cast<size_t>(nslots) * H * V * K * 4)
    return fail(COMBA_ERR_WORKSPACE, "chunk_states is smaller than comba_chunk_states_size()");
  if (!workspace || workspace_bytes < (cached ? w.cached : w.total))
    return fail(COMBA_ERR_WORKSPACE, cached ? "workspace is NULL or smaller than comba_chunk_bwd_cached_workspace_size()"
                                            : "workspace is NULL or smaller than comba_chunk_bwd_workspace_size()");
  char* ws = static_cast<char*>(workspace);
  hipStream_t st = static_cast<hipStream_t>(stream);
  float* hck = const_cast<float*>(chunk_states);
  if (!cached) {
    // forward pass that keeps every chunk's incoming state (no output)
    hck = reinterpret_cast<float*>(ws + w.hck);
    comba::FwdArgs f = a;
    f.o = hck;  // never written: no-output mode
    f.sf = nullptr;
    f.order = nullptr;
    f.fusion = comba::kModeNoOutput;
    f.hck = hck;
    rc = launched(in_dtype == COMBA_BF16 ? comba::launch_chunk_bf16(f, st) : comba::launch_chunk_fp32(f, st));
    if (rc != COMBA_OK) return rc;
  }
  comba::BwdArgs g{q, k, v, alpha, beta, d, d_o, cu_seqlens, a.N, a.B, a.T, H, K, V, in_dtype, d_final_state,
                   hck, reinterpret_cast<float*>(ws + w.dhck), reinterpret_cast<float*>(ws + w.dd),
                   reinterpret_cast<float*>(ws + w.tm), reinterpret_cast<float*>(ws + w.pm),
                   reinterpret_cast<float*>(ws + w.kk), reinterpret_cast<float*>(ws + w.gt), dq, dk, dv, dalpha,
                   dbeta, dd, d_initial_state};
  return launched(comba::launch_chunk_bwd(g, st));
}

}  // namespace

COMBA_API int32_t comba_chunk_bwd(const void* q, const void* k, const void* v, const float* alpha,
                                  const float* beta, const float* d, const float* initial_state,
                                  const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T, int32_t H,
                                  int32_t K, int32_t V, int32_t in_dtype, const void* d_o,
                                  const float* d_final_state, float* dq, float* dk, float* dv, float* dalpha,
                                  float* dbeta, float* dd, float* d_initial_state, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  return chunk_bwd_impl(q, k, v, alpha, beta, d, initial_state, cu_seqlens, num_seqs, B, T, H, K, V, in_dtype, d_o,
                        d_final_state, dq, dk, dv, dalpha, dbeta, dd, d_initial_state, nullptr, 0, workspace,
                        workspace_bytes, stream);
}

COMBA_API size_t comba_chunk_bwd_cached_workspace_size(int32_t B, int32_t T, int32_t H, int32_t K, int32_t V,
                                                       int32_t num_seqs) {
  if (B < 1 || T < 0 || H < 1 || K < 1 || V < 1) return 0;
  const bool packed = num_seqs > 0;
  return bwd_workspace(comba::chunk_slots(packed, B, T, packed ? num_seqs : B), H, K, V).cached;
}

COMBA_API int32_t comba_chunk_bwd_cached(const void* q, const void* k, const void* v, const float* alpha,
                                         const float* beta, const float* d, const float* initial_state,
                                         const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T,
                                         int32_t H, int32_t K, int32_t V, int32_t in_dtype, const void* d_o,
                                         const float* d_final_state, const float* chunk_states,
                                         size_t chunk_states_bytes, float* dq, float* dk, float* dv,
                                         float* dalpha, float* dbeta, float* dd, float* d_initial_state,
                                         void* workspace, size_t workspace_bytes, void* stream) {
  if (!chunk_states) return fail(COMBA_ERR_INVALID_ARG, "chunk_states must be non-NULL");
  return chunk_bwd_impl(q, k, v, alpha, beta, d, initial_state, cu_seqlens, num_seqs, B, T, H, K, V, in_dtype, d_o,
                        d_final_state, dq, dk, dv, dalpha, dbeta, dd, d_initial_state, chunk_states,
                        chunk_states_bytes, workspace, workspace_bytes, stream);
}

COMBA_API int32_t comba_varlen_order(const int32_t* cu_seqlens, int32_t num_seqs, int32_t* order,
                                     void* stream) {
  if (!cu_seqlens || !order) return fail(COMBA_ERR_INVALID_ARG, "cu_seqlens and order must be non-NULL");
  if (num_seqs < 1) return fail(COMBA_ERR_INVALID_ARG, "num_seqs must be >= 1");
  return launched(comba::launch_varlen_order(cu_seqlens, num_seqs, order, static_cast<hipStream_t>(stream)));
}

COMBA_API int32_t comba_check_inputs(const float* alpha, int64_t n_alpha, const int32_t* cu_seqlens,
                                     int32_t num_seqs, int32_t T, uint32_t* flags, void* stream) {
  if (!alpha || !flags) return fail(COMBA_ERR_INVALID_ARG, "alpha and flags must be non-NULL");
  if (n_alpha < 0) return fail(COMBA_ERR_INVALID_ARG, "n_alpha must be >= 0");
  if (cu_seqlens && (num_seqs < 1 || T < 0))
    return fail(COMBA_ERR_INVALID_ARG, "with cu_seqlens, num_seqs must be >= 1 and T >= 0");
  return launched(comba::launch_check_inputs(alpha, n_alpha, cu_seqlens, cu_seqlens ? num_seqs : 0, T, flags,
                                             static_cast<hipStream_t>(stream)));
}

COMBA_API int32_t comba_mfma_peak_probe(float* sink, int32_t blocks, int32_t iters, void* stream) {
  if (!sink) return fail(COMBA_ERR_INVALID_ARG, "sink must be non-NULL");
  if (blocks < 1 || iters < 1) return fail(COMBA_ERR_INVALID_ARG, "blocks and iters must be >= 1");
  if (static_cast<int64_t>(blocks) * comba::kPeakProbeThreads > INT_MAX)
    return fail(COMBA_ERR_UNSUPPORTED, "blocks * 256 must fit 31 bits");
  return launched(comba::launch_mfma_peak_probe(sink, blocks, iters, static_cast<hipStream_t>(stream)));
}

COMBA_API int32_t comba_lds_probe(int32_t kind, const int32_t* lane_offsets, int32_t iters, uint32_t* sink,
                                  int32_t blocks, void* stream) {
  if (!lane_offsets || !sink) return fail(COMBA_ERR_INVALID_ARG, "lane_offsets and sink must be non-NULL");
  if (kind < 0 || kind > 7) return fail(COMBA_ERR_INVALID_ARG, "kind must be 0..7");
  if (blocks < 1 || iters < 1) return fail(COMBA_ERR_INVALID_ARG, "blocks and iters must be >= 1");
  if (static_cast<int64_t>(blocks) * comba::kLdsProbeThreads > INT_MAX)
    return fail(COMBA_ERR_UNSUPPORTED, "blocks * 256 must fit 31 bits");
  static constexpr int kWidth[8] = {16, 8, 4, 8, 16, 8, 4, 2};
  const int width = kWidth[kind];
  comba::LdsLaneOffsets offs;
  for (int l = 0; l < 64; ++l) {
    const int32_t o = lane_offsets[l];
    if (o < 0 || o > comba::kLdsProbeBytes - width || o % width != 0)
      return fail(COMBA_ERR_INVALID_ARG, "every lane offset must be aligned to the access width and lie inside 64 KiB");
    offs.v[l] = o;
  }
  return launched(comba::launch_lds_probe(kind, offs, iters, sink, blocks, static_cast<hipStream_t>(stream)));
}
