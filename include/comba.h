/*
 * comba.h — C ABI of the Comba mixer hot path on AMD Instinct MI355X (gfx950).
 *
 * The mixer (Comba: Improving Bilinear RNNs with Closed-loop Control; arXiv
 * abstract, and the PaperWeekly write-up, section "Comba架构：基于闭环控制理论")
 * is a bilinear RNN with a scalar-plus-low-rank state transition in which the
 * key is the feedback vector that corrects first the value and then the
 * output. Per head, with S_t a V x K state (one row per value channel):
 *
 *     S_t = S_{t-1} (alpha_t I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *     o_t = S_t (q_t - d k_t)
 *
 * The write-up's printed equation was lost from the page text; this is the
 * plainest form consistent with the three facts above. No 1/sqrt(K) query
 * scale is applied; callers L2-normalise q and k themselves if they want to.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every tensor pointer is a DEVICE pointer owned by the caller. Tensors are
 *   row-major and contiguous:
 *       q, k           [B, T, H, K]   in_dtype
 *       v              [B, T, H, V]   in_dtype
 *       alpha, beta    [B, T, H]      float32, alpha in (0, 1] (log alpha is used)
 *       d              [H]            float32, output-correction factor per head
 *       initial_state  [N, H, V, K]   float32, or NULL for zeros
 *       o              [B, T, H, V]   out_dtype
 *       final_state    [N, H, V, K]   float32, or NULL (not written)
 *   The state keeps the value channel as its row index and K contiguous.
 * - cu_seqlens (int32 [N + 1], device memory) packs N variable-length
 *   sequences along T of a single batch row: sequence n owns tokens
 *   cu_seqlens[n] .. cu_seqlens[n+1]-1 and starts from initial_state[n].
 *   It requires B == 1, cu_seqlens[0] == 0, cu_seqlens[N] == T and
 *   non-decreasing values. Without it, N == B and every batch row is one
 *   sequence. A sequence of length 0 returns its initial state. Violating the
 *   device-side preconditions (monotone cu_seqlens, alpha > 0) gives
 *   unspecified values but no out-of-bounds access.
 * - Supported shapes: K, V in {64, 128}; B, H >= 1; T >= 1 (T >= 0 with
 *   cu_seqlens); H * max(K, V) <= 2^22 (up to 32768 heads of 128), else
 *   COMBA_ERR_UNSUPPORTED. Tensors may exceed 4 GiB: token and state offsets
 *   are 64-bit. dtypes: COMBA_BF16 or COMBA_FP32 for q/k/v and for o.
 * - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream). The
 *   call returns without synchronising and never allocates device memory.
 * - Errors detectable on the host (NULL required pointer, bad shape or dtype,
 *   short workspace) are returned before anything is enqueued. A failed
 *   launch returns COMBA_ERR_HIP. comba_last_error() then holds a
 *   human-readable message for the calling thread.
 * - Entry points keep no state between calls and are thread-safe.
 */
#ifndef COMBA_H_
#define COMBA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define COMBA_ABI_VERSION 6

/* Status codes returned by every entry point. */
enum {
  COMBA_OK = 0,
  COMBA_ERR_INVALID_ARG = -1,  /* NULL required pointer, bad size or dtype code */
  COMBA_ERR_UNSUPPORTED = -2,  /* valid but not implemented (e.g. K = 96)      */
  COMBA_ERR_WORKSPACE = -3,    /* workspace NULL or smaller than required       */
  COMBA_ERR_HIP = -4           /* the HIP runtime reported a launch error       */
};

/* Element types of q, k, v (in_dtype) and o (out_dtype). */
enum { COMBA_BF16 = 0, COMBA_FP32 = 1 };

/* Version of this ABI (COMBA_ABI_VERSION of the built library). */
int32_t comba_abi_version(void);

/* Static text for a status code. Never NULL. */
const char* comba_status_string(int32_t status);

/* Detail of the last failure on the calling thread ("" if none). */
const char* comba_last_error(void);

/*
 * Bytes of device workspace comba_chunk_fwd needs for these sizes (0 when
 * none; a NULL workspace is then accepted). num_seqs is N when cu_seqlens is
 * used and 0 otherwise. Returns 0 for invalid sizes as well.
 */
size_t comba_chunk_fwd_workspace_size(int32_t B, int32_t T, int32_t H, int32_t K, int32_t V,
                                      int32_t num_seqs, int32_t in_dtype);

/*
 * Chunk-wise parallel forward (write-up, section "硬件高效的分块并行计算":
 * recurrent across chunks, parallel matrix products inside a chunk, and one
 * matrix inverse per chunk for the intermediates W and U).
 *
 * Computes o for every token and, if final_state is not NULL, S after the
 * last token of every sequence. Chunks of 64 tokens restart at every
 * sequence start; the result does not depend on the chunk size beyond
 * rounding. Floating point work accumulates in float32; bf16 inputs feed the
 * matrix cores exactly and every non-input operand is carried as a pair of
 * bf16 values (high and low part), so the result matches an fp64 evaluation
 * of the recurrence to the rounding of o itself. fp32 inputs use float32
 * arithmetic throughout.
 *
 * workspace: device memory of at least comba_chunk_fwd_workspace_size(...)
 * bytes, used only during this call on `stream`. final_state may be the same
 * pointer as initial_state (each workgroup reads its slice of the initial
 * state before it writes the same slice); a partial overlap is rejected with
 * COMBA_ERR_INVALID_ARG, and final_state must not overlap any other input.
 */
int32_t comba_chunk_fwd(const void* q, const void* k, const void* v,
                        const float* alpha, const float* beta, const float* d,
                        const float* initial_state,
                        const int32_t* cu_seqlens, int32_t num_seqs,
                        int32_t B, int32_t T, int32_t H, int32_t K, int32_t V,
                        int32_t in_dtype, int32_t out_dtype,
                        void* o, float* final_state,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * comba_chunk_fwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). Same arguments, results and errors as
 * comba_chunk_fwd, which it runs with the same kernels.
 *
 * The longest-first order of packed sequences goes to a device array inside
 * the library instead of a workspace: 64 KiB per GPU, held until the process
 * ends, for at most 16384 sequences (more return COMBA_ERR_UNSUPPORTED). Its
 * device address is looked up on the first call per GPU. Every call on one
 * GPU shares that array, so calls that overlap in time on one GPU (on two
 * streams without ordering between them) race and give unspecified values;
 * calls ordered on one stream are safe. The call never allocates, frees or
 * synchronises.
 */
int32_t comba_chunk_fwd_noalloc(const void* q, const void* k, const void* v,
                                const float* alpha, const float* beta, const float* d,
                                const float* initial_state,
                                const int32_t* cu_seqlens, int32_t num_seqs,
                                int32_t B, int32_t T, int32_t H, int32_t K, int32_t V,
                                int32_t in_dtype, int32_t out_dtype,
                                void* o, float* final_state, void* stream);

/*
 * Recurrent form (write-up, section "硬件高效的分块并行计算": the token-by-
 * token recurrence), one token after another from the initial state. With
 * T == 1 this is the single-token decode step of generation. Per value row i:
 *     a = S[i,:] . k,   b = S[i,:] . (q - d k),   u = v_i - a
 *     S'[i,:] = alpha S[i,:] + beta u k^T,        o_i = alpha b + beta u (k . (q - d k))
 * which is the recurrence above expanded for one step.
 *
 * final_state may be the same pointer as initial_state (in-place update of a
 * state resident in device memory); any other overlap is not allowed.
 */
int32_t comba_recurrent_step(const void* q, const void* k, const void* v,
                             const float* alpha, const float* beta, const float* d,
                             const float* initial_state,
                             const int32_t* cu_seqlens, int32_t num_seqs,
                             int32_t B, int32_t T, int32_t H, int32_t K, int32_t V,
                             int32_t in_dtype, int32_t out_dtype,
                             void* o, float* final_state, void* stream);

/*
 * Input-side fusion (CARVE summary, section 2.3 "键轴衰减与融合": the decay
 * gate is evaluated inside the kernel; the GLA/KDA blog, sections 2.1 and
 * 3.1: log-sigmoid and sigmoid gates; the normalisation of q and k is not
 * spelled out by the pages and is taken as the plain per-token L2 norm that
 * keeps the Comba transition alpha I - beta k k^T contractive). Flags for the
 * fused entry points below; any combination, 0 = no fusion:
 *   COMBA_FUSE_GATE_LOGITS  alpha and beta hold logits a, b; the kernels use
 *                           alpha = sigmoid(a) and beta = sigmoid(b), formed
 *                           from e^-|x| so that no logit overflows (alpha
 *                           below the smallest normal float is clamped to it).
 *   COMBA_FUSE_QK_L2NORM    q and k are normalised per (token, head) inside
 *                           the kernels: x / sqrt(sum_i x_i^2 + 1e-6).
 * The normalisation never rounds a normalised q or k to bf16: the factor
 * 1 / sqrt(...) of each token is computed in float32 (in the bf16 chunk
 * kernel with the hardware reciprocal square root, about 1 ulp) and applied
 * to the float32 results of the products in which q or k take part, so fused
 * and unfused calls meet the same accuracy bounds.
 */
enum { COMBA_FUSE_GATE_LOGITS = 1, COMBA_FUSE_QK_L2NORM = 2 };

/*
 * comba_chunk_fwd with input-side fusion: same arguments, layouts, workspace
 * and errors, plus `fusion` (an OR of COMBA_FUSE_* flags; unknown bits are
 * COMBA_ERR_INVALID_ARG). With fusion == 0 it is comba_chunk_fwd.
 */
int32_t comba_chunk_fwd_fused(const void* q, const void* k, const void* v,
                              const float* alpha, const float* beta, const float* d,
                              const float* initial_state,
                              const int32_t* cu_seqlens, int32_t num_seqs,
                              int32_t B, int32_t T, int32_t H, int32_t K, int32_t V,
                              int32_t in_dtype, int32_t out_dtype,
                              void* o, float* final_state,
                              void* workspace, size_t workspace_bytes, uint32_t fusion, void* stream);

/*
 * comba_recurrent_step with input-side fusion (same arguments plus `fusion`,
 * as for comba_chunk_fwd_fused). With fusion == 0 it is comba_recurrent_step.
 */
int32_t comba_recurrent_step_fused(const void* q, const void* k, const void* v,
                                   const float* alpha, const float* beta, const float* d,
                                   const float* initial_state,
                                   const int32_t* cu_seqlens, int32_t num_seqs,
                                   int32_t B, int32_t T, int32_t H, int32_t K, int32_t V,
                                   int32_t in_dtype, int32_t out_dtype,
                                   void* o, float* final_state, uint32_t fusion, void* stream);

/*
 * Shared q / k heads (the Comba write-up, section "硬件高效的分块并行计算",
 * last paragraph: the Mamba-form models share a query and key of dimension
 * 128 across value heads, like multi-value attention; the GLA/KDA blog,
 * section 4.2: grouped value attention). q and k hold num_qk_heads heads,
 * [B, T, num_qk_heads, K]; v, o, alpha, beta, d and the states keep H value
 * heads, and value head h reads q / k head h / (H / num_qk_heads)
 * (consecutive value heads share one q / k head). num_qk_heads must divide
 * H; num_qk_heads == H is the plain layout. Otherwise as comba_chunk_fwd_fused
 * and comba_recurrent_step_fused. COMBA_FUSE_QK_L2NORM normalises each
 * shared q / k row.
 */
int32_t comba_chunk_fwd_ex(const void* q, const void* k, const void* v,
                           const float* alpha, const float* beta, const float* d,
                           const float* initial_state,
                           const int32_t* cu_seqlens, int32_t num_seqs,
                           int32_t B, int32_t T, int32_t H, int32_t num_qk_heads, int32_t K, int32_t V,
                           int32_t in_dtype, int32_t out_dtype,
                           void* o, float* final_state,
                           void* workspace, size_t workspace_bytes, uint32_t fusion, void* stream);

int32_t comba_recurrent_step_ex(const void* q, const void* k, const void* v,
                                const float* alpha, const float* beta, const float* d,
                                const float* initial_state,
                                const int32_t* cu_seqlens, int32_t num_seqs,
                                int32_t B, int32_t T, int32_t H, int32_t num_qk_heads, int32_t K, int32_t V,
                                int32_t in_dtype, int32_t out_dtype,
                                void* o, float* final_state, uint32_t fusion, void* stream);

/*
 * Segment-parallel chunk forward for batches of few, long sequences
 * (fixed-length batches only: no cu_seqlens). Same result as comba_chunk_fwd
 * up to rounding order. The recurrence's state map over a stretch of tokens
 * is affine in the state it starts from (Comba write-up, section
 * "Comba架构：基于闭环控制理论": each step multiplies the state by
 * alpha_t I - beta_t k_t k_t^T and adds beta_t v_t k_t^T), so every sequence is
 * cut into S segments of L tokens (L a multiple of 64) that run in parallel:
 *   1. each segment from a zero state gives its final state b_j;
 *   2. each segment with v = 0 from the identity gives its K x K map Phi_j;
 *   3. a scan X_{j+1} = X_j Phi_j + b_j (fp32), X_0 = initial_state, gives
 *      every segment's true initial state and, as X_S, final_state;
 *   4. each segment runs again from X_j and writes o.
 * This is about three times the arithmetic of comba_chunk_fwd, spread over
 * S times as many workgroups: it pays when B * H * ceil(V / 64) is well below
 * the chip's 256 compute units.
 *
 * Arguments as comba_chunk_fwd_ex (without cu_seqlens / num_seqs), plus:
 *   num_segments  S per sequence; 0 chooses it: enough workgroups to fill 256
 *                 compute units once, segments of at least 512 tokens.
 *                 Capped at ceil(T / 64). When the plan has one segment the
 *                 call is comba_chunk_fwd and uses no workspace.
 *   workspace     device scratch of at least
 *                 comba_chunk_fwd_segmented_workspace_size(B, T, H, K, V,
 *                 num_segments) bytes, 256-byte aligned, not read before it is
 *                 written; it holds the segment bounds, the b_j, Phi_j and X_j.
 *   fusion        as for comba_chunk_fwd_fused, applied in every pass.
 * Errors: as comba_chunk_fwd; COMBA_ERR_INVALID_ARG for num_segments < 0 or
 * unknown fusion bits; COMBA_ERR_UNSUPPORTED when B * T exceeds 2^31 - 1.
 * initial_state == final_state is allowed.
 */
size_t comba_chunk_fwd_segmented_workspace_size(int32_t B, int32_t T, int32_t H, int32_t K, int32_t V,
                                                int32_t num_segments);

int32_t comba_chunk_fwd_segmented(const void* q, const void* k, const void* v,
                                  const float* alpha, const float* beta, const float* d,
                                  const float* initial_state,
                                  int32_t B, int32_t T, int32_t H, int32_t num_qk_heads, int32_t K, int32_t V,
                                  int32_t in_dtype, int32_t out_dtype,
                                  void* o, float* final_state, int32_t num_segments,
                                  void* workspace, size_t workspace_bytes, uint32_t fusion, void* stream);

/*
 * Chunk-wise backward (the training path; the write-up, section
 * "硬件高效的分块并行计算", notes that the backward either reuses the
 * cached chunk inverse and chunk states or recomputes them): gradients of a
 * loss L for given d_o = dL/do [B, T, H, V] (in_dtype) and d_final_state =
 * dL/dS_final [N, H, V, K] (fp32; NULL means 0). Inputs as comba_chunk_fwd
 * (one q / k head per value head, no fusion; the output dtype is not an
 * input). Outputs, all fp32, written in full:
 *   dq, dk [B, T, H, K]; dv [B, T, H, V]; dalpha, dbeta [B, T, H];
 *   dd [H] (summed over the batch and the tokens);
 *   d_initial_state [N, H, V, K] (may be NULL: not written).
 * The call recomputes the forward, keeping every chunk's incoming state,
 * forms each chunk's inverse and score matrices, then runs a reverse scan over
 * the chunks and a chunk-parallel gradient pass. It needs a device workspace
 * of at least comba_chunk_bwd_workspace_size(B, T, H, K, V, num_seqs) bytes
 * (per chunk and head two fp32 states, three fp32 64 x 64 matrices and the
 * chunk's decay gates: about 1.4 GiB for B = 8, T = 4096, H = 16,
 * K = V = 128), 256-byte aligned.
 * Errors: as comba_chunk_fwd, COMBA_ERR_INVALID_ARG for a NULL d_o or
 * gradient output, COMBA_ERR_WORKSPACE for a short workspace.
 */
size_t comba_chunk_bwd_workspace_size(int32_t B, int32_t T, int32_t H, int32_t K, int32_t V, int32_t num_seqs);

int32_t comba_chunk_bwd(const void* q, const void* k, const void* v,
                        const float* alpha, const float* beta, const float* d,
                        const float* initial_state,
                        const int32_t* cu_seqlens, int32_t num_seqs,
                        int32_t B, int32_t T, int32_t H, int32_t K, int32_t V,
                        int32_t in_dtype, const void* d_o, const float* d_final_state,
                        float* dq, float* dk, float* dv, float* dalpha, float* dbeta, float* dd,
                        float* d_initial_state, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The backward that reuses the forward's chunk states instead of recomputing
 * them (the write-up, section "硬件高效的分块并行计算", weighs exactly this
 * choice: keep the chunk states from the forward, or recompute them in the
 * backward). For training, where the forward runs anyway:
 *
 *   comba_chunk_states_size(B, T, H, K, V, num_seqs)
 *       bytes of the chunk-state buffer: one fp32 V x K state per 64-token
 *       chunk and head, laid out [slot, H, V, K]. Slots are the chunks of
 *       every sequence in order (fixed-length batches: b * ceil(T / 64) + c;
 *       packed batches: chunk c of sequence n at cu_seqlens[n] / 64 + n + c).
 *       num_seqs as for comba_chunk_bwd_workspace_size (0 without cu_seqlens).
 *   comba_chunk_fwd_keep_states(...)
 *       comba_chunk_fwd (same arguments and results, no fusion) that also
 *       writes every chunk's incoming state into chunk_states (device, at
 *       least comba_chunk_states_size bytes, caller-owned). Costs one extra
 *       write of the buffer.
 *   comba_chunk_bwd_cached(...)
 *       comba_chunk_bwd (same arguments and results) that reads the chunk
 *       states written by comba_chunk_fwd_keep_states on the same inputs
 *       instead of recomputing them, with a smaller workspace of
 *       comba_chunk_bwd_cached_workspace_size bytes. The results are
 *       bit-identical to comba_chunk_bwd's.
 * Errors: as comba_chunk_fwd / comba_chunk_bwd; COMBA_ERR_INVALID_ARG for a
 * NULL chunk_states, COMBA_ERR_WORKSPACE when chunk_states_bytes or the
 * workspace is short.
 */
size_t comba_chunk_states_size(int32_t B, int32_t T, int32_t H, int32_t K, int32_t V, int32_t num_seqs);

int32_t comba_chunk_fwd_keep_states(const void* q, const void* k, const void* v,
                                    const float* alpha, const float* beta, const float* d,
                                    const float* initial_state,
                                    const int32_t* cu_seqlens, int32_t num_seqs,
                                    int32_t B, int32_t T, int32_t H, int32_t K, int32_t V,
                                    int32_t in_dtype, int32_t out_dtype,
                                    void* o, float* final_state,
                                    void* workspace, size_t workspace_bytes,
                                    float* chunk_states, size_t chunk_states_bytes, void* stream);

size_t comba_chunk_bwd_cached_workspace_size(int32_t B, int32_t T, int32_t H, int32_t K, int32_t V,
                                             int32_t num_seqs);

int32_t comba_chunk_bwd_cached(const void* q, const void* k, const void* v,
                               const float* alpha, const float* beta, const float* d,
                               const float* initial_state,
                               const int32_t* cu_seqlens, int32_t num_seqs,
                               int32_t B, int32_t T, int32_t H, int32_t K, int32_t V,
                               int32_t in_dtype, const void* d_o, const float* d_final_state,
                               const float* chunk_states, size_t chunk_states_bytes,
                               float* dq, float* dk, float* dv, float* dalpha, float* dbeta, float* dd,
                               float* d_initial_state, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Longest-first order of packed sequences (integer work, exact): writes into
 * order[0..N-1] the sequence indices sorted by decreasing length
 * cu_seqlens[n+1] - cu_seqlens[n], ties by increasing index. comba_chunk_fwd
 * runs this itself for packed batches so that the longest sequences start
 * first; it is exported for callers that schedule their own work and for
 * testing. cu_seqlens and order are device pointers; N >= 1.
 */
int32_t comba_varlen_order(const int32_t* cu_seqlens, int32_t num_seqs, int32_t* order,
                           void* stream);

/*
 * Device-side preconditions, checked on demand (a debug aid: no other entry
 * point runs it). Comba's gate alpha is the scalar part of the
 * scalar-plus-low-rank transition (the recurrence at the top of this header;
 * write-up, section "Comba架构：基于闭环控制理论") and the chunk form takes its
 * logarithm (write-up, section "硬件高效的分块并行计算"), so every alpha must
 * lie in (0, 1]; a packed
 * batch's cu_seqlens must start at 0, end at T and never decrease (the
 * layout rules at the top of this header). The call enqueues two small
 * kernels on `stream`: the first stores 0 to *flags, the second ORs in
 *   COMBA_CHECK_ALPHA_RANGE  an alpha outside (0, 1], or NaN;
 *   COMBA_CHECK_CU_ORDER     cu_seqlens[n+1] < cu_seqlens[n] for some n;
 *   COMBA_CHECK_CU_BOUNDS    cu_seqlens[0] != 0 or cu_seqlens[N] != T.
 * *flags is 0 when every precondition holds; read it after the stream has
 * run. Do not pass the gate logits of the fused entry points as alpha.
 * alpha: device float32, n_alpha entries (B * T * H); cu_seqlens: device int32
 * [num_seqs + 1], or NULL (then num_seqs and T are not read); flags: device,
 * one uint32, owned by the caller. Calls that share a flags word race.
 * Errors: COMBA_ERR_INVALID_ARG for NULL alpha or flags, n_alpha < 0, or
 * with cu_seqlens num_seqs < 1 or T < 0.
 */
#define COMBA_CHECK_ALPHA_RANGE 1u
#define COMBA_CHECK_CU_ORDER 2u
#define COMBA_CHECK_CU_BOUNDS 4u
int32_t comba_check_inputs(const float* alpha, int64_t n_alpha, const int32_t* cu_seqlens, int32_t num_seqs,
                           int32_t T, uint32_t* flags, void* stream);

/*
 * Measurement aid, not part of the recurrence: the matrix-core ceiling of the
 * device it runs on, to set beside the published dense bf16 peak when the
 * chunk kernels are rated against it. Launches `blocks` workgroups of four
 * wavefronts; every wavefront runs `iters` iterations of four independent
 * 16x16x32 bf16 MFMAs (16,384 flops each) on register operands, so one call
 * performs blocks * 4 * iters * 4 * 16384 flops and reads no memory. It
 * writes one float per thread to sink (device, blocks * 256 floats, owned by
 * the caller; the values carry no meaning). Time it with events on `stream`.
 * Errors: COMBA_ERR_INVALID_ARG for a NULL sink or blocks, iters < 1;
 * COMBA_ERR_UNSUPPORTED when blocks * 256 exceeds 2^31 - 1.
 */
int32_t comba_mfma_peak_probe(float* sink, int32_t blocks, int32_t iters, void* stream);

/*
 * Measurement aid, not part of the recurrence: one LDS access pattern in
 * isolation, for reading a profiler's LDS bank-conflict counters
 * (SQ_LDS_BANK_CONFLICT, SQ_LDS_IDX_ACTIVE) for that pattern alone. The
 * chunk kernels' LDS layouts were chosen with it. Launches `blocks`
 * workgroups of four wavefronts over a 64 KiB LDS array; lane l of every
 * wavefront accesses byte offset lane_offsets[l] once per iteration, `iters`
 * times. kind: 0, 1, 2 read 16, 8, 4 bytes; 3 is the 8-byte transposing
 * read (ds_read_b64_tr_b16); 4, 5, 6, 7 write 16, 8, 4, 2 bytes.
 * lane_offsets: host, 64 int32; sink: device, blocks * 256 uint32 (written,
 * values meaningless), owned by the caller.
 * Errors: COMBA_ERR_INVALID_ARG for NULL pointers, kind outside 0..7,
 * blocks or iters < 1, or an offset that is negative, not a multiple of the
 * access width or past 64 KiB minus the width; COMBA_ERR_UNSUPPORTED when
 * blocks * 256 exceeds 2^31 - 1.
 */
int32_t comba_lds_probe(int32_t kind, const int32_t* lane_offsets, int32_t iters, uint32_t* sink, int32_t blocks,
                        void* stream);

#ifdef __cplusplus
}
#endif

#endif /* COMBA_H_ */
