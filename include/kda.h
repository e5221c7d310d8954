/*
 * kda.h - C ABI of libkda.so, a gfx950 (MI355X) implementation of the Kimi
 * Delta Attention (KDA) gated delta-rule recurrence.
 *
 * What is computed.  For every (sequence n, head h) the library carries a
 * float32 state S in R^{dk x dv} (ejkernel "kernel_delta_attention" page,
 * module description: one memory matrix of key by value dimension per head
 * and batch item; AWS Neuron "KDA TKG Kernel API Reference", parameter S:
 * [B, num_head, dk, dv]).
 * Per token, from raw inputs (kda_tkg parameters q, k, g, beta, a_log,
 * dt_bias, scale, lower_bound):
 *     qh    = scale * q / sqrt(sum q^2 + 1e-6)       (scale folded into the query)
 *     kh    = k / sqrt(sum k^2 + 1e-6)
 *     gamma = lower_bound * sigmoid(exp(a_log[h]) * (g + dt_bias[:, h]))   per key channel
 *     beta  = sigmoid(beta_logit)
 *     S <- Diag(exp(gamma)) S;  S <- S + beta * kh (v - S^T kh)^T;  o = S^T qh
 * With KDA_QK_L2NORM clear, qh = scale * q and kh = k.
 * With KDA_EJK set, the ejkernel ordering of "The core recurrence" is used
 * instead: g is a per-head scalar log-decay d (NULL means 0), beta is used as
 * given, and S <- exp(d) S + beta * kh (v - S^T kh)^T with the residual taken
 * against the undecayed state; o = S^T qh.
 *
 * Conventions shared by every entry point.
 *  - Every tensor pointer is a DEVICE pointer to a contiguous row-major buffer
 *    owned by the caller.  The library never allocates, frees or synchronises.
 *  - `stream` is a hipStream_t (NULL = the default stream).  KDA_OK means the
 *    work was enqueued on that stream; results are valid once it completes.
 *  - Host-checkable argument errors return a non-OK status before any HIP
 *    call is made and enqueue nothing.  Device-side values are not
 *    inspected: NaN/Inf propagate, and out-of-range cu_seqlens entries are
 *    clamped to [0, T] (a decreasing pair is an empty sequence) so they can
 *    never address memory outside the buffers.  Ranges that overlap are
 *    memory-safe too, but their outputs and states are then unspecified
 *    (several sequences write the same rows).
 *  - kda_last_error() returns a thread-local message for the last non-OK
 *    status of the calling thread.  The library holds no other mutable state
 *    and is re-entrant; calls on one stream execute in order.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 3

typedef enum {
    KDA_OK = 0,
    KDA_EINVAL = 1,        /* malformed arguments (null pointer, bad shape, bad flag) */
    KDA_EUNSUPPORTED = 2,  /* well-formed but outside what the kernels implement      */
    KDA_EHIP = 3           /* a HIP launch failed; message from hipGetErrorString      */
} kda_status_t;

typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype_t;

/* flags */
#define KDA_QK_L2NORM (1u << 0) /* ejkernel use_qk_l2norm (its default is on)          */
#define KDA_CHUNKED   (1u << 1) /* ejkernel use_chunked: chunk-parallel algorithm;     */
                                /* clear = token-by-token recurrent scan               */
#define KDA_EJK       (1u << 2) /* ejkernel ordering with a scalar per-head decay      */

/*
 * kda_prefill - run the recurrence over whole sequences (ejkernel
 * "kernel_delta_attention" run(): query, key, value, beta, decay,
 * initial_state, softmax_scale, chunk_size, use_qk_l2norm, use_chunked,
 * return_state; varlen packing as in ejkernel "recurrent" run(): cu_seqlens).
 *
 * Shapes (dense batch): q [B, T, H, dk]; k [B, T, Hkv, dk]; v [B, T, Hkv, dv];
 * o [B, T, H, dv]; states [B, H, dk, dv].  Grouped heads (ejkernel
 * "recurrent" run(): key and value carry num_kv_heads, query, gates, state
 * and output num_heads): head h reads the key and value of head
 * h / (H / Hkv); Hkv must divide H, and Hkv = 0 means Hkv = H.  With cu_seqlens ([num_seqs + 1] int32, device,
 * cu[0] = 0, non-decreasing, cu[num_seqs] = T) the batch must be B = 1 and
 * sequence n covers tokens [cu[n], cu[n+1]); states are [num_seqs, H, dk, dv]
 * and every sequence restarts from its own initial state.
 *
 *   q, k, v        in_dtype (KDA_BF16 or KDA_F32)
 *   Hkv            key/value heads (0 = H)
 *   g              KDA: raw gate [B, T, H, dk] float32 (required);
 *                  EJK: log-decay [B, T, H] float32, NULL = 0 (no decay)
 *   beta           KDA: logits [B, T, H]; EJK: activated [B, T, H]; float32
 *   a_log          [H] float32 (KDA; ignored for EJK; required for KDA)
 *   dt_bias        [dk, H] float32 (KDA; NULL = 0)
 *   initial_state  [N, H, dk, dv] float32, NULL = zeros
 *   scale          query scale; <= 0 or NaN selects 1/sqrt(dk)
 *   lower_bound    KDA gate bound, finite and <= 0 (the kda_tkg documented
 *                  range is [-5, 0]; below -5 the call takes the
 *                  token-by-token kernel, see Routing)
 *   chunk_size     64 (the ejkernel default) when KDA_CHUNKED is set; the
 *                  float32-arithmetic chunked kernel computes the same result
 *                  in chunks of 16 or 32 (see Routing)
 *   o              out_dtype; KDA_BF16 output needs bf16 input
 *   final_state    [N, H, dk, dv] float32 or NULL (return_state = False);
 *                  may alias initial_state exactly (in-place carry)
 *   workspace      device scratch of kda_prefill_workspace_bytes() bytes,
 *                  may be NULL when that size is 0
 *
 * Dimensions: dk, dv in {16, 32, 64, 128} (kda_tkg: dk <= 128); H and the
 * number of sequences at most 65535.  B = 0 or
 * T = 0 is a no-op, except that final_state then receives initial_state (or
 * zeros).  Routing (which kernel runs; every route computes the same function
 * and meets the same accuracy bar):
 *   - KDA_CHUNKED with bf16 inputs and dk = 128 (any of the dv above) runs
 *     the MFMA chunked kernel (64-token chunks; KDA and EJK modes) when q, k,
 *     v, o and (KDA) g are 16-byte aligned and, in KDA mode,
 *     lower_bound >= -5 (its decay factors then stay inside the bf16/float32
 *     exponent range);
 *   - KDA_CHUNKED with float32 inputs (any dk) or bf16 inputs with dk < 128
 *     computes in float32 (float32 MFMA) when q, k and (KDA) g are 16-byte
 *     aligned and, in KDA mode, lower_bound >= -5: with H * dk >= 128, when
 *     the workspace holds them, as two kernels on 16-token chunks (every
 *     chunk's state-independent operands in parallel, then a scan per 16
 *     state columns); otherwise as one kernel (chunks of 32 tokens at
 *     dk <= 32 and 16 above).  The rule depends on neither the token count
 *     nor the packing, so packed sequences take the route of the sequences
 *     run alone.  The chunking and the split change rounding only;
 *   - every other call (KDA_CHUNKED clear, unaligned pointers, or
 *     lower_bound < -5 in KDA mode), whatever its input dtype, runs the
 *     float32 token-by-token kernel.
 * EJK decays are expected to be <= 0 (the ejkernel page says so); the chunked
 * kernels scale by e^{sum of decays} within a chunk, so a positive decay
 * large enough to overflow float32 there gives inf/NaN where the
 * token-by-token kernel would only overflow later.
 */
kda_status_t kda_prefill(const void* q, const void* k, const void* v, kda_dtype_t in_dtype,
                         const float* g, const float* beta, const float* a_log,
                         const float* dt_bias, const float* initial_state,
                         const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T,
                         int32_t H, int32_t Hkv, int32_t dk, int32_t dv, float scale, float lower_bound,
                         int32_t chunk_size, uint32_t flags, void* o, kda_dtype_t out_dtype,
                         float* final_state, void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * kda_prefill_noalloc - kda_prefill without a workspace argument, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  Arguments, routing,
 * results and status codes are those of kda_prefill; the call itself
 * allocates nothing.  The chunked MFMA route takes its workspace from a fixed
 * device array of KDA_NOALLOC_SCRATCH_BYTES (256 MiB) inside the library: one
 * copy per GPU, held from the library's first use on that GPU until the
 * process ends.  A dense call on that route that needs more than that runs in
 * segments of whole chunks inside the array (as kda_prefill does with a small
 * workspace, below); a packed call that needs more (kda_prefill_workspace_bytes()
 * of its arguments; about 1 KiB per token and head, e.g. 16384 tokens at
 * H = 16), or a dense one with more than about 4000 (sequence, head) pairs,
 * returns KDA_EUNSUPPORTED before any launch.  The two-kernel float32 route uses the same array when its blocks
 * fit (about 1.7 KiB per token and head at dk 128), and otherwise runs as one
 * kernel.  The array is used on the calling thread's current HIP device,
 * which must be the device of `stream` and of the tensors.  Every call on one
 * GPU shares the array and leaves its contents behind: calls that may overlap
 * in time on one GPU (other streams, other host threads) race and must be
 * ordered by the caller; calls on one stream are ordered already.
 */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
kda_status_t kda_prefill_noalloc(const void* q, const void* k, const void* v, kda_dtype_t in_dtype,
                                 const float* g, const float* beta, const float* a_log,
                                 const float* dt_bias, const float* initial_state,
                                 const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T,
                                 int32_t H, int32_t Hkv, int32_t dk, int32_t dv, float scale,
                                 float lower_bound, int32_t chunk_size, uint32_t flags, void* o,
                                 kda_dtype_t out_dtype, float* final_state, void* stream);

/* Device workspace (bytes) kda_prefill needs for these arguments; 0 = none.
 * The chunked routes that split a call into kernels use it: per (chunk,
 * head) it holds the state-independent operands of that chunk (the MFMA
 * route: 64.5 KiB per 64-token chunk; the two-kernel float32 route: 6.25,
 * 9.25, 15.5 and 27.75 KiB per 16-token chunk at dk 16, 32, 64 and 128), plus
 * the chunk offsets
 * of packed sequences (num_seqs > 0 with B == 1 means packed).  The caller
 * allocates it (the library never allocates); it must not be shared by calls
 * that may run concurrently.  A float32-route call given less runs as one
 * kernel, which needs none.  A dense call (no cu_seqlens) on the MFMA route
 * given less runs in segments of whole 64-token chunks of every sequence, each
 * segment's final state the next one's initial state, with the same result bit
 * for bit; it needs at least 64.5 KiB per (sequence, head), plus
 * N * H * dk * dv * 4 bytes (rounded up to 256) for the carried state when
 * final_state is NULL.  Packed calls need the whole size. */
size_t kda_prefill_workspace_bytes(int32_t num_seqs, int32_t B, int32_t T, int32_t H,
                                   int32_t dk, int32_t dv, kda_dtype_t in_dtype,
                                   uint32_t flags);

/*
 * kda_prefill_backward - gradients of kda_prefill: the training pass that the
 * chunked mode of the ejkernel "kernel_delta_attention" page (section
 * "Algorithm modes"; run() use_chunked) is there for.  Given dL/do and
 * dL/d(final state), it writes dL/d of every input of the same call.
 * Inputs q ... lower_bound, cu_seqlens, num_seqs, B, T, H, Hkv, dk, dv and
 * the flags KDA_QK_L2NORM / KDA_EJK are kda_prefill's, with the same shapes
 * and meaning (KDA_CHUNKED is accepted and changes nothing: the backward is
 * always chunk-parallel, in float32 arithmetic, chunks of 16 tokens).  H and
 * the number of sequences at most 65535, their product at most 2^26
 * (KDA_EUNSUPPORTED beyond).
 *   d_o              [B, T, H, dv] in do_dtype (KDA_F32 or KDA_BF16)
 *   d_final_state    [N, H, dk, dv] float32, NULL = 0
 * Outputs (device, float32, caller-allocated, fully written):
 *   dq [B, T, H, dk]; dk_out [B, T, Hkv, dk]; dv_out [B, T, Hkv, dv] (grouped heads:
 *   summed over the heads that read each key/value head)
 *   dg     KDA: [B, T, H, dk], dL/d(raw gate g) (required);
 *          EJK: [B, T, H], dL/d(decay) (NULL = not wanted; also given where
 *          g itself is NULL, as the gradient at a zero decay)
 *   dbeta  [B, T, H]: dL/d(beta logit) for KDA, dL/d(beta) for EJK
 *   da_log [H], ddt_bias [dk, H]: KDA only, each NULL = not wanted
 *   d_initial_state [N, H, dk, dv] or NULL
 * KDA mode needs lower_bound >= -5 (KDA_EUNSUPPORTED otherwise): within 16
 * tokens the decay factors then stay inside float32's normal range.
 * The workspace (kda_prefill_backward_workspace_bytes) holds the state
 * entering and the state gradient leaving every pair of 16-token chunks
 * (2 x dk x dv x 4 bytes per pair and head), each chunk's Y = V - Kg S0, U
 * and Z (3 x 16 x dv x 4 bytes per chunk and head) and column-independent
 * operands, per-chunk parameter partials and, with grouped heads, per-head
 * key/value gradients; it is caller-owned and must
 * not be shared by calls that may run concurrently.  With no tokens the call
 * still writes d_initial_state (= d_final_state, or 0) and zero parameter
 * gradients.
 */
size_t kda_prefill_backward_workspace_bytes(int32_t num_seqs, int32_t B, int32_t T, int32_t H, int32_t Hkv,
                                            int32_t dk, int32_t dv);
kda_status_t kda_prefill_backward(const void* q, const void* k, const void* v, kda_dtype_t in_dtype,
                                  const float* g, const float* beta, const float* a_log,
                                  const float* dt_bias, const float* initial_state,
                                  const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T,
                                  int32_t H, int32_t Hkv, int32_t dk, int32_t dv, float scale,
                                  float lower_bound, uint32_t flags, const void* d_o, kda_dtype_t do_dtype,
                                  const float* d_final_state, float* dq, float* dk_out, float* dv_out, float* dg,
                                  float* dbeta, float* da_log, float* ddt_bias, float* d_initial_state,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * kda_recurrent_attention - the gated recurrent attention of the ejkernel
 * "recurrent" page (recurrent_attention(): query, key, value, g, g_gamma,
 * gk, gv, softmax_scale, initial_state, reverse, cu_seqlens, return_state).
 * The page gives the gates' names and shapes but no formula; the reading
 * implemented (every gate a log-space factor, used as given; absent = 0):
 *     S <- exp(g_gamma[b, h]) Diag(exp(gk_t)) S Diag(exp(gv_t))   layer, key, value gates
 *     S <- S + k_t v_t^T
 *     o_t = S^T (scale exp(g_t) q_t)                              query gate
 * with the tokens of each sequence taken in order, or last to first when
 * reverse = 1 (o_t is then read after the tokens t..end).  No delta rule, no
 * L2 norm.  Shapes: q [B, T, H, dk]; k [B, T, Hkv, dk]; v [B, T, Hkv, dv]
 * (in_dtype); g, gk [B, T, H, dk]; gv [B, T, H, dv]; g_gamma [B, H] (packed:
 * [1, H]) - float32, each NULL = absent; states [N, H, dk, dv] float32
 * (initial NULL = zeros; final NULL = not returned); o [B, T, H, dv]
 * (out_dtype; bf16 needs bf16 input).  scale <= 0 or NaN selects 1/sqrt(dk).
 * Grouped heads, cu_seqlens and num_seqs as for kda_prefill.  dk, dv in
 * {16, 32, 64, 128}; H times the number of sequences at most 2^26.  Computed in float32 in chunks of 16 tokens (an exact
 * regrouping of the token loop): the chunks' key-axis operands are formed
 * in parallel into the workspace, then each (sequence, head, 16 state
 * columns) walks its chunks in order.  The workspace
 * (kda_recurrent_attention_workspace_bytes, caller-owned, device memory,
 * not to be shared by calls that may run concurrently) holds about
 * 18.4 KiB per 16-token chunk and head at dk = 128; a smaller one gives
 * KDA_EINVAL.
 */
size_t kda_recurrent_attention_workspace_bytes(int32_t num_seqs, int32_t B, int32_t T, int32_t H, int32_t dk,
                                               int32_t dv);
kda_status_t kda_recurrent_attention(const void* q, const void* k, const void* v, kda_dtype_t in_dtype,
                                     const float* g, const float* g_gamma, const float* gk, const float* gv,
                                     const float* initial_state, const int32_t* cu_seqlens, int32_t num_seqs,
                                     int32_t B, int32_t T, int32_t H, int32_t Hkv, int32_t dk, int32_t dv,
                                     float scale, int32_t reverse, void* o, kda_dtype_t out_dtype,
                                     float* final_state, void* workspace, size_t workspace_bytes,
                                     void* stream);

/*
 * kda_decode_step - advance the recurrence by exactly one token for each of
 * B requests (AWS Neuron "KDA TKG Kernel API Reference", kda_tkg: same
 * tensors, layouts and in-place state; scale and lower_bound are host floats
 * here instead of [1, 1] device tensors).  All float32:
 *   q, g      [B, dk, H] raw (EJK: g is the log-decay [B, 1, H], NULL = 0)
 *   k         [B, dk, Hkv] raw;  v [B, Hkv, dv]: Hkv key/value heads, head h
 *             reads those of head h / (H / Hkv) (Hkv divides H; 0 = H)
 *   beta      [B, 1, H] logits (EJK: activated)
 *   a_log     [1, H] (ignored for EJK);  dt_bias [dk, H] (NULL = 0)
 *   out       [B, H, dv], caller-allocated, written
 *   S         [B, H, dk, dv] IN/OUT: read, then overwritten with the new state
 * flags: KDA_QK_L2NORM and KDA_EJK (KDA_CHUNKED is meaningless here and is
 * rejected).  dk, dv in {16, 32, 64, 128}; B = 0 is a no-op.
 */
kda_status_t kda_decode_step(const float* q, const float* k, const float* g, const float* v,
                             const float* beta, const float* a_log, const float* dt_bias,
                             float scale, float lower_bound, int32_t B, int32_t H, int32_t Hkv,
                             int32_t dk, int32_t dv, uint32_t flags, float* out, float* S, void* stream);

/* Message for the calling thread's last non-OK status ("" if none). */
const char* kda_last_error(void);

/* KDA_ABI_VERSION of the loaded library. */
int kda_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
