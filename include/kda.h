/*
 * kda.h -- C ABI of libkda, Kimi Delta Attention (KDA) kernels for AMD MI355X
 * (gfx950).
 *
 * KDA is the gated delta rule with a per-channel forget gate, eq. (1) on page
 * "Kimi K3论文：Kimi Linear", section 3:
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
 *     o_t = S_t^T q_t,
 *
 * with S_t a d_k x d_v fp32 state, alpha_t = exp(g_t) in (0,1]^{d_k} and
 * beta_t in [0,1].  The same page (section 4) splits the work into a
 * chunkwise-parallel prefill and a cheaper recurrent decode step; this library
 * exports one entry point for each.
 *
 * Conventions shared by every entry point:
 *  - All data pointers are DEVICE pointers (HIP global memory) owned by the
 *    caller.  The library allocates nothing, frees nothing and keeps no pointer
 *    after it returns.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t passed as
 *    void*, NULL = the default stream).  No call synchronises the host; buffers
 *    must stay alive until the stream work has finished.
 *  - Layouts are dense, row-major (C order), no padding.  Every data pointer
 *    must be 16-byte aligned, except `beta`, which needs its element size.
 *  - Only d_k = d_v = 128 is supported; other sizes return KDA_ERR_UNSUPPORTED.
 *  - Arguments are validated on the host before anything is launched; a
 *    failed check returns a negative status and touches no memory.  Values
 *    are not inspected: NaN and Inf pass through.
 *  - Calls keep no state between them and are safe from several host threads.
 *  - A `workspace` is caller-owned device scratch.  Where one is required, a
 *    NULL workspace returns KDA_ERR_INVALID_ARG and one of fewer bytes than
 *    the call needs returns KDA_ERR_WORKSPACE, before anything is launched.
 *
 * Numeric range of the gate: g (= log alpha) must be finite and <= 0.  The
 * chunked prefill splits each in-chunk decay exp(G_r - G_i) at a reference
 * point (page "Kimi K3论文：Kimi Linear", section 4: chunking below the chunk
 * because of the reciprocal of the cumulative decay).  A 64-token chunk whose
 * cumulative log-decay stays above -66 in every channel uses the chunk start;
 * any other chunk uses the ends of its four 16-token sub-chunks, which only
 * needs every channel's log-decay over each such sub-chunk to stay above -87
 * (chunk totals down to about -350).  Stronger gates are outside the
 * supported range.  The backward pass (kda_chunk_bwd*) references its decay
 * factors to the same sub-chunk ends and has the same range.  The decode step
 * has no limit.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k, v, beta and o.  g and the state are always fp32. */
typedef enum {
    KDA_F32 = 0,  /* IEEE fp32 */
    KDA_BF16 = 1  /* bfloat16 (upper half of an fp32) */
} kda_dtype_t;

/*
 * Kind of forget gate, for the *_gated entry points.  KDA's gate is one decay
 * per key channel (eq. (1) of page "Kimi K3论文：Kimi Linear", section 3); the
 * same page (section 2) places KDA after Gated DeltaNet, whose gate is one
 * decay per head and token, and DeltaNet, which has no decay (alpha = 1).
 * The three share the recurrence and these kernels.
 */
typedef enum {
    KDA_GATE_CHANNEL = 0,  /* log_alpha [.., H, dk] fp32: KDA                  */
    KDA_GATE_HEAD = 1,     /* log_alpha [.., H] fp32: Gated DeltaNet           */
    KDA_GATE_NONE = 2      /* no decay, log_alpha must be NULL: DeltaNet       */
} kda_gate_t;

/* Status codes. */
enum {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARG = -1, /* NULL pointer, negative size, overlapping buffers */
    KDA_ERR_UNSUPPORTED = -2, /* d_k or d_v != 128, unknown dtype, size overflow */
    KDA_ERR_ALIGNMENT = -3,   /* pointer not aligned as documented above */
    KDA_ERR_HIP = -4,         /* a HIP launch or runtime call failed */
    KDA_ERR_WORKSPACE = -5    /* a workspace smaller than the call needs */
};

/*
 * Chunkwise prefill: runs eq. (1) over T tokens of B x H independent heads, in
 * chunks of 64 tokens (page "Kimi Linear：高效注意力机制在长序列处理中的创新应用",
 * sections 2.1-2.3, and page "Kimi K3论文：Kimi Linear", section 4: in-chunk
 * cumulative decay, masked intra-chunk matrices Aqk and Akk, inversion of the
 * unit-lower-triangular I + Akk by forward substitution, WY factors, and a
 * sequential chunk-to-chunk pass of the state).
 *
 *   q, k      [B, T, H, dk]  dtype          queries, keys (L2-normalised by the caller)
 *   v         [B, T, H, dv]  dtype          values
 *   log_alpha [B, T, H, dk]  fp32           g_t = log(alpha_t), finite, <= 0
 *   beta      [B, T, H]      dtype          write strength
 *   S0        [B, H, dk, dv] fp32           initial state; NULL means zeros
 *   o         [B, T, H, dv]  dtype   out    o_t = S_t^T q_t
 *   S_T       [B, H, dk, dv] fp32    out    final state; NULL means not written.
 *                                           S_T may equal S0 (updated in place);
 *                                           any other overlap is rejected.
 *   workspace                 device scratch, owned by the caller, or NULL.
 *                             With dtype == KDA_BF16 and workspace_bytes >=
 *                             B * H * ceil(T / 64) * 60416, the call runs two
 *                             kernels: the key-side operands of every chunk
 *                             are computed in parallel into the workspace,
 *                             then a serial scan applies them to the state.
 *                             With 16 heads or fewer (B * H) and at least
 *                             kda_chunk_fwd_workspace_size() bytes, the scan
 *                             runs each head's chunks in segments in parallel
 *                             (per-segment end state and transition, then
 *                             each segment from its entry state: the state
 *                             after r chunks is an affine map of the state
 *                             before them, page "Kimi Linear：高效注意力机制在
 *                             长序列处理中的创新应用", section 2.1); results
 *                             agree with the one-pass scan to rounding.
 *                             With workspace NULL (or dtype KDA_F32, where
 *                             the workspace is ignored) one fused kernel does
 *                             both and no workspace is touched.  A non-NULL
 *                             workspace of fewer bytes than
 *                             kda_chunk_fwd_scan_workspace_size() returns
 *                             KDA_ERR_WORKSPACE (bf16, T >= 1), and with a
 *                             workspace B * H * ceil(T / 64) must stay below
 *                             2^31 (else KDA_ERR_UNSUPPORTED).  The
 *                             workspace must be 256-byte aligned and overlap
 *                             no other buffer; its contents on entry and exit
 *                             are unspecified.
 * T may be any value >= 0 (a partial last chunk is handled exactly); T = 0
 * copies S0 (or zeros) to S_T.  B*H = 0 is a no-op.  `o` must not overlap any
 * input.  Returns KDA_OK or a negative status.
 */
int kda_chunk_fwd(const void* q, const void* k, const void* v,
                  const float* log_alpha, const void* beta, const float* S0,
                  void* o, float* S_T,
                  int B, int T, int H, int dk, int dv, int dtype,
                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * kda_chunk_fwd with a choice of forget gate (kda_gate_t): `log_alpha` is
 * [B, T, H, dk] fp32 for KDA_GATE_CHANNEL (identical to kda_chunk_fwd),
 * [B, T, H] fp32 (4-byte aligned) for KDA_GATE_HEAD, and NULL for
 * KDA_GATE_NONE.  With one decay per head the decay factors are computed once
 * per token and the gate input shrinks from 512 to 4 bytes per head-token.
 * The workspace rules (and kda_chunk_fwd_workspace_size) are those of
 * kda_chunk_fwd.  An unknown gate returns KDA_ERR_UNSUPPORTED.
 */
int kda_chunk_fwd_gated(const void* q, const void* k, const void* v,
                        const float* log_alpha, int gate, const void* beta, const float* S0,
                        void* o, float* S_T,
                        int B, int T, int H, int dk, int dv, int dtype,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Chunked prefill over variable-length sequences packed along one token axis
 * (serving batches).  Sequence s is tokens cu_seqlens[s] .. cu_seqlens[s+1]-1
 * of total_tokens; it is chunked from its own first token and has its own
 * initial and final state, exactly as one kda_chunk_fwd_gated call per
 * sequence would compute it.
 *
 *   q, k         [total_tokens, H, dk]  dtype
 *   v, o         [total_tokens, H, dv]  dtype   (o: out)
 *   log_alpha    [total_tokens, H, dk] / [total_tokens, H] fp32 / NULL, by gate
 *   beta         [total_tokens, H]      dtype
 *   cu_seqlens   [num_seqs + 1]         int32, DEVICE memory, non-decreasing
 *                from 0 to total_tokens.  Not read by the host; the kernel
 *                clamps each entry to [0, total_tokens] (and each end to at
 *                least its start), so no offset can address outside the
 *                buffers; tokens outside every sequence get no output.
 *   S0, S_T      [num_seqs, H, dk, dv]  fp32   (S0 NULL = zeros; S_T NULL =
 *                not written; S_T == S0 updates in place)
 * Runs the fused kernel (no workspace).  num_seqs * H = 0 is a no-op.
 * Errors as for kda_chunk_fwd_gated; cu_seqlens must be 4-byte aligned and
 * must not overlap an output.
 */
int kda_chunk_fwd_varlen(const void* q, const void* k, const void* v,
                         const float* log_alpha, int gate, const void* beta,
                         const int32_t* cu_seqlens, int num_seqs, const float* S0,
                         void* o, float* S_T, int total_tokens, int H, int dk, int dv,
                         int dtype, void* stream);

/*
 * Workspace bytes that kda_chunk_fwd should be given for the fastest schedule
 * on this shape: B * H * ceil(T / 64) * 60416 when the two-kernel schedule is
 * expected to win (bf16 with fewer than 128 heads in total), plus, when its
 * scan runs in nseg > 1 segments (16 heads or fewer, at least two chunks per
 * segment), B * H * (3 * (nseg - 1) + 1) * 65536 for the segment summaries
 * and entry states, or, when prep and scan run pipelined in one launch (24
 * to 48 heads, a multiple of 8, at least two chunks), (B * H * ceil(T / 64)
 * + 8) * 4 for the per-block ready flags and per-XCD arrival counters; else 0
 * (the fused kernel is used and no workspace is needed).
 * Invalid arguments return 0.
 */
size_t kda_chunk_fwd_workspace_size(int B, int T, int H, int dk, int dv, int dtype);

/*
 * Smallest workspace with which kda_chunk_fwd runs the two-kernel schedule
 * (with a one-pass state scan) on this shape, whatever the fastest schedule
 * is: B * H * ceil(T / 64) * kda_chunk_fwd_block_bytes() for dtype KDA_BF16
 * and T >= 1; 0 for fp32 (no workspace is used) or invalid arguments.
 */
size_t kda_chunk_fwd_scan_workspace_size(int B, int T, int H, int dk, int dv, int dtype);

/* Bytes of one per-(batch, head, 64-token chunk) operand block of the
 * two-kernel schedule's workspace. */
size_t kda_chunk_fwd_block_bytes(void);

/*
 * kda_chunk_fwd_gated for callers that cannot allocate device memory -- code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Instead of a caller-supplied workspace, the two-kernel
 * schedule's scratch is a static device array inside the library,
 * KDA_NOALLOC_SCRATCH_BYTES on each GPU, held until the process ends.  The
 * call allocates and frees nothing.  It runs the schedule kda_chunk_fwd_gated
 * runs with kda_chunk_fwd_workspace_size() bytes of workspace (or, when that
 * exceeds the array, with kda_chunk_fwd_scan_workspace_size() bytes); shapes
 * whose scratch exceeds the array even then return KDA_ERR_WORKSPACE.  Shapes
 * served by the fused kernel use no scratch.  Arguments, results and other
 * errors are those of kda_chunk_fwd_gated.  The device is the current HIP
 * device.  Every call on one GPU uses that GPU's one array: calls that can
 * overlap in time on one GPU (other streams, other host threads) race and
 * must be serialised by the caller; calls on one stream are ordered.
 */
#define KDA_NOALLOC_SCRATCH_BYTES (128u << 20)
int kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v,
                          const float* log_alpha, int gate, const void* beta, const float* S0,
                          void* o, float* S_T,
                          int B, int T, int H, int dk, int dv, int dtype, void* stream);

/*
 * Backward pass of kda_chunk_fwd: for a scalar loss L, given dL/do (grad_o)
 * and dL/dS_T (grad_S_T), the gradient of L with respect to every input of the
 * forward call.  The chunkwise algorithm (same pages and sections as
 * kda_chunk_fwd) computes eq. (1) exactly, so these are the gradients of the
 * recurrence itself; they are formed by reverse mode through the chunked form:
 * the forward pass is recomputed chunk by chunk, a serial reverse pass carries
 * dL/dS from the last chunk to the first, and the per-token gradients of all
 * chunks are then formed in parallel.
 *
 *   q, k, v, log_alpha, beta, S0   as for kda_chunk_fwd (S0 NULL means zeros)
 *   grad_o         [B, T, H, dv]  bf16          dL/do
 *   grad_S_T       [B, H, dk, dv] fp32          dL/dS_T; NULL means zero
 *   grad_q, grad_k [B, T, H, dk]  bf16   out
 *   grad_v         [B, T, H, dv]  bf16   out
 *   grad_log_alpha [B, T, H, dk]  fp32   out    with respect to g = log alpha
 *   grad_beta      [B, T, H]      bf16   out
 *   grad_S0        [B, H, dk, dv] fp32   out    dL/dS0; NULL means not written
 *   workspace  device scratch of at least kda_chunk_bwd_workspace_size(...)
 *              bytes, 256-byte aligned, owned by the caller; contents on entry
 *              and exit unspecified.  It holds the recomputed forward pass:
 *              per (batch, head, 64-token chunk) 235,520 bytes -- the key-side
 *              operand blocks of both scans and, in bf16, the state entering
 *              the chunk, its gradient on leaving it, V - Kh S, Vn and
 *              Tm^T dVn.
 * dtype must be KDA_BF16 (KDA_F32 returns KDA_ERR_UNSUPPORTED).  T = 0 writes
 * grad_S0 = grad_S_T (or zeros); B*H = 0 is a no-op.  Outputs must not
 * overlap any input, each other or the workspace.  Returns KDA_OK or a
 * negative status.
 */
int kda_chunk_bwd(const void* q, const void* k, const void* v,
                  const float* log_alpha, const void* beta, const float* S0,
                  const void* grad_o, const float* grad_S_T,
                  void* grad_q, void* grad_k, void* grad_v, float* grad_log_alpha,
                  void* grad_beta, float* grad_S0,
                  int B, int T, int H, int dk, int dv, int dtype,
                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * kda_chunk_bwd with a choice of forget gate (see kda_chunk_fwd_gated):
 * `log_alpha` and `grad_log_alpha` are [B, T, H, dk] fp32 (16-byte aligned)
 * for KDA_GATE_CHANNEL (identical to kda_chunk_bwd), [B, T, H] fp32 (4-byte
 * aligned) for KDA_GATE_HEAD -- there the gradient of a head's one decay is
 * the sum over its channels of the per-channel gradient, since that decay
 * enters every channel -- and both NULL for KDA_GATE_NONE (a non-NULL pointer
 * returns KDA_ERR_INVALID_ARG).  Same workspace, other arguments and errors
 * as kda_chunk_bwd; an unknown gate returns KDA_ERR_UNSUPPORTED.
 */
int kda_chunk_bwd_gated(const void* q, const void* k, const void* v,
                        const float* log_alpha, int gate, const void* beta, const float* S0,
                        const void* grad_o, const float* grad_S_T,
                        void* grad_q, void* grad_k, void* grad_v, float* grad_log_alpha,
                        void* grad_beta, float* grad_S0,
                        int B, int T, int H, int dk, int dv, int dtype,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Workspace bytes kda_chunk_bwd needs: B * H * ceil(T / 64) * 235520 for
 * dtype == KDA_BF16 and d_k = d_v = 128; 0 for invalid or unsupported
 * arguments.
 */
size_t kda_chunk_bwd_workspace_size(int B, int T, int H, int dk, int dv, int dtype);

/*
 * Recurrent decode step: applies eq. (1) once (one token) to each of N x H
 * independent heads, updating the state in place, and returns o = S^T q
 * (page "Kimi K3论文：Kimi Linear", section 3 eq. (1) and section 4, the
 * recurrent kernel used for decoding).
 *
 *   q, k      [N, H, dk]      dtype
 *   v         [N, H, dv]      dtype
 *   log_alpha [N, H, dk]      fp32
 *   beta      [N, H]          dtype
 *   S         [N, H, dk, dv]  fp32   in/out  read, then overwritten with S_t
 *   o         [N, H, dv]      dtype  out
 * N*H = 0 is a no-op.  `S` and `o` must not overlap each other or any input.
 */
int kda_recurrent_step(const void* q, const void* k, const void* v,
                       const float* log_alpha, const void* beta, float* S,
                       void* o, int N, int H, int dk, int dv, int dtype,
                       void* stream);

/*
 * kda_recurrent_step with a choice of forget gate: `log_alpha` is [N, H, dk]
 * for KDA_GATE_CHANNEL (identical to kda_recurrent_step), [N, H] (4-byte
 * aligned) for KDA_GATE_HEAD, NULL for KDA_GATE_NONE.
 */
int kda_recurrent_step_gated(const void* q, const void* k, const void* v,
                             const float* log_alpha, int gate, const void* beta, float* S,
                             void* o, int N, int H, int dk, int dv, int dtype,
                             void* stream);

/*
 * m recurrent steps per head in one call: multi-token and speculative
 * decoding (page "Kimi K3论文：Kimi Linear", section 8: the KDA kernel inside a
 * serving engine; section 3 eq. (1) applied token after token).  Sequence n
 * brings m tokens (drafted tokens, or several known ones); with `accept`
 * NULL all m are applied, otherwise only its first accept[n] (clamped to
 * [0, m]; 0 leaves the state untouched) -- the accepted prefix once a
 * verifier has checked the drafted tokens, e.g. from the outputs of
 * kda_chunk_fwd run on them with S_T = NULL.  The state stays on chip between
 * the tokens, so it crosses HBM once in and once out per call.
 *
 *   q, k      [N, m, H, dk]   dtype        token i of sequence n at [n, i]
 *   v         [N, m, H, dv]   dtype
 *   log_alpha [N, m, H, dk] / [N, m, H] fp32 / NULL, by gate (kda_gate_t)
 *   beta      [N, m, H]       dtype
 *   accept    [N]             int32, DEVICE memory, or NULL (all m)
 *   S         [N, H, dk, dv]  fp32   in/out  state before, then after the
 *                                            applied tokens
 *   o         [N, m, H, dv]   dtype  out     outputs of the applied tokens
 *                                            (others untouched), or NULL
 * N*H = 0 or m = 0 is a no-op.  S and o must not overlap each other or any
 * input; accept must be 4-byte aligned.  Errors as for kda_recurrent_step.
 */
int kda_recurrent_steps(const void* q, const void* k, const void* v,
                        const float* log_alpha, int gate, const void* beta, const int32_t* accept,
                        float* S, void* o, int N, int m, int H, int dk, int dv, int dtype, void* stream);

/*
 * One KDA token-mixing layer (page "Kimi K3论文：Kimi Linear", section 3:
 * input parameterisation of q, k, v, alpha, beta, the KDA recurrence and the
 * gated output path), for B sequences of T tokens, all bf16 except where noted:
 *
 *   q = L2Norm(Swish(ShortConv(W_q x)))    k likewise with W_k, conv_k
 *   v = Swish(ShortConv(W_v x))
 *   log alpha = -softplus(W_up (W_down x))  (fp32, rank = rows of W_down)
 *   beta = Sigmoid(W_beta x)
 *   o = KDA(q, k, v, log alpha, beta), zero initial state, per head
 *   y = W_o (RMSNorm(o, per head) * Sigmoid(W_g x))
 *
 * ShortConv is causal and depthwise with 4 taps: for channel c,
 * conv(x)_t = sum_{j=0..3} w[c][j] x_{t-3+j}, with x_s = 0 before the start of
 * the sequence.  Swish(x) = x Sigmoid(x); L2Norm divides a head's 128 channels
 * by sqrt(sum of squares + 1e-6); RMSNorm divides them by sqrt(mean of squares
 * + 1e-6) (no gain).  No biases.
 *
 *   x       [B, T, d_model]            layer input
 *   W_q, W_k, W_v, W_g  [H*128, d_model]
 *   conv_q, conv_k, conv_v  [H*128, 4] taps, tap 3 multiplies the current token
 *   W_down  [rank, d_model]   W_up [H*128, rank]   W_beta [H, d_model]
 *   W_o     [d_model, H*128]
 *   y       [B, T, d_model]   out
 *   workspace  device scratch of at least kda_layer_workspace_layout(...)
 *              bytes, 256-byte aligned, owned by the caller.  After the call
 *              it holds the layer's intermediate tensors at the offsets that
 *              kda_layer_workspace_layout reports (regions below).
 * Requires d_model and rank to be multiples of 64, H >= 1 and B * T * 4 * H *
 * 128 < 2^31.  T = 0 or B = 0 is a no-op.  Errors as for kda_chunk_fwd; y
 * must not overlap any input or the workspace.  The intermediate activations
 * are rounded to bf16 between steps (log alpha and the low-rank gate input
 * stay fp32); the KDA step runs the same kernels as kda_chunk_fwd, with the
 * same range of the decay (see the top of this header).
 */
enum {
    KDA_LAYER_WS_PRE = 0,  /* [B*T, 4*H*128] bf16: W_q x | W_k x | W_v x | W_g x   */
    KDA_LAYER_WS_LOW,      /* [B*T, ldz] fp32, ldz = rank + H rounded up to 4:
                              W_down x (rank columns) then W_beta x (H columns)  */
    KDA_LAYER_WS_Q,        /* [B, T, H, 128] bf16                                */
    KDA_LAYER_WS_K,        /* [B, T, H, 128] bf16                                */
    KDA_LAYER_WS_V,        /* [B, T, H, 128] bf16                                */
    KDA_LAYER_WS_G,        /* [B, T, H, 128] fp32 log alpha                      */
    KDA_LAYER_WS_BETA,     /* [B, T, H] bf16                                     */
    KDA_LAYER_WS_O,        /* [B, T, H, 128] bf16 KDA output                     */
    KDA_LAYER_WS_ZG,       /* [B*T, H*128] bf16 RMSNorm(o) * Sigmoid(W_g x)      */
    KDA_LAYER_WS_CHUNK,    /* scratch of the chunked KDA schedule                */
    KDA_LAYER_WS_REGIONS
};

int kda_layer_fwd(const void* x, const void* W_q, const void* W_k, const void* W_v,
                  const void* W_g, const void* conv_q, const void* conv_k, const void* conv_v,
                  const void* W_down, const void* W_up, const void* W_beta, const void* W_o,
                  void* y, int B, int T, int d_model, int H, int rank,
                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * Workspace bytes kda_layer_fwd needs for this shape; when `offsets` is not
 * NULL it receives the byte offset of each of the KDA_LAYER_WS_REGIONS
 * regions.  Invalid arguments return 0.
 */
size_t kda_layer_workspace_layout(int B, int T, int d_model, int H, int rank, size_t* offsets);

/*
 * Decode step of a full-attention layer with no position encoding -- the
 * reference KDA's decode is compared against.  Page "Kimi K3论文：Kimi
 * Linear", section 5: the hybrid's full-attention layers are MLA without
 * position encoding, which at inference runs as MQA over a per-token latent;
 * section 7 compares decode time per output token at 1M context.  For every
 * query head h of sequence b, with the latent c_t as key and value:
 *
 *     o[b,h,:] = sum_t softmax_t(scale * q[b,h,:] . c[b,t,:]) c[b,t,:]
 *
 *   q      [B, H, D]  bf16      cache  [B, T, D]  bf16      o  [B, H, D]  bf16 out
 * D must be 512 and H 16 or 32, 1 <= T <= 2^22 (else KDA_ERR_UNSUPPORTED or
 * KDA_ERR_INVALID_ARG for T < 1).
 * workspace: at least kda_mqa_decode_workspace_size(B, T, H, D) bytes,
 * 256-byte aligned (per-split partial results).  B = 0 is a no-op.  o must not
 * overlap q, the cache or the workspace.
 */
int kda_mqa_decode(const void* q, const void* cache, void* o, int B, int T, int H, int D,
                   float scale, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes kda_mqa_decode needs (0 for invalid or unsupported sizes). */
size_t kda_mqa_decode_workspace_size(int B, int T, int H, int D);

/*
 * Chunked forward of the general diagonal-plus-low-rank (DPLR) recurrence,
 * the comparison point for KDA (page "Kimi K3论文：Kimi Linear", section 4:
 * the general gated delta rule with transition D_t - a_t b_t^T, of which KDA
 * is the case a_t = beta_t k_t, b_t = alpha_t * k_t):
 *
 *   S_t = (Diag(alpha_t) - a_t b_t^T) S_{t-1} + k_t v_t^T,   o_t = S_t^T q_t
 *
 * independently for each (batch, head), with alpha_t = exp(log_alpha_t).
 *   q, k, a, b [B, T, H, dk]  bf16        v [B, T, H, dv]  bf16
 *   log_alpha  [B, T, H, dk]  fp32        S0, S_T [B, H, dk, dv] fp32
 *   o          [B, T, H, dv]  bf16 out
 * dk = dv = 128 and dtype = KDA_BF16 only (else KDA_ERR_UNSUPPORTED).  S0
 * NULL means zeros; S_T NULL means not written; S_T == S0 updates in place.
 * workspace: at least kda_dplr_chunk_fwd_workspace_size(...) bytes, 256-byte
 * aligned, owned by the caller, contents unspecified on entry and exit (per
 * 64-token chunk the scan's operand block and the state-independent terms of
 * the chunk form, 103 KiB per (batch, head, chunk) plus 512 bytes per
 * head-token and 256 bytes).  T = 0 copies S0 (or zeros) to S_T; B*H = 0 is a no-op.  o,
 * S_T and the workspace must not overlap any input or each other.  All
 * pointers 16-byte aligned.  Returns KDA_OK or a negative status.
 */
int kda_dplr_chunk_fwd(const void* q, const void* k, const void* v, const void* a, const void* b,
                       const float* log_alpha, const float* S0, void* o, float* S_T,
                       int B, int T, int H, int dk, int dv, int dtype,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes kda_dplr_chunk_fwd needs (0 for invalid or unsupported arguments). */
size_t kda_dplr_chunk_fwd_workspace_size(int B, int T, int H, int dk, int dv, int dtype);

/* Static, human-readable text for a status code (never NULL). */
const char* kda_status_string(int status);

/* Library version as "major.minor.patch" (static string). */
const char* kda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
