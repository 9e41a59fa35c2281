// kda_internal.h -- launchers behind the C ABI (internal to libkda).
// Every launcher assumes the arguments were validated by the C ABI layer.
#pragma once
#include <hip/hip_runtime.h>

#include "../../include/kda.h"

namespace kda {

// Decode step over `heads` = N*H independent heads; dtype 0 = fp32, 1 = bf16;
// `gate` as for launch_chunk_fwd (g [heads, 128], [heads] or unused).
hipError_t launch_decode_step(const void* q, const void* k, const void* v,
                              const float* g, const void* beta, float* S, void* o,
                              long long heads, int dtype, hipStream_t stream,
                              int gate = KDA_GATE_CHANNEL);

// m decode steps per head, tokens [N, m, H, .]; with `accept` (device,
// [N]) sequence n applies only its first accept[n] tokens (clamped to
// [0, m]).  `o` may be null.  heads = N * H.
hipError_t launch_decode_steps(const void* q, const void* k, const void* v, const float* g, const void* beta,
                               const int* accept, float* S, void* o, long long heads, int m, int H, int dtype,
                               hipStream_t stream, int gate = KDA_GATE_CHANNEL);

// Chunked prefill over B*H heads of T >= 1 tokens (d_k = d_v = 128).  With
// `ws` non-null (bf16 only, at least chunk_ws_bytes(B, T, H) bytes) the
// two-kernel schedule runs; otherwise the fused single kernel.  With `seg`
// (ws then holds chunk_fwd_ws_bytes(B, T, H) bytes) its state scan runs in
// segments when chunk_seg_count(B, T, H) > 1.  `gate` is a
// kda_gate_t: g is [B, T, H, 128] (per channel), [B, T, H] (per head) or
// unused (no decay).  With cu_seqlens (device, B + 1 entries) the B
// "batches" are sequences packed along one token axis of T tokens (fused
// kernel, `ws` ignored).
hipError_t launch_chunk_fwd(const void* q, const void* k, const void* v,
                            const float* g, const void* beta, const float* S0,
                            void* o, float* S_T, int B, int T, int H, int dtype,
                            void* ws, hipStream_t stream, int gate = KDA_GATE_CHANNEL,
                            const int* cu_seqlens = nullptr, bool seg = false);

// kda_chunk_fwd_gated's validation and launch; with scratch_bytes > 0 the
// two-kernel schedule takes scratch_bytes of the static scratch array of
// kda_noalloc.hip instead of `workspace` (the allocation-free entry point).
int chunk_fwd_entry(const void* q, const void* k, const void* v, const float* log_alpha, int gate,
                    const void* beta, const float* S0, void* o, float* S_T, int B, int T, int H, int dk,
                    int dv, int dtype, void* workspace, size_t workspace_bytes, size_t scratch_bytes,
                    void* stream);

// Device address of the current device's copy of the library's static
// scratch array (KDA_NOALLOC_SCRATCH_BYTES; looked up once per device), or
// nullptr with *err set.
void* noalloc_scratch(hipError_t* err);

// Bytes of the key-side operand blocks of the two-kernel schedule: one
// 72,704-byte block per (batch, head, 64-token chunk).
size_t chunk_ws_bytes(long long B, long long T, long long H);

// Segments per head of the two-kernel schedule's state scan (1: one pass over
// all chunks; more with 16 heads or fewer, see chunk_scan_kernel).
int chunk_seg_count(long long B, long long T, long long H);

// Whether the two-kernel schedule with its full workspace runs prep and scan
// in one pipelined launch (24 to 48 heads, a multiple of 8).
bool chunk_uses_pipe(long long B, long long T, long long H);

// Bytes of workspace the two-kernel forward schedule needs: the operand
// blocks, then with segments the segment summaries [B*H][nseg-1][128][256]
// and entry states [B*H][nseg][128][128] (fp32), or for the pipelined launch
// one int32 ready flag per block and 8 arrival counters.
size_t chunk_fwd_ws_bytes(long long B, long long T, long long H);

// Whether the two-kernel schedule is expected to be faster for this shape.
bool chunk_prefers_two_kernel(long long B, long long T, long long H, int dtype);

// Backward pass of the chunked prefill (bf16, T >= 1): regions of its
// workspace, in order.
enum {
    KDA_BWD_WS_FWD = 0,   // forward operand blocks, chunk_ws_bytes(B, T, H)
    KDA_BWD_WS_BWD,       // reverse-scan operand blocks, WSB_CHUNK per chunk
    KDA_BWD_WS_S,         // S entering each chunk, bf16 [128][128]
    KDA_BWD_WS_DS,        // gradient of the state leaving each chunk, bf16 [128][128]
    KDA_BWD_WS_Y,         // V - Kh S per chunk, bf16 [64][128]
    KDA_BWD_WS_VN,        // Vn per chunk, bf16 [64][128]
    KDA_BWD_WS_DZ,        // Tm^T dVn per chunk, bf16 [64][128]
    KDA_BWD_WS_REGIONS
};
// Byte offsets of the regions (to `off` when non-null); returns the total.
size_t chunk_bwd_ws_layout(long long B, long long T, long long H, size_t* off);

// The prep kernel (writing both operand blocks) and the forward scan in save
// mode, as the first half of the backward pass.
typedef __bf16 bf16_t;
hipError_t launch_bwd_forward_part(const void* q, const void* k, const void* v, const float* g,
                                   const void* beta, const float* S0, int B, int T, int H,
                                   char* ws_fwd, char* ws_bwd, bf16_t* svS, bf16_t* svY, bf16_t* svVn,
                                   hipStream_t stream, int gate = KDA_GATE_CHANNEL);

// dq, dk, dv, dg, dbeta (and dS0 when non-null) from dO (and dS_T when
// non-null); `ws` holds chunk_bwd_ws_layout(B, T, H) bytes.  g and dg follow
// `gate`: [B, T, H, 128], [B, T, H], or unused (GATE_NONE).
hipError_t launch_chunk_bwd(const void* q, const void* k, const void* v, const float* g,
                            const void* beta, const float* S0, const void* dO, const float* dST,
                            void* dq, void* dk, void* dv, float* dg, void* dbeta, float* dS0,
                            int B, int T, int H, char* ws, hipStream_t stream, int gate = KDA_GATE_CHANNEL);

// State scan over the DPLR prep kernel's output: per-chunk operand blocks,
// U0 and O0 [B, T, H, 128] bf16 and H0 [B*H*chunks][128][128] bf16.
hipError_t launch_dplr_scan(const char* blocks, const bf16_t* u0, const bf16_t* h0, const bf16_t* o0,
                            const float* S0, void* o, float* S_T, int B, int T, int H, hipStream_t stream);

// General diagonal-plus-low-rank chunked forward (bf16): workspace regions
// (blocks, H0, U0, O0, a 256-byte sink for the rows past T) and the launch of
// both kernels.
enum { KDA_DPLR_WS_BLK = 0, KDA_DPLR_WS_H0, KDA_DPLR_WS_U0, KDA_DPLR_WS_O0, KDA_DPLR_WS_SINK, KDA_DPLR_WS_REGIONS };
size_t dplr_ws_layout(long long B, long long T, long long H, size_t* off);
hipError_t launch_dplr_chunk_fwd(const void* q, const void* k, const void* v, const void* a, const void* b,
                                 const float* g, const float* S0, void* o, float* S_T, int B, int T, int H,
                                 char* ws, hipStream_t stream);

// Full-attention (MQA over a 512-wide latent) decode step, split over the
// cache: mqa_ws_bytes of scratch for the per-split partial results.
size_t mqa_ws_bytes(long long B, long long T, long long H);
hipError_t launch_mqa_decode(const void* q, const void* cache, void* o, int B, int T, int H, float scale,
                             void* ws, hipStream_t stream);

// S_T = S0 (or zeros when S0 is NULL) for `heads` states; used when T = 0.
hipError_t launch_state_copy(const float* S0, float* S_T, long long heads,
                             hipStream_t stream);

// C[M, N] = A[M, K] B[N, K]^T (both K-contiguous, K % 64 == 0, leading
// dimensions in elements, multiples of 8).  A is bf16 or, with a_f32, fp32
// (split into bf16 hi + lo parts); B is bf16; C is fp32 (c_f32) or bf16.
// epilogue 0: none, 1: c -> -softplus(c).  With B2, rows n >= n_split of B
// are rows n - n_split of B2 (two weight matrices stacked, one pass over A).
hipError_t launch_gemm_nt(const void* A, bool a_f32, const bf16_t* B, void* C, bool c_f32,
                          int epilogue, int M, int N, int K, int lda, int ldb, int ldc,
                          hipStream_t stream, const bf16_t* B2 = nullptr, int n_split = 0);

// The same product (bf16 A and C) with B made of `nmat` (1 to 4) weight
// matrices of n_split rows each, stacked along N: C[:, i n_split ..] =
// A B[i]^T.  Requires gemm_stacked_ok (M >= 256, n_split % 256 == 0).
bool gemm_stacked_ok(int M, int n_split, int nmat);
hipError_t launch_gemm_nt_stacked(const bf16_t* A, const bf16_t* const* B, int nmat, bf16_t* C, int M,
                                  int n_split, int K, int lda, int ldb, int ldc, hipStream_t stream);

// Weights of one KDA token-mixing layer, all bf16, [out_features, in_features]
// (conv taps [H*128, 4]).
struct LayerWeights {
    const bf16_t *W_q, *W_k, *W_v, *W_g, *conv_q, *conv_k, *conv_v, *W_down, *W_up, *W_beta, *W_o;
};

// Byte offsets of the layer's workspace regions (indexed by KDA_LAYER_WS_*,
// written to `off` when non-null); returns the total size.
size_t layer_ws_layout(long long B, long long T, long long H, long long rank, size_t* off);

hipError_t launch_layer_fwd(const LayerWeights& W, const bf16_t* x, bf16_t* y, int B, int T,
                            int d_model, int H, int rank, char* ws, hipStream_t stream);

}  // namespace kda
