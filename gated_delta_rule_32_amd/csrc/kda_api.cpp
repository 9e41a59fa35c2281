// kda_api.cpp -- the C ABI of libkda: argument validation and dispatch.
//
// Validation is pure host code that runs before any HIP call, so every error
// path can be exercised on a machine without a GPU.
#include "../../include/kda.h"
#include "kda_internal.h"

#include <limits.h>
#include <stdint.h>

namespace {

constexpr int kHeadDim = 128;

struct Range {
    const void* p;
    size_t bytes;
};

bool overlap(Range a, Range b) {
    if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
    const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
    return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

int check_ptr(const void* p, size_t align) {
    if (!p) return KDA_ERR_INVALID_ARG;
    if ((uintptr_t)p % align) return KDA_ERR_ALIGNMENT;
    return KDA_OK;
}

size_t elem_size(int dtype) { return dtype == KDA_BF16 ? 2 : 4; }

// Product of non-negative ints as size_t, or 0 with *ok = false on overflow
// past 2^62 (far beyond any device memory).
size_t mul3(long long a, long long b, long long c, bool* ok) {
    const long long lim = (long long)1 << 62;
    long long r = a;
    if (b && r > lim / b) { *ok = false; return 0; }
    r *= b;
    if (c && r > lim / c) { *ok = false; return 0; }
    return (size_t)(r * c);
}

}  // namespace

extern "C" {

const char* kda_status_string(int status) {
    switch (status) {
        case KDA_OK: return "ok";
        case KDA_ERR_INVALID_ARG: return "invalid argument (NULL pointer, negative size or overlapping buffers)";
        case KDA_ERR_UNSUPPORTED: return "unsupported configuration (d_k and d_v must be 128; dtype must be KDA_F32 or KDA_BF16)";
        case KDA_ERR_ALIGNMENT: return "misaligned pointer (data pointers need 16-byte alignment, beta its element size)";
        case KDA_ERR_HIP: return "HIP runtime or launch error";
        case KDA_ERR_WORKSPACE: return "workspace too small for this call (see the *_workspace_size queries)";
        default: return "unknown status";
    }
}

const char* kda_version(void) { return "0.1.0"; }

size_t kda_chunk_fwd_workspace_size(int B, int T, int H, int dk, int dv, int dtype)
{
    if (B <= 0 || T <= 0 || H <= 0 || dk != kHeadDim || dv != kHeadDim || dtype != KDA_BF16) return 0;
    if (!kda::chunk_prefers_two_kernel(B, T, H, dtype)) return 0;
    return kda::chunk_fwd_ws_bytes(B, T, H);
}

size_t kda_chunk_fwd_scan_workspace_size(int B, int T, int H, int dk, int dv, int dtype)
{
    if (B <= 0 || T <= 0 || H <= 0 || dk != kHeadDim || dv != kHeadDim || dtype != KDA_BF16) return 0;
    return kda::chunk_ws_bytes(B, T, H);
}

size_t kda_chunk_fwd_block_bytes(void) { return kda::chunk_ws_bytes(1, 1, 1); }

int kda_chunk_fwd(const void* q, const void* k, const void* v,
                  const float* log_alpha, const void* beta, const float* S0,
                  void* o, float* S_T,
                  int B, int T, int H, int dk, int dv, int dtype,
                  void* workspace, size_t workspace_bytes, void* stream)
{
    return kda_chunk_fwd_gated(q, k, v, log_alpha, KDA_GATE_CHANNEL, beta, S0, o, S_T, B, T, H, dk, dv,
                               dtype, workspace, workspace_bytes, stream);
}

int kda_chunk_fwd_gated(const void* q, const void* k, const void* v,
                        const float* log_alpha, int gate, const void* beta, const float* S0,
                        void* o, float* S_T,
                        int B, int T, int H, int dk, int dv, int dtype,
                        void* workspace, size_t workspace_bytes, void* stream)
{
    return kda::chunk_fwd_entry(q, k, v, log_alpha, gate, beta, S0, o, S_T, B, T, H, dk, dv, dtype, workspace,
                                workspace_bytes, 0, stream);
}

}  // extern "C"

// The body of kda_chunk_fwd_gated.  With scratch_bytes > 0 (the
// allocation-free entry point) `workspace` is ignored: once the arguments
// have passed validation, a schedule that wants scratch takes scratch_bytes
// of the library's static array (kda::noalloc_scratch) instead.
int kda::chunk_fwd_entry(const void* q, const void* k, const void* v,
                         const float* log_alpha, int gate, const void* beta, const float* S0,
                         void* o, float* S_T,
                         int B, int T, int H, int dk, int dv, int dtype,
                         void* workspace, size_t workspace_bytes, size_t scratch_bytes, void* stream)
{
    if (B < 0 || T < 0 || H < 0) return KDA_ERR_INVALID_ARG;
    if (dtype != KDA_F32 && dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (gate != KDA_GATE_CHANNEL && gate != KDA_GATE_HEAD && gate != KDA_GATE_NONE) return KDA_ERR_UNSUPPORTED;
    if (dk != kHeadDim || dv != kHeadDim) return KDA_ERR_UNSUPPORTED;
    if ((long long)B * H == 0) return KDA_OK;

    bool ok = true;
    const size_t es = elem_size(dtype);
    const size_t tok = mul3(B, T, H, &ok);            // tokens x heads
    const size_t heads = mul3(B, H, 1, &ok);
    const size_t n_qk = mul3((long long)tok, kHeadDim, 1, &ok);
    const size_t n_state = mul3((long long)heads, kHeadDim, kHeadDim, &ok);
    if (!ok) return KDA_ERR_UNSUPPORTED;
    if (heads * 64 > (size_t)INT_MAX) return KDA_ERR_UNSUPPORTED;  // grid size

    int rc;
    if (S0 && (rc = check_ptr(S0, 16)) != KDA_OK) return rc;
    if (S_T && (rc = check_ptr(S_T, 16)) != KDA_OK) return rc;
    const Range rS0{S0, S0 ? n_state * 4 : 0}, rST{S_T, S_T ? n_state * 4 : 0};
    // gate input: per channel, per head, or none (must be NULL)
    const size_t g_bytes = gate == KDA_GATE_CHANNEL ? n_qk * 4 : gate == KDA_GATE_HEAD ? tok * 4 : 0;
    if (gate == KDA_GATE_NONE && log_alpha) return KDA_ERR_INVALID_ARG;
    if (T > 0) {
        if ((rc = check_ptr(q, 16)) || (rc = check_ptr(k, 16)) || (rc = check_ptr(v, 16)) ||
            (gate != KDA_GATE_NONE && (rc = check_ptr(log_alpha, gate == KDA_GATE_CHANNEL ? 16 : 4))) ||
            (rc = check_ptr(beta, es)) || (rc = check_ptr(o, 16)))
            return rc;
        const Range in[] = {{q, n_qk * es}, {k, n_qk * es}, {v, n_qk * es},
                            {log_alpha, g_bytes}, {beta, tok * es}, rS0};
        const Range ro{o, n_qk * es};
        for (const Range& r : in)
            if (overlap(ro, r)) return KDA_ERR_INVALID_ARG;
        if (overlap(ro, rST)) return KDA_ERR_INVALID_ARG;
        for (int i = 0; i < 5; ++i)
            if (overlap(rST, in[i])) return KDA_ERR_INVALID_ARG;
    }
    // S_T may coincide with S0 exactly (in-place update), never partially.
    if (overlap(rS0, rST) && (const void*)S0 != (const void*)S_T) return KDA_ERR_INVALID_ARG;

    // two-kernel schedule when a large enough workspace is supplied (bf16)
    void* ws = nullptr;
    bool seg = false;
    const long long grid_prep = (long long)heads * ((T + 63) / 64);
    if (scratch_bytes > 0) {
        workspace = nullptr;
        if (T > 0 && dtype == KDA_BF16) {
            if (scratch_bytes < kda::chunk_ws_bytes(B, T, H)) return KDA_ERR_WORKSPACE;
            if (grid_prep > INT_MAX) return KDA_ERR_UNSUPPORTED;
            hipError_t e;
            ws = kda::noalloc_scratch(&e);
            if (!ws) return KDA_ERR_HIP;
            seg = scratch_bytes >= kda::chunk_fwd_ws_bytes(B, T, H);
        }
    }
    if (T > 0 && workspace && dtype == KDA_BF16) {
        if (workspace_bytes < kda::chunk_ws_bytes(B, T, H)) return KDA_ERR_WORKSPACE;
        if (grid_prep > INT_MAX) return KDA_ERR_UNSUPPORTED;
        if ((rc = check_ptr(workspace, 256)) != KDA_OK) return rc;
        // with room for the segment buffers too, the scan may run in segments
        seg = workspace_bytes >= kda::chunk_fwd_ws_bytes(B, T, H);
        const Range rw{workspace, seg ? kda::chunk_fwd_ws_bytes(B, T, H) : kda::chunk_ws_bytes(B, T, H)};
        const Range all[] = {{q, n_qk * es}, {k, n_qk * es}, {v, n_qk * es}, {log_alpha, g_bytes},
                             {beta, tok * es}, rS0, rST, {o, n_qk * es}};
        for (const Range& r : all)
            if (overlap(rw, r)) return KDA_ERR_INVALID_ARG;
        ws = workspace;
    }

    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    if (T == 0) {
        if (!S_T || (const void*)S0 == (const void*)S_T) return KDA_OK;
        e = kda::launch_state_copy(S0, S_T, (long long)heads, s);
    } else {
        e = kda::launch_chunk_fwd(q, k, v, log_alpha, beta, S0, o, S_T, B, T, H, dtype, ws, s, gate, nullptr, seg);
    }
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

extern "C" {

size_t kda_chunk_bwd_workspace_size(int B, int T, int H, int dk, int dv, int dtype)
{
    if (B < 0 || T < 0 || H < 0 || dk != kHeadDim || dv != kHeadDim || dtype != KDA_BF16) return 0;
    return kda::chunk_bwd_ws_layout(B, T, H, nullptr);
}

int kda_chunk_bwd(const void* q, const void* k, const void* v,
                  const float* log_alpha, const void* beta, const float* S0,
                  const void* grad_o, const float* grad_S_T,
                  void* grad_q, void* grad_k, void* grad_v, float* grad_log_alpha,
                  void* grad_beta, float* grad_S0,
                  int B, int T, int H, int dk, int dv, int dtype,
                  void* workspace, size_t workspace_bytes, void* stream)
{
    return kda_chunk_bwd_gated(q, k, v, log_alpha, KDA_GATE_CHANNEL, beta, S0, grad_o, grad_S_T, grad_q,
                               grad_k, grad_v, grad_log_alpha, grad_beta, grad_S0, B, T, H, dk, dv, dtype,
                               workspace, workspace_bytes, stream);
}

int kda_chunk_bwd_gated(const void* q, const void* k, const void* v,
                        const float* log_alpha, int gate, const void* beta, const float* S0,
                        const void* grad_o, const float* grad_S_T,
                        void* grad_q, void* grad_k, void* grad_v, float* grad_log_alpha,
                        void* grad_beta, float* grad_S0,
                        int B, int T, int H, int dk, int dv, int dtype,
                        void* workspace, size_t workspace_bytes, void* stream)
{
    if (B < 0 || T < 0 || H < 0) return KDA_ERR_INVALID_ARG;
    if (dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED;   // bf16 only
    if (gate != KDA_GATE_CHANNEL && gate != KDA_GATE_HEAD && gate != KDA_GATE_NONE) return KDA_ERR_UNSUPPORTED;
    if (gate == KDA_GATE_NONE && (log_alpha || grad_log_alpha)) return KDA_ERR_INVALID_ARG;
    if (dk != kHeadDim || dv != kHeadDim) return KDA_ERR_UNSUPPORTED;
    if ((long long)B * H == 0) return KDA_OK;

    bool ok = true;
    const size_t es = 2;
    const size_t tok = mul3(B, T, H, &ok);
    const size_t heads = mul3(B, H, 1, &ok);
    const size_t n_qk = mul3((long long)tok, kHeadDim, 1, &ok);
    const size_t n_state = mul3((long long)heads, kHeadDim, kHeadDim, &ok);
    const size_t units = mul3((long long)heads, (T + 63) / 64, 1, &ok);
    if (!ok) return KDA_ERR_UNSUPPORTED;
    if (heads * 8 > (size_t)INT_MAX || units > (size_t)INT_MAX) return KDA_ERR_UNSUPPORTED;   // grids

    int rc;
    const Range rS0{S0, S0 ? n_state * 4 : 0}, rdST{grad_S_T, grad_S_T ? n_state * 4 : 0};
    const Range rdS0{grad_S0, grad_S0 ? n_state * 4 : 0};
    if (S0 && (rc = check_ptr(S0, 16)) != KDA_OK) return rc;
    if (grad_S_T && (rc = check_ptr(grad_S_T, 16)) != KDA_OK) return rc;
    if (grad_S0 && (rc = check_ptr(grad_S0, 16)) != KDA_OK) return rc;
    if (overlap(rdS0, rS0) || overlap(rdS0, rdST)) return KDA_ERR_INVALID_ARG;

    hipStream_t s = (hipStream_t)stream;
    if (T == 0) {
        if (!grad_S0) return KDA_OK;
        return kda::launch_state_copy(grad_S_T, grad_S0, (long long)heads, s) == hipSuccess ? KDA_OK
                                                                                          : KDA_ERR_HIP;
    }

    const void* ins[] = {q, k, v, grad_o, grad_q, grad_k, grad_v};
    for (const void* p : ins)
        if ((rc = check_ptr(p, 16)) != KDA_OK) return rc;
    if ((rc = check_ptr(beta, es)) != KDA_OK || (rc = check_ptr(grad_beta, es)) != KDA_OK) return rc;
    // gate input and its gradient: per channel, per head, or none (both NULL)
    const size_t g_bytes = gate == KDA_GATE_CHANNEL ? n_qk * 4 : gate == KDA_GATE_HEAD ? tok * 4 : 0;
    if (gate != KDA_GATE_NONE) {
        const size_t ga = gate == KDA_GATE_CHANNEL ? 16 : 4;
        if ((rc = check_ptr(log_alpha, ga)) != KDA_OK || (rc = check_ptr(grad_log_alpha, ga)) != KDA_OK)
            return rc;
    }
    const size_t need = kda::chunk_bwd_ws_layout(B, T, H, nullptr);
    if (!workspace) return KDA_ERR_INVALID_ARG;
    if (workspace_bytes < need) return KDA_ERR_WORKSPACE;
    if ((rc = check_ptr(workspace, 256)) != KDA_OK) return rc;

    const Range in[] = {{q, n_qk * es}, {k, n_qk * es}, {v, n_qk * es}, {log_alpha, g_bytes},
                        {beta, tok * es}, rS0, {grad_o, n_qk * es}, rdST};
    const Range out[] = {{grad_q, n_qk * es}, {grad_k, n_qk * es}, {grad_v, n_qk * es},
                         {grad_log_alpha, g_bytes}, {grad_beta, tok * es}, rdS0,
                         {workspace, need}};
    constexpr int n_out = sizeof(out) / sizeof(out[0]);
    for (int i = 0; i < n_out; ++i) {
        for (const Range& r : in)
            if (overlap(out[i], r)) return KDA_ERR_INVALID_ARG;
        for (int j = i + 1; j < n_out; ++j)
            if (overlap(out[i], out[j])) return KDA_ERR_INVALID_ARG;
    }

    hipError_t e = kda::launch_chunk_bwd(q, k, v, log_alpha, beta, S0, grad_o, grad_S_T,
                                         grad_q, grad_k, grad_v, grad_log_alpha, grad_beta, grad_S0,
                                         B, T, H, (char*)workspace, s, gate);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int kda_chunk_fwd_varlen(const void* q, const void* k, const void* v,
                         const float* log_alpha, int gate, const void* beta,
                         const int32_t* cu_seqlens, int num_seqs, const float* S0,
                         void* o, float* S_T, int total_tokens, int H, int dk, int dv,
                         int dtype, void* stream)
{
    if (num_seqs < 0 || total_tokens < 0 || H < 0) return KDA_ERR_INVALID_ARG;
    if (dtype != KDA_F32 && dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (gate != KDA_GATE_CHANNEL && gate != KDA_GATE_HEAD && gate != KDA_GATE_NONE) return KDA_ERR_UNSUPPORTED;
    if (dk != kHeadDim || dv != kHeadDim) return KDA_ERR_UNSUPPORTED;
    if ((long long)num_seqs * H == 0) return KDA_OK;

    bool ok = true;
    const size_t es = elem_size(dtype);
    const size_t tok = mul3(total_tokens, H, 1, &ok);
    const size_t heads = mul3(num_seqs, H, 1, &ok);
    const size_t n_qk = mul3((long long)tok, kHeadDim, 1, &ok);
    const size_t n_state = mul3((long long)heads, kHeadDim, kHeadDim, &ok);
    if (!ok) return KDA_ERR_UNSUPPORTED;
    if (heads * 8 > (size_t)INT_MAX) return KDA_ERR_UNSUPPORTED;   // grid size

    int rc;
    if ((rc = check_ptr(cu_seqlens, 4)) != KDA_OK) return rc;
    if (gate == KDA_GATE_NONE && log_alpha) return KDA_ERR_INVALID_ARG;
    if (S0 && (rc = check_ptr(S0, 16)) != KDA_OK) return rc;
    if (S_T && (rc = check_ptr(S_T, 16)) != KDA_OK) return rc;
    const size_t g_bytes = gate == KDA_GATE_CHANNEL ? n_qk * 4 : gate == KDA_GATE_HEAD ? tok * 4 : 0;
    const Range rS0{S0, S0 ? n_state * 4 : 0}, rST{S_T, S_T ? n_state * 4 : 0};
    const Range rcu{cu_seqlens, ((size_t)num_seqs + 1) * 4};
    if (total_tokens > 0) {
        if ((rc = check_ptr(q, 16)) || (rc = check_ptr(k, 16)) || (rc = check_ptr(v, 16)) ||
            (gate != KDA_GATE_NONE && (rc = check_ptr(log_alpha, gate == KDA_GATE_CHANNEL ? 16 : 4))) ||
            (rc = check_ptr(beta, es)) || (rc = check_ptr(o, 16)))
            return rc;
    }
    const Range in[] = {{q, n_qk * es}, {k, n_qk * es}, {v, n_qk * es}, {log_alpha, g_bytes},
                        {beta, tok * es}, rS0, rcu};
    const Range ro{total_tokens > 0 ? o : nullptr, n_qk * es};
    for (const Range& r : in)
        if (overlap(ro, r)) return KDA_ERR_INVALID_ARG;
    if (overlap(ro, rST)) return KDA_ERR_INVALID_ARG;
    for (int i = 0; i < 5; ++i)
        if (overlap(rST, in[i])) return KDA_ERR_INVALID_ARG;
    if (overlap(rST, rcu)) return KDA_ERR_INVALID_ARG;
    if (overlap(rS0, rST) && (const void*)S0 != (const void*)S_T) return KDA_ERR_INVALID_ARG;

    hipError_t e = kda::launch_chunk_fwd(q, k, v, log_alpha, beta, S0, o, S_T, num_seqs, total_tokens, H,
                                         dtype, nullptr, (hipStream_t)stream, gate, cu_seqlens);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int kda_recurrent_step(const void* q, const void* k, const void* v,
                       const float* log_alpha, const void* beta, float* S,
                       void* o, int N, int H, int dk, int dv, int dtype,
                       void* stream)
{
    return kda_recurrent_step_gated(q, k, v, log_alpha, KDA_GATE_CHANNEL, beta, S, o, N, H, dk, dv,
                                    dtype, stream);
}

int kda_recurrent_step_gated(const void* q, const void* k, const void* v,
                             const float* log_alpha, int gate, const void* beta, float* S,
                             void* o, int N, int H, int dk, int dv, int dtype,
                             void* stream)
{
    if (N < 0 || H < 0) return KDA_ERR_INVALID_ARG;
    if (dtype != KDA_F32 && dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (gate != KDA_GATE_CHANNEL && gate != KDA_GATE_HEAD && gate != KDA_GATE_NONE) return KDA_ERR_UNSUPPORTED;
    if (dk != kHeadDim || dv != kHeadDim) return KDA_ERR_UNSUPPORTED;
    if ((long long)N * H == 0) return KDA_OK;

    bool ok = true;
    const size_t es = elem_size(dtype);
    const size_t heads = mul3(N, H, 1, &ok);
    const size_t n_vec = mul3((long long)heads, kHeadDim, 1, &ok);
    const size_t n_state = mul3((long long)heads, kHeadDim, kHeadDim, &ok);
    if (!ok || heads > (size_t)INT_MAX) return KDA_ERR_UNSUPPORTED;

    int rc;
    if (gate == KDA_GATE_NONE && log_alpha) return KDA_ERR_INVALID_ARG;
    if ((rc = check_ptr(q, 16)) || (rc = check_ptr(k, 16)) || (rc = check_ptr(v, 16)) ||
        (gate != KDA_GATE_NONE && (rc = check_ptr(log_alpha, gate == KDA_GATE_CHANNEL ? 16 : 4))) ||
        (rc = check_ptr(beta, es)) || (rc = check_ptr(S, 16)) || (rc = check_ptr(o, 16)))
        return rc;
    const size_t g_bytes = gate == KDA_GATE_CHANNEL ? n_vec * 4 : gate == KDA_GATE_HEAD ? heads * 4 : 0;
    const Range in[] = {{q, n_vec * es}, {k, n_vec * es}, {v, n_vec * es},
                        {log_alpha, g_bytes}, {beta, heads * es}};
    const Range rS{S, n_state * 4}, ro{o, n_vec * es};
    for (const Range& r : in)
        if (overlap(rS, r) || overlap(ro, r)) return KDA_ERR_INVALID_ARG;
    if (overlap(rS, ro)) return KDA_ERR_INVALID_ARG;

    hipError_t e = kda::launch_decode_step(q, k, v, log_alpha, beta, S, o,
                                           (long long)heads, dtype, (hipStream_t)stream, gate);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int kda_recurrent_steps(const void* q, const void* k, const void* v,
                        const float* log_alpha, int gate, const void* beta, const int32_t* accept,
                        float* S, void* o, int N, int m, int H, int dk, int dv, int dtype, void* stream)
{
    if (N < 0 || m < 0 || H < 0) return KDA_ERR_INVALID_ARG;
    if (dtype != KDA_F32 && dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (gate != KDA_GATE_CHANNEL && gate != KDA_GATE_HEAD && gate != KDA_GATE_NONE) return KDA_ERR_UNSUPPORTED;
    if (dk != kHeadDim || dv != kHeadDim) return KDA_ERR_UNSUPPORTED;
    if ((long long)N * H == 0 || m == 0) return KDA_OK;

    bool ok = true;
    const size_t es = elem_size(dtype);
    const size_t heads = mul3(N, H, 1, &ok);
    const size_t toks = mul3(N, m, H, &ok);                 // (sequence, token, head) entries
    const size_t n_vec = mul3((long long)toks, kHeadDim, 1, &ok);
    const size_t n_state = mul3((long long)heads, kHeadDim, kHeadDim, &ok);
    if (!ok || heads > (size_t)INT_MAX) return KDA_ERR_UNSUPPORTED;

    int rc;
    if (gate == KDA_GATE_NONE && log_alpha) return KDA_ERR_INVALID_ARG;
    if ((rc = check_ptr(q, 16)) || (rc = check_ptr(k, 16)) || (rc = check_ptr(v, 16)) ||
        (gate != KDA_GATE_NONE && (rc = check_ptr(log_alpha, gate == KDA_GATE_CHANNEL ? 16 : 4))) ||
        (rc = check_ptr(beta, es)) || (rc = check_ptr(S, 16)))
        return rc;
    if (o && (rc = check_ptr(o, 16))) return rc;
    if (accept && (rc = check_ptr(accept, 4))) return rc;
    const size_t g_bytes = gate == KDA_GATE_CHANNEL ? n_vec * 4 : gate == KDA_GATE_HEAD ? toks * 4 : 0;
    const Range in[] = {{q, n_vec * es}, {k, n_vec * es}, {v, n_vec * es},
                        {log_alpha, g_bytes}, {beta, toks * es}, {accept, accept ? (size_t)N * 4 : 0}};
    const Range rS{S, n_state * 4}, ro{o, o ? n_vec * es : 0};
    for (const Range& r : in)
        if (overlap(rS, r) || overlap(ro, r)) return KDA_ERR_INVALID_ARG;
    if (overlap(rS, ro)) return KDA_ERR_INVALID_ARG;

    hipError_t e = kda::launch_decode_steps(q, k, v, log_alpha, beta, accept, S, o, (long long)heads, m, H, dtype,
                                            (hipStream_t)stream, gate);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

size_t kda_mqa_decode_workspace_size(int B, int T, int H, int D)
{
    if (B < 0 || T < 1 || T > (1 << 22) || (H != 16 && H != 32) || D != 512) return 0;
    return kda::mqa_ws_bytes(B, T, H);
}

int kda_mqa_decode(const void* q, const void* cache, void* o, int B, int T, int H, int D,
                   float scale, void* workspace, size_t workspace_bytes, void* stream)
{
    if (B < 0 || T < 0) return KDA_ERR_INVALID_ARG;
    if (D != 512 || (H != 16 && H != 32)) return KDA_ERR_UNSUPPORTED;
    if (B == 0) return KDA_OK;
    if (T < 1) return KDA_ERR_INVALID_ARG;
    bool ok = true;
    const size_t nq = mul3(B, H, D, &ok) * 2;
    const size_t nc = mul3(B, T, D, &ok) * 2;
    if (!ok || B > 65535 || T > (1 << 22)) return KDA_ERR_UNSUPPORTED;   // at most 1024 splits of 4096
    int rc;
    if ((rc = check_ptr(q, 16)) || (rc = check_ptr(cache, 16)) || (rc = check_ptr(o, 16))) return rc;
    const size_t need = kda::mqa_ws_bytes(B, T, H);
    if (!workspace) return KDA_ERR_INVALID_ARG;
    if (workspace_bytes < need) return KDA_ERR_WORKSPACE;
    if ((rc = check_ptr(workspace, 256)) != KDA_OK) return rc;
    const Range rq{q, nq}, rc_{cache, nc}, ro{o, nq}, rw{workspace, need};
    if (overlap(ro, rq) || overlap(ro, rc_) || overlap(ro, rw) || overlap(rw, rq) || overlap(rw, rc_))
        return KDA_ERR_INVALID_ARG;
    hipError_t e = kda::launch_mqa_decode(q, cache, o, B, T, H, scale, workspace, (hipStream_t)stream);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

size_t kda_dplr_chunk_fwd_workspace_size(int B, int T, int H, int dk, int dv, int dtype)
{
    if (B < 0 || T < 0 || H < 0 || dk != kHeadDim || dv != kHeadDim || dtype != KDA_BF16) return 0;
    return kda::dplr_ws_layout(B, T, H, nullptr);
}

int kda_dplr_chunk_fwd(const void* q, const void* k, const void* v, const void* a, const void* b,
                       const float* log_alpha, const float* S0, void* o, float* S_T,
                       int B, int T, int H, int dk, int dv, int dtype,
                       void* workspace, size_t workspace_bytes, void* stream)
{
    if (B < 0 || T < 0 || H < 0) return KDA_ERR_INVALID_ARG;
    if (dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED;   // bf16 only
    if (dk != kHeadDim || dv != kHeadDim) return KDA_ERR_UNSUPPORTED;
    if ((long long)B * H == 0) return KDA_OK;

    bool ok = true;
    const size_t tok = mul3(B, T, H, &ok);
    const size_t heads = mul3(B, H, 1, &ok);
    const size_t n_qk = mul3((long long)tok, kHeadDim, 1, &ok);
    const size_t n_state = mul3((long long)heads, kHeadDim, kHeadDim, &ok);
    const size_t units = mul3((long long)heads, (T + 63) / 64, 1, &ok);
    if (!ok) return KDA_ERR_UNSUPPORTED;
    if (heads * 8 > (size_t)INT_MAX || units > (size_t)INT_MAX) return KDA_ERR_UNSUPPORTED;   // grids

    int rc;
    if (S0 && (rc = check_ptr(S0, 16)) != KDA_OK) return rc;
    if (S_T && (rc = check_ptr(S_T, 16)) != KDA_OK) return rc;
    const Range rS0{S0, S0 ? n_state * 4 : 0}, rST{S_T, S_T ? n_state * 4 : 0};
    // S_T may coincide with S0 exactly (in-place update), never partially.
    if (overlap(rS0, rST) && (const void*)S0 != (const void*)S_T) return KDA_ERR_INVALID_ARG;
    hipStream_t s = (hipStream_t)stream;
    if (T == 0) {
        if (!S_T || (const void*)S0 == (const void*)S_T) return KDA_OK;
        return kda::launch_state_copy(S0, S_T, (long long)heads, s) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
    }

    const void* ptrs[] = {q, k, v, a, b, log_alpha, o};
    for (const void* p : ptrs)
        if ((rc = check_ptr(p, 16)) != KDA_OK) return rc;
    const size_t need = kda::dplr_ws_layout(B, T, H, nullptr);
    if (!workspace) return KDA_ERR_INVALID_ARG;
    if (workspace_bytes < need) return KDA_ERR_WORKSPACE;
    if ((rc = check_ptr(workspace, 256)) != KDA_OK) return rc;
    const Range in[] = {{q, n_qk * 2}, {k, n_qk * 2}, {v, n_qk * 2}, {a, n_qk * 2},
                        {b, n_qk * 2}, {log_alpha, n_qk * 4}, rS0};
    const Range out[] = {{o, n_qk * 2}, rST, {workspace, need}};
    for (int i = 0; i < 3; ++i) {
        for (const Range& r : in)
            if (overlap(out[i], r) && !(i == 1 && r.p == (const void*)S0)) return KDA_ERR_INVALID_ARG;
        for (int j = i + 1; j < 3; ++j)
            if (overlap(out[i], out[j])) return KDA_ERR_INVALID_ARG;
    }
    hipError_t e = kda::launch_dplr_chunk_fwd(q, k, v, a, b, log_alpha, S0, o, S_T, B, T, H,
                                              (char*)workspace, s);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

size_t kda_layer_workspace_layout(int B, int T, int d_model, int H, int rank, size_t* offsets)
{
    if (B < 0 || T < 0 || H <= 0 || d_model <= 0 || rank <= 0) return 0;
    if (d_model % 64 || rank % 64) return 0;
    const long long elems = (long long)B * T * 4 * H * kHeadDim;
    if (elems >= ((long long)1 << 31)) return 0;
    return kda::layer_ws_layout(B, T, H, rank, offsets);
}

int kda_layer_fwd(const void* x, const void* W_q, const void* W_k, const void* W_v,
                  const void* W_g, const void* conv_q, const void* conv_k, const void* conv_v,
                  const void* W_down, const void* W_up, const void* W_beta, const void* W_o,
                  void* y, int B, int T, int d_model, int H, int rank,
                  void* workspace, size_t workspace_bytes, void* stream)
{
    if (B < 0 || T < 0 || H <= 0 || d_model <= 0 || rank <= 0) return KDA_ERR_INVALID_ARG;
    if (d_model % 64 || rank % 64) return KDA_ERR_UNSUPPORTED;
    const long long R = (long long)B * T, HDm = (long long)H * kHeadDim;
    if (R * 4 * HDm >= ((long long)1 << 31)) return KDA_ERR_UNSUPPORTED;
    if (R == 0) return KDA_OK;

    const size_t need = kda::layer_ws_layout(B, T, H, rank, nullptr);
    if (!workspace) return KDA_ERR_INVALID_ARG;
    if (workspace_bytes < need) return KDA_ERR_WORKSPACE;
    int rc;
    const void* ptrs[] = {x, W_q, W_k, W_v, W_g, conv_q, conv_k, conv_v, W_down, W_up, W_beta, W_o, y};
    for (const void* p : ptrs)
        if ((rc = check_ptr(p, 16)) != KDA_OK) return rc;
    if ((rc = check_ptr(workspace, 256)) != KDA_OK) return rc;
    const size_t dm = (size_t)d_model, hd = (size_t)HDm, r = (size_t)rank;
    const Range in[] = {{x, (size_t)R * dm * 2},   {W_q, hd * dm * 2},    {W_k, hd * dm * 2},
                        {W_v, hd * dm * 2},        {W_g, hd * dm * 2},    {conv_q, hd * 8},
                        {conv_k, hd * 8},          {conv_v, hd * 8},      {W_down, r * dm * 2},
                        {W_up, hd * r * 2},        {W_beta, (size_t)H * dm * 2},
                        {W_o, dm * hd * 2}};
    const Range ry{y, (size_t)R * dm * 2}, rw{workspace, need};
    for (const Range& a : in)
        if (overlap(ry, a) || overlap(rw, a)) return KDA_ERR_INVALID_ARG;
    if (overlap(ry, rw)) return KDA_ERR_INVALID_ARG;

    typedef const kda::bf16_t* P;
    const kda::LayerWeights Wt{(P)W_q, (P)W_k, (P)W_v, (P)W_g, (P)conv_q, (P)conv_k,
                               (P)conv_v, (P)W_down, (P)W_up, (P)W_beta, (P)W_o};
    hipError_t e = kda::launch_layer_fwd(Wt, (P)x, (kda::bf16_t*)y, B, T, d_model, H, rank,
                                         (char*)workspace, (hipStream_t)stream);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // extern "C"
