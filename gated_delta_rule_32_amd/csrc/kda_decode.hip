// kda_decode.hip -- recurrent KDA decode step for gfx950.
//
// One token per head: eq. (1) on page "Kimi K3论文：Kimi Linear" (section 3),
// applied once.  Section 4 of the same page notes that decoding switches from
// the chunk kernel to a cheaper recurrent kernel whose state does not grow
// with the context; this is that kernel.
//
// Per head, with S' = Diag(alpha) S:
//     r = S'^T k,   s = S'^T q,   u = beta (v - r)
//     S <- S' + k u^T
//     o  = S^T q = s + (k . q) u
// The last line avoids a second pass over the state: the read-out after the
// write is the read-out before it plus the rank-1 term.
//
// The step is HBM-bound (about 0.9 FLOP per byte): each head streams its
// 128 x 128 fp32 state (64 KiB) in once and out once.  One 1024-thread
// workgroup owns one head and keeps its whole state in registers between the
// reduction and the write-back, so the state crosses HBM exactly twice.
//   thread t: column group cg = t % 32 (columns 4cg .. 4cg+3),
//             row group    rg = t / 32 (rows rg, rg+32, rg+64, rg+96)
// Each load/store instruction of the workgroup covers 32 whole rows (16 KiB
// contiguous), 16 B per lane.  Every thread reads the k, q and g entries of
// its own four rows straight from memory (the 32 lanes of a row group read
// the same address), and each wave forms k . q with shuffles, so the only
// barrier is the one that combines the 16 waves' partial sums of S'^T k and
// S'^T q.  The small token loads are issued before the state loads.
//
// GATE: per-channel decay (KDA, g [heads, 128]), one decay per head (Gated
// DeltaNet, g [heads]) or none (DeltaNet, alpha = 1, g unused).
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

constexpr int DEC_THREADS = 1024;

constexpr int GATE_CHANNEL = 0, GATE_HEAD = 1, GATE_NONE = 2;

template <typename TI, int GATE>
__global__ void __launch_bounds__(DEC_THREADS)
decode_step_kernel(const TI* __restrict__ q, const TI* __restrict__ k,
                   const TI* __restrict__ v, const float* __restrict__ g,
                   const TI* __restrict__ beta, float* __restrict__ S,
                   TI* __restrict__ o)
{
    constexpr int D = 128, RG = DEC_THREADS / 32, RPT = D / RG, NWV = DEC_THREADS / 64;
    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int cg = t & 31, rg = t >> 5;
    const size_t head = blockIdx.x;
    const size_t vbase = head * D;

    __shared__ f32x4 s_part[NWV][2][32];   // per-wave partial r and s, 4 columns per entry

    float rk[RPT], rq[RPT], rg_[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int row = rg + RG * i;
        rk[i] = to_f32(k[vbase + row]);
        rq[i] = to_f32(q[vbase + row]);
        if constexpr (GATE == GATE_CHANNEL) rg_[i] = g[vbase + row];
    }
    if constexpr (GATE == GATE_HEAD) {
        const float gh = g[head];
#pragma unroll
        for (int i = 0; i < RPT; ++i) rg_[i] = gh;
    }
    float kq = to_f32(k[vbase + lane]) * to_f32(q[vbase + lane]) +
               to_f32(k[vbase + lane + 64]) * to_f32(q[vbase + lane + 64]);
    const f32x4 vv = load4(v + vbase + 4 * cg);
    const float b = to_f32(beta[head]);

    f32x4 st[RPT];
    const f32x4* Sin = reinterpret_cast<const f32x4*>(S + head * (D * D));
#pragma unroll
    for (int i = 0; i < RPT; ++i) st[i] = __builtin_nontemporal_load(&Sin[(rg + RG * i) * 32 + cg]);

#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) kq += __shfl_xor(kq, off);

    f32x4 r = {0.f, 0.f, 0.f, 0.f}, s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        if constexpr (GATE != GATE_NONE) st[i] *= exp_fast(rg_[i]);
        r += st[i] * rk[i];
        s += st[i] * rq[i];
    }
    // lanes l and l^32 of a wave hold the same columns for row groups 2w, 2w+1
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        r[c] += __shfl_xor(r[c], 32);
        s[c] += __shfl_xor(s[c], 32);
    }
    if (lane < 32) { s_part[wave][0][cg] = r; s_part[wave][1][cg] = s; }
    __syncthreads();

    r = s_part[0][0][cg];
    s = s_part[0][1][cg];
#pragma unroll
    for (int w = 1; w < NWV; ++w) {
        r += s_part[w][0][cg];
        s += s_part[w][1][cg];
    }
    const f32x4 u = b * (vv - r);
    if (rg == 0) store4(o + vbase + 4 * cg, s + kq * u);

    f32x4* Sout = reinterpret_cast<f32x4*>(S + head * (D * D));
#pragma unroll
    for (int i = 0; i < RPT; ++i)
        __builtin_nontemporal_store(st[i] + rk[i] * u, &Sout[(rg + RG * i) * 32 + cg]);
}

// m tokens per head in one launch (multi-token and speculative decoding, page
// "Kimi K3论文：Kimi Linear", section 8: the kernel inside a serving engine):
// the same step as decode_step_kernel, applied to tokens 0 .. cnt-1 of the
// head's sequence with the state kept in registers in between, so the state
// crosses HBM twice however many tokens are applied.  cnt = m, or accept[n]
// clamped to [0, m] (the accepted prefix of m drafted tokens).  Token i of
// sequence n, head h sits at [n, i, h, :]; o (optional) gets the applied
// tokens' outputs.  The partial sums of each step go through one of two LDS
// buffers in turn, so one barrier per token orders them.
template <typename TI, int GATE>
__global__ void __launch_bounds__(DEC_THREADS)
decode_steps_kernel(const TI* __restrict__ q, const TI* __restrict__ k,
                    const TI* __restrict__ v, const float* __restrict__ g,
                    const TI* __restrict__ beta, const int* __restrict__ accept, float* __restrict__ S,
                    TI* __restrict__ o, int m, int H)
{
    constexpr int D = 128, RG = DEC_THREADS / 32, RPT = D / RG, NWV = DEC_THREADS / 64;
    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int cg = t & 31, rg = t >> 5;
    const size_t head = blockIdx.x;               // n * H + h
    const size_t n = head / H, h = head % H;
    int cnt = m;
    if (accept) cnt = min(max(accept[n], 0), m);
    cnt = __builtin_amdgcn_readfirstlane(cnt);

    __shared__ f32x4 s_part[2][NWV][2][32];

    f32x4 st[RPT];
    const f32x4* Sin = reinterpret_cast<const f32x4*>(S + head * (D * D));
#pragma unroll
    for (int i = 0; i < RPT; ++i) st[i] = __builtin_nontemporal_load(&Sin[(rg + RG * i) * 32 + cg]);

    for (int i = 0; i < cnt; ++i) {
        const size_t tok = (n * m + i) * H + h;   // (sequence, token, head)
        const size_t vbase = tok * D;
        float rk[RPT], rq[RPT], rg_[RPT];
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
            const int row = rg + RG * j;
            rk[j] = to_f32(k[vbase + row]);
            rq[j] = to_f32(q[vbase + row]);
            if constexpr (GATE == GATE_CHANNEL) rg_[j] = g[vbase + row];
        }
        if constexpr (GATE == GATE_HEAD) {
            const float gh = g[tok];
#pragma unroll
            for (int j = 0; j < RPT; ++j) rg_[j] = gh;
        }
        float kq = to_f32(k[vbase + lane]) * to_f32(q[vbase + lane]) +
                   to_f32(k[vbase + lane + 64]) * to_f32(q[vbase + lane + 64]);
        const f32x4 vv = load4(v + vbase + 4 * cg);
        const float b = to_f32(beta[tok]);
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) kq += __shfl_xor(kq, off);

        f32x4 r = {0.f, 0.f, 0.f, 0.f}, s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
            if constexpr (GATE != GATE_NONE) st[j] *= exp_fast(rg_[j]);
            r += st[j] * rk[j];
            s += st[j] * rq[j];
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            r[c] += __shfl_xor(r[c], 32);
            s[c] += __shfl_xor(s[c], 32);
        }
        // buffer i % 2: the previous use of this buffer (token i - 2) was read
        // before the barrier of token i - 1
        if (lane < 32) { s_part[i & 1][wave][0][cg] = r; s_part[i & 1][wave][1][cg] = s; }
        __syncthreads();
        r = s_part[i & 1][0][0][cg];
        s = s_part[i & 1][0][1][cg];
#pragma unroll
        for (int w = 1; w < NWV; ++w) {
            r += s_part[i & 1][w][0][cg];
            s += s_part[i & 1][w][1][cg];
        }
        const f32x4 u = b * (vv - r);
        if (o && rg == 0) store4(o + vbase + 4 * cg, s + kq * u);
#pragma unroll
        for (int j = 0; j < RPT; ++j) st[j] += rk[j] * u;
    }

    if (cnt > 0) {
        f32x4* Sout = reinterpret_cast<f32x4*>(S + head * (D * D));
#pragma unroll
        for (int i = 0; i < RPT; ++i) __builtin_nontemporal_store(st[i], &Sout[(rg + RG * i) * 32 + cg]);
    }
}

template <int GATE>
void launch_steps_gate(const void* q, const void* k, const void* v, const float* g, const void* beta,
                       const int* accept, float* S, void* o, long long heads, int m, int H, int dtype,
                       hipStream_t stream)
{
    const dim3 grid((unsigned)heads), block(DEC_THREADS);
    if (dtype == 1) {
        hipLaunchKernelGGL((decode_steps_kernel<bf16_t, GATE>), grid, block, 0, stream,
                           (const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v, g,
                           (const bf16_t*)beta, accept, S, (bf16_t*)o, m, H);
    } else {
        hipLaunchKernelGGL((decode_steps_kernel<float, GATE>), grid, block, 0, stream,
                           (const float*)q, (const float*)k, (const float*)v, g,
                           (const float*)beta, accept, S, (float*)o, m, H);
    }
}

hipError_t launch_decode_steps(const void* q, const void* k, const void* v, const float* g, const void* beta,
                               const int* accept, float* S, void* o, long long heads, int m, int H, int dtype,
                               hipStream_t stream, int gate)
{
    if (heads <= 0 || m <= 0) return hipSuccess;
    if (gate == GATE_HEAD) launch_steps_gate<GATE_HEAD>(q, k, v, g, beta, accept, S, o, heads, m, H, dtype, stream);
    else if (gate == GATE_NONE) launch_steps_gate<GATE_NONE>(q, k, v, g, beta, accept, S, o, heads, m, H, dtype, stream);
    else launch_steps_gate<GATE_CHANNEL>(q, k, v, g, beta, accept, S, o, heads, m, H, dtype, stream);
    return hipGetLastError();
}

template <int GATE>
void launch_decode_gate(const void* q, const void* k, const void* v, const float* g, const void* beta,
                        float* S, void* o, long long heads, int dtype, hipStream_t stream)
{
    const dim3 grid((unsigned)heads), block(DEC_THREADS);
    if (dtype == 1) {
        hipLaunchKernelGGL((decode_step_kernel<bf16_t, GATE>), grid, block, 0, stream,
                           (const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v, g,
                           (const bf16_t*)beta, S, (bf16_t*)o);
    } else {
        hipLaunchKernelGGL((decode_step_kernel<float, GATE>), grid, block, 0, stream,
                           (const float*)q, (const float*)k, (const float*)v, g,
                           (const float*)beta, S, (float*)o);
    }
}

hipError_t launch_decode_step(const void* q, const void* k, const void* v,
                              const float* g, const void* beta, float* S, void* o,
                              long long heads, int dtype, hipStream_t stream, int gate)
{
    if (heads <= 0) return hipSuccess;
    if (gate == GATE_HEAD) launch_decode_gate<GATE_HEAD>(q, k, v, g, beta, S, o, heads, dtype, stream);
    else if (gate == GATE_NONE) launch_decode_gate<GATE_NONE>(q, k, v, g, beta, S, o, heads, dtype, stream);
    else launch_decode_gate<GATE_CHANNEL>(q, k, v, g, beta, S, o, heads, dtype, stream);
    return hipGetLastError();
}

}  // namespace kda
