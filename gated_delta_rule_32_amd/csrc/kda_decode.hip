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
// 128 x 128 fp32 state (64 KiB) in once and out once.  One 256-thread
// workgroup owns one head and keeps its whole state in registers between the
// reduction and the write-back, so the state crosses HBM exactly twice.
//   thread t: column group cg = t % 32 (columns 4cg .. 4cg+3),
//             row group    rg = t / 32 (rows rg, rg+8, ..., rg+120)
// Every load/store instruction of the workgroup covers 8 whole rows (4 KiB
// contiguous), 16 B per lane.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

template <typename TI>
__global__ void __launch_bounds__(256)
decode_step_kernel(const TI* __restrict__ q, const TI* __restrict__ k,
                   const TI* __restrict__ v, const float* __restrict__ g,
                   const TI* __restrict__ beta, float* __restrict__ S,
                   TI* __restrict__ o)
{
    constexpr int D = 128;
    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int cg = t & 31, rg = t >> 5;
    const size_t head = blockIdx.x;
    const size_t vbase = head * D;

    __shared__ float s_k[D], s_q[D], s_a[D];
    __shared__ f32x4 s_part[4][2][32];   // per-wave partial r and s, 4 columns per entry
    __shared__ float s_kq;

    // Issue the 16 state loads first so they overlap everything else.
    f32x4 st[16];
    const f32x4* Sin = reinterpret_cast<const f32x4*>(S + head * (D * D));
#pragma unroll
    for (int i = 0; i < 16; ++i) st[i] = __builtin_nontemporal_load(&Sin[(rg + 8 * i) * 32 + cg]);

    if (t < D) {
        s_k[t] = to_f32(k[vbase + t]);
        s_q[t] = to_f32(q[vbase + t]);
        s_a[t] = exp_fast(g[vbase + t]);
    }
    const f32x4 vv = load4(v + vbase + 4 * cg);
    const float b = to_f32(beta[head]);
    __syncthreads();

    if (wave == 0) {   // k . q, one wave
        float p = s_k[lane] * s_q[lane] + s_k[lane + 64] * s_q[lane + 64];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) p += __shfl_xor(p, off);
        if (lane == 0) s_kq = p;
    }

    f32x4 r = {0.f, 0.f, 0.f, 0.f}, s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int row = rg + 8 * i;
        st[i] *= s_a[row];
        r += st[i] * s_k[row];
        s += st[i] * s_q[row];
    }
    // lanes l and l^32 of a wave hold the same columns for row groups 2w, 2w+1
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        r[c] += __shfl_xor(r[c], 32);
        s[c] += __shfl_xor(s[c], 32);
    }
    if (lane < 32) { s_part[wave][0][cg] = r; s_part[wave][1][cg] = s; }
    __syncthreads();

    r = s_part[0][0][cg] + s_part[1][0][cg] + s_part[2][0][cg] + s_part[3][0][cg];
    s = s_part[0][1][cg] + s_part[1][1][cg] + s_part[2][1][cg] + s_part[3][1][cg];
    const f32x4 u = b * (vv - r);
    if (rg == 0) store4(o + vbase + 4 * cg, s + s_kq * u);

    f32x4* Sout = reinterpret_cast<f32x4*>(S + head * (D * D));
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int row = rg + 8 * i;
        __builtin_nontemporal_store(st[i] + s_k[row] * u, &Sout[row * 32 + cg]);
    }
}

hipError_t launch_decode_step(const void* q, const void* k, const void* v,
                              const float* g, const void* beta, float* S, void* o,
                              long long heads, int dtype, hipStream_t stream)
{
    if (heads <= 0) return hipSuccess;
    const dim3 grid((unsigned)heads), block(256);
    if (dtype == 1) {
        hipLaunchKernelGGL(decode_step_kernel<bf16_t>, grid, block, 0, stream,
                           (const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v, g,
                           (const bf16_t*)beta, S, (bf16_t*)o);
    } else {
        hipLaunchKernelGGL(decode_step_kernel<float>, grid, block, 0, stream,
                           (const float*)q, (const float*)k, (const float*)v, g,
                           (const float*)beta, S, (float*)o);
    }
    return hipGetLastError();
}

}  // namespace kda
