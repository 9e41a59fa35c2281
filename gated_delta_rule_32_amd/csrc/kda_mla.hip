// kda_mla.hip -- decode step of a full-attention layer with no position
// encoding, the comparison point for KDA's decode (gfx950).
//
// Page "Kimi K3论文：Kimi Linear", section 5: the hybrid's full-attention
// layers are MLA without position encoding, which at inference runs as MQA
// over the per-token latent; section 7 compares decode time per output token
// at 1M context against a full-MLA model.  The step computes, for every query
// head h of sequence b, with the latent c_t as key and value,
//     o[b,h] = sum_t softmax_t(scale * q[b,h] . c[b,t]) c[b,t].
//
// It reads the whole cache once (D = 512 bf16 = 1 KiB per token): HBM-bound.
// Split-K ("flash decoding"): one 512-thread workgroup per (sequence, 4096
// tokens).  Per 64-token tile the latent rows go global -> LDS with 16-byte
// LDS-destination loads (double-buffered, the next tile in flight during the
// current one; 16-byte units XOR-swizzled by row so both read patterns below
// avoid bank conflicts).  Scores S^T = C Q^T on MFMA with the query heads'
// fragments held in registers (wave w: 16 tokens x 16 heads); an online
// softmax per head (running maximum and sum in LDS, double-buffered); then
// O += P C on MFMA (wave w: 64 latent columns of every head), with the C^T
// fragments formed from the same LDS tile on the matrix cores (identity
// products, 8-byte reads).  A second kernel merges the splits.
#include "kda_chunk_common.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int MD = 512;            // latent width
constexpr int MTILE = 64;          // tokens per tile
constexpr int MSPLIT = 4096;       // tokens per workgroup
constexpr int MTHREADS = 512;

struct MqaLds {
    static constexpr int PP = 2 * 32 + 8;                 // P row pitch (64 tokens + 8)
    static constexpr int OFF_C = 0;                       // 2 x [64][512] bf16, swizzled
    static constexpr int SZ_C = MTILE * MD * 2;
    static constexpr int OFF_P = 2 * SZ_C;                // P [32 heads][72] bf16
    static constexpr int OFF_RED = OFF_P + 32 * PP * 2;   // tile maxima [4][32] fp32
    static constexpr int OFF_RED2 = OFF_RED + 4 * 32 * 4; // tile sums [4][32]
    static constexpr int OFF_M = OFF_RED2 + 4 * 32 * 4;   // running maximum [2][32]
    static constexpr int OFF_L = OFF_M + 2 * 32 * 4;      // running sum [2][32]
    static constexpr int OFF_A = OFF_L + 2 * 32 * 4;      // rescale factor [32]
    static constexpr int TOTAL = OFF_A + 32 * 4;
    static_assert(TOTAL <= 160 * 1024, "LDS budget");
};

__device__ __forceinline__ int swz(int row, int unit) { return unit ^ (row & 15); }

// part: [B][nsplit][H][MD] fp32 partial outputs; ml: [B][nsplit][H][2] (max, sum)
template <int HB>
__global__ void __launch_bounds__(MTHREADS)
mqa_split_kernel(const bf16_t* q, const bf16_t* cache, float* part, float* ml, int T, float scale_log2)
{
    using L = MqaLds;
    constexpr int H = 16 * HB;
    __shared__ __attribute__((aligned(1024))) char smem[L::TOTAL];
    bf16_t* sP = reinterpret_cast<bf16_t*>(smem + L::OFF_P);
    float* red = reinterpret_cast<float*>(smem + L::OFF_RED);
    float* red2 = reinterpret_cast<float*>(smem + L::OFF_RED2);
    float* msh = reinterpret_cast<float*>(smem + L::OFF_M);
    float* lsh = reinterpret_cast<float*>(smem + L::OFF_L);
    float* ash = reinterpret_cast<float*>(smem + L::OFF_A);

    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int ln = lane & 15, lg = lane >> 4;
    const int nsplit = gridDim.x, sp = blockIdx.x, b = blockIdx.y;
    const int tok0 = sp * MSPLIT, tok_end = min(T, tok0 + MSPLIT);
    const int ntiles = (tok_end - tok0 + MTILE - 1) / MTILE;
    const bf16_t* cb = cache + (size_t)b * T * MD;

    // tile n -> buffer n % 2: row r of the tile is wave r % 8's instruction r / 8
    auto load_tile = [&](int n) {
        char* dst = smem + L::OFF_C + (n & 1) * L::SZ_C;
#pragma unroll
        for (int i = 0; i < MTILE / 8; ++i) {
            const int r = wave + 8 * i;
            const int tok = min(tok0 + MTILE * n + r, T - 1);
            __builtin_amdgcn_global_load_lds(cb + (size_t)tok * MD + 8 * swz(r, lane),
                                             (__attribute__((address_space(3))) void*)(dst + r * 1024), 16, 0, 0);
        }
    };

    // S phase role: tokens 16 tb .. of the tile, heads 16 hb ..
    const int tb = wave & 3, hb = wave >> 2;
    const bool s_wave = hb < HB;
    bf16x8 qf[16];
    if (s_wave) {
        const bf16_t* qr = q + ((size_t)b * H + 16 * hb + ln) * MD + 8 * lg;
#pragma unroll
        for (int s = 0; s < 16; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(qr + 32 * s);
    }
    // O phase role: latent columns 64 wave + 16 j + ln, heads 16 hb2 + 4 lg + e
    f32x4 acc[HB][4];
#pragma unroll
    for (int h2 = 0; h2 < HB; ++h2)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[h2][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (t < H) { msh[t] = -INFINITY; lsh[t] = 0.f; }
    load_tile(0);
    __builtin_amdgcn_s_waitcnt(0);
    lds_barrier();

    for (int n = 0; n < ntiles; ++n) {
        const int cur = n & 1;
        if (n + 1 < ntiles) load_tile(n + 1);
        const char* ct = smem + L::OFF_C + cur * L::SZ_C;

        // ---- scores of 16 tokens x 16 heads, tile maxima
        float sc[4];
        if (s_wave) {
            f32x4 a = {0.f, 0.f, 0.f, 0.f};
            const int r = 16 * tb + ln;
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                const bf16x8 cf = *reinterpret_cast<const bf16x8*>(ct + r * 1024 + swz(r, 4 * s + lg) * 16);
                a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cf, qf[s], a, 0, 0, 0);
            }
            float mx = -INFINITY;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bool ok = tok0 + MTILE * n + 16 * tb + 4 * lg + e < tok_end;
                sc[e] = ok ? a[e] * scale_log2 : -INFINITY;
                mx = fmaxf(mx, sc[e]);
            }
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            if (lg == 0) red[tb * 32 + 16 * hb + ln] = mx;
        }
        lds_barrier();

        // ---- probabilities, tile sums, new running maximum
        if (s_wave) {
            const int h = 16 * hb + ln;
            const float m_old = msh[cur * 32 + h];
            const float m_new = fmaxf(fmaxf(m_old, fmaxf(red[h], red[32 + h])), fmaxf(red[64 + h], red[96 + h]));
            f32x4 p;
            float ps = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) { p[e] = __builtin_amdgcn_exp2f(sc[e] - m_new); ps += p[e]; }
            store_vec4<bf16_t>(sP + h * L::PP + 16 * tb + 4 * lg, p);
            ps += __shfl_xor(ps, 16);
            ps += __shfl_xor(ps, 32);
            if (lg == 0) red2[tb * 32 + h] = ps;
            if (tb == 0 && lg == 0) {
                msh[(cur ^ 1) * 32 + h] = m_new;
                ash[h] = __builtin_amdgcn_exp2f(m_old - m_new);   // 0 on the first tile
            }
        }
        lds_barrier();

        // ---- O = Diag(alpha) O + P C
        if (t < H)
            lsh[(cur ^ 1) * 32 + t] = ash[t] * lsh[cur * 32 + t] +
                                      (red2[t] + red2[32 + t]) + (red2[64 + t] + red2[96 + t]);
#pragma unroll
        for (int h2 = 0; h2 < HB; ++h2) {
            const f32x4 al = *reinterpret_cast<const f32x4*>(ash + 16 * h2 + 4 * lg);
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[h2][j] *= al;
        }
        // C^T fragments (tokens along k) from the row-major tile on the matrix
        // cores: A = 16 tile rows x 4 latent columns per lane (one 8-byte read),
        // B = identity, so accumulator lane (ln, lg) holds tokens 4lg .. 4lg+3
        // of latent column ln (bf16 times one summed in fp32: exact).  Two such
        // blocks give the k order {32s + 4lg .., 32s + 16 + 4lg ..}; P is read in
        // the same order.
        bf16x4 ident;
#pragma unroll
        for (int e = 0; e < 4; ++e) ident[e] = (bf16_t)(4 * lg + e == ln ? 1.f : 0.f);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            bf16x8 pa[HB];
#pragma unroll
            for (int h2 = 0; h2 < HB; ++h2) {
                const bf16_t* pr = sP + (16 * h2 + ln) * L::PP + 32 * s + 4 * lg;
                pa[h2] = cat8(*reinterpret_cast<const bf16x4*>(pr), *reinterpret_cast<const bf16x4*>(pr + 16));
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int d = 64 * wave + 16 * j + 4 * lg;            // this lane's 4 latent columns of the A read
                const int unit = d >> 3, el = d & 7;
                bf16x4 half[2];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int r = 32 * s + 16 * hh + ln;
                    const bf16x4 a = *reinterpret_cast<const bf16x4*>(ct + r * 1024 + swz(r, unit) * 16 + el * 2);
                    half[hh] = to_bf16x4(__builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, ident, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0));
                }
                const bf16x8 cfr = cat8(half[0], half[1]);
#pragma unroll
                for (int h2 = 0; h2 < HB; ++h2)
                    acc[h2][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[h2], cfr, acc[h2][j], 0, 0, 0);
            }
        }
        __builtin_amdgcn_s_waitcnt(0);     // the next tile has landed
        lds_barrier();
    }

    // ---- partial results of this split
    const size_t pbase = ((size_t)b * nsplit + sp) * H;
#pragma unroll
    for (int h2 = 0; h2 < HB; ++h2)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                part[(pbase + 16 * h2 + 4 * lg + e) * MD + 64 * wave + 16 * j + ln] = acc[h2][j][e];
    if (t < H) {
        ml[(pbase + t) * 2] = msh[(ntiles & 1) * 32 + t];
        ml[(pbase + t) * 2 + 1] = lsh[(ntiles & 1) * 32 + t];
    }
}

// Merge of the splits: workgroup (sequence, head, 64 latent columns); the
// split weights e^{m_s - M} are formed once in LDS, then 16 lanes per column
// each sum a sixteenth of the splits (many loads in flight: the merge is
// latency-bound), and the 16 partial sums are added in LDS.
constexpr int CMB_COLS = 64, CMB_LANES = 16, CMB_MAXSPLIT = 1024;
__global__ void __launch_bounds__(CMB_COLS * CMB_LANES)
mqa_combine_kernel(const float* part, const float* ml, bf16_t* o, int nsplit, int H)
{
    __shared__ float w_s[CMB_MAXSPLIT];
    __shared__ float red[CMB_COLS * CMB_LANES];
    __shared__ float Lsh;
    const int t = threadIdx.x, bh = blockIdx.x, cb = blockIdx.y;
    const int b = bh / H, h = bh % H;
    const size_t base = (size_t)b * nsplit * H + h;      // split s at base + s * H
    float m = -INFINITY;
    for (int s = t; s < nsplit; s += blockDim.x) m = fmaxf(m, ml[(base + (size_t)s * H) * 2]);
    red[t] = m;
    __syncthreads();
    for (int k = blockDim.x / 2; k > 0; k >>= 1) {
        if (t < k) red[t] = fmaxf(red[t], red[t + k]);
        __syncthreads();
    }
    const float M = red[0];
    __syncthreads();
    float l = 0.f;
    for (int s = t; s < nsplit; s += blockDim.x) {
        const size_t i = base + (size_t)s * H;
        const float w = __builtin_amdgcn_exp2f(ml[i * 2] - M);
        w_s[s] = w;
        l += w * ml[i * 2 + 1];
    }
    red[t] = l;
    __syncthreads();
    for (int k = blockDim.x / 2; k > 0; k >>= 1) {
        if (t < k) red[t] += red[t + k];
        __syncthreads();
    }
    if (t == 0) Lsh = red[0];
    __syncthreads();
    const int col = t % CMB_COLS, lane4 = t / CMB_COLS;
    const int d = CMB_COLS * cb + col;
    float acc = 0.f;
    for (int s = lane4; s < nsplit; s += CMB_LANES) acc += w_s[s] * part[(base + (size_t)s * H) * MD + d];
    red[t] = acc;
    __syncthreads();
    if (lane4 == 0) {
        float sum = 0.f;
#pragma unroll
        for (int i = 0; i < CMB_LANES; ++i) sum += red[col + i * CMB_COLS];
        o[(size_t)bh * MD + d] = (bf16_t)(sum / Lsh);
    }
}

}  // namespace

size_t mqa_ws_bytes(long long B, long long T, long long H)
{
    const size_t nsplit = (size_t)((T + MSPLIT - 1) / MSPLIT);
    const size_t part = (size_t)B * nsplit * (size_t)H * MD * 4;
    const size_t ml = (size_t)B * nsplit * (size_t)H * 2 * 4;
    return (part + 255) / 256 * 256 + (ml + 255) / 256 * 256;
}

hipError_t launch_mqa_decode(const void* q, const void* cache, void* o, int B, int T, int H, float scale,
                             void* ws, hipStream_t stream)
{
    const int nsplit = (T + MSPLIT - 1) / MSPLIT;   // <= CMB_MAXSPLIT (T < 2^22, checked by the caller)
    float* part = reinterpret_cast<float*>(ws);
    const size_t part_bytes = (size_t)B * nsplit * H * MD * 4;
    float* ml = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + (part_bytes + 255) / 256 * 256);
    const float sl2 = scale * LOG2E;
    const dim3 grid((unsigned)nsplit, (unsigned)B);
    if (H == 32)
        hipLaunchKernelGGL(mqa_split_kernel<2>, grid, dim3(MTHREADS), 0, stream,
                           (const bf16_t*)q, (const bf16_t*)cache, part, ml, T, sl2);
    else
        hipLaunchKernelGGL(mqa_split_kernel<1>, grid, dim3(MTHREADS), 0, stream,
                           (const bf16_t*)q, (const bf16_t*)cache, part, ml, T, sl2);
    hipLaunchKernelGGL(mqa_combine_kernel, dim3((unsigned)(B * H), MD / CMB_COLS), dim3(CMB_COLS * CMB_LANES), 0,
                       stream, part, ml, (bf16_t*)o, nsplit, H);
    return hipGetLastError();
}

}  // namespace kda
