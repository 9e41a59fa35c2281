// kda_dplr.hip -- chunked forward of the general diagonal-plus-low-rank (DPLR)
// recurrence for gfx950, the comparison point for KDA's restricted form.
//
// Page "Kimi K3论文：Kimi Linear", section 4: the general gated delta rule
// S_t = (D_t - a_t b_t^T) S_{t-1} + k_t v_t^T (D_t = Diag(alpha_t)), of which
// KDA is the case a = beta k, b = alpha * k; the page credits KDA's tie of a
// and b to k with halving the intra-chunk matrices (two instead of four) and
// about doubling the operator's speed.  Output o_t = S_t^T q_t as for KDA.
//
// Chunk form (C = 64, entry state S, G = in-chunk cumulative sum of
// g = log alpha, G_{r-1} the exclusive sum, u_i = S_{i-1}^T b_i):
//
//   Qh = e^{G} q,  Bh = e^{G_{r-1}} b,  Kb = e^{-G} k,  Ab = e^{-G} a     [64 x 128]
//   A_qk = tril(Qh Kb^T), A_qa = tril(Qh Ab^T)                 (i <= r)
//   A_bk = stril(Bh Kb^T), A_ba = stril(Bh Ab^T)                (i < r)
//   T = (I + A_ba)^{-1}                                          (UT transform)
//   -U = U0 - W S  with  W = T Bh,  U0 = -T A_bk V
//   O  = Qh S + A_qk V + A_qa (-U)
//   S <- Diag(e^{G_64}) (S + Ab^T (-U)) + H0,  H0 = (e^{G_64 - G} k)^T V
//
// Two kernels.  dplr_prep_kernel (this file) does everything that does not
// depend on S, one workgroup per (head, 4 chunks), the next chunk's inputs
// loading while the current one's products run: the four 64 x 64 products,
// the UT transform, W, U0, O0 = A_qk V and H0.  It writes Qh, W, Ab^T, A_qa
// and e^{G_64} in the operand-block layout of the KDA state scan (Kh -> W,
// Kb -> Ab, Aqk -> A_qa), and U0, O0, H0 beside it; chunk_scan_kernel in its
// DPLR mode then walks the chunks of each head: Vn = U0 - W S, output
// Qh S + A_qa Vn + O0, state Diag(gamma)(S + Ab^T Vn) + H0.
//
// All products are v_mfma_f32_16x16x32_bf16 on bf16 operands in LDS with fp32
// accumulation; the decay factorisation e^{G_r - G_i} = e^{G_r} e^{-G_i} is
// the one the KDA kernels use (exact up to rounding while |G| stays below
// about 80 within a chunk).
#include "kda_chunk_common.h"
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

struct DplrLds {
    static constexpr int P128 = DK + 8, P64 = C + 8, PA = C + 4;
    static constexpr int R64 = C * P128 * 2;               // [64][136] bf16
    static constexpr int T128 = DK * P64 * 2;              // [128][72] bf16
    static constexpr int CC = C * P64 * 2;                 // [64][72] bf16
    // region X: token-major operands of the 64 x 64 products, later the
    // channel-major operands of the 64-deep products
    static constexpr int OFF_Q = 0, OFF_KB = R64, OFF_AB = 2 * R64, OFF_BH = 3 * R64;
    static constexpr int OFF_BHT = 0, OFF_ABT = T128;      // Bh^T, Ab^T (swizzled as in the block)
    static constexpr int X_END = 4 * R64;
    static constexpr int OFF_RA = X_END;                   // A_ba fp32 [64][68], then T's diagonal blocks
    static constexpr int OFF_QA = OFF_RA + C * PA * 4;     // A_qa
    static constexpr int OFF_XT = OFF_RA;                  // (A_bk V)^T [128][72], over RA and A_qa
    static constexpr int OFF_QK = OFF_QA + CC;             // A_qk
    static constexpr int OFF_BK = OFF_QK + CC;             // A_bk
    static constexpr int OFF_RT = OFF_BK + CC;             // T in bf16
    static constexpr int OFF_GAM = OFF_RT + CC;            // e^{G_64} [128] fp32
    static constexpr int OFF_ONE = OFF_GAM + DK * 4;       // 1.0 [64] fp32 (column scales of T)
    static constexpr int OFF_KTT = OFF_ONE + C * 4;        // (e^{G_64 - G} k)^T [128][72]
    static constexpr int OFF_VT = OFF_KTT + T128;          // V^T [128][72]
    static constexpr int TOTAL = OFF_VT + T128;
    static_assert(2 * T128 <= X_END, "Bh^T and Ab^T fit in region X");
    static_assert(T128 == DK * WS_P64 * 2, "Ab^T has the block's layout");
    static_assert(T128 <= C * PA * 4 + CC, "(A_bk V)^T fits over A_ba and A_qa");
    static_assert(TOTAL <= 160 * 1024, "LDS budget");
};

__device__ __forceinline__ bf16x8 ld8(const bf16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// 16 x 16 tile of X Y^T with X rows x0.., Y rows y0.. (both with the
// contraction index contiguous, K = 32 * KS); acc[e] = D[4(lane/16) + e][lane % 16].
template <int KS>
__device__ __forceinline__ f32x4 tile(const bf16_t* X, int ldx, int x0, const bf16_t* Y, int ldy, int y0,
                                      int ln, int lg) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s)
        acc = mma(ld8(X + (x0 + ln) * ldx + 32 * s + 8 * lg), ld8(Y + (y0 + ln) * ldy + 32 * s + 8 * lg), acc);
    return acc;
}
// x of the lane s places lower in the same 16-lane row (0 for the first s lanes)
template <int S>
__device__ __forceinline__ float row_shr(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x110 + S, 0xF, 0xF, true));
}
__device__ __forceinline__ float readlane(float x, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}
// the six 16 x 16 blocks above the diagonal of a 64 x 64 matrix, (row, column)
__device__ __forceinline__ int upper_m(int u) { return u < 3 ? 0 : u < 5 ? 1 : 2; }
__device__ __forceinline__ int upper_n(int u) { return u < 3 ? u + 1 : u < 5 ? u - 1 : 3; }
__device__ __forceinline__ void st4(bf16_t* p, const f32x4& x, float s = 1.f) {
    bf16x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = (bf16_t)(s * x[e]);
    *reinterpret_cast<bf16x4*>(p) = r;
}

constexpr int DPLR_PREP_CHUNKS = 4;      // chunks per prep workgroup (inputs of the next prefetched)

// Raw inputs of one chunk for one thread: token row = lane, 16 channels of the
// wave's block (32 bytes of each of q, k, a, b, v and 64 bytes of g).
struct DplrIn {
    bf16x8 q[2], k[2], a[2], b[2], v[2];
    f32x4 g[4];
};

__global__ void __launch_bounds__(512)
dplr_prep_kernel(const bf16_t* q, const bf16_t* k, const bf16_t* v, const bf16_t* a, const bf16_t* b,
                 const float* g, int T, int H, char* blocks, bf16_t* h0, bf16_t* u0, bf16_t* o0, bf16_t* sink)
{
    using L = DplrLds;
    __shared__ __attribute__((aligned(1024))) char smem[L::TOTAL];
    bf16_t* sQ = reinterpret_cast<bf16_t*>(smem + L::OFF_Q);
    bf16_t* sKb = reinterpret_cast<bf16_t*>(smem + L::OFF_KB);
    bf16_t* sAb = reinterpret_cast<bf16_t*>(smem + L::OFF_AB);
    bf16_t* sBh = reinterpret_cast<bf16_t*>(smem + L::OFF_BH);
    bf16_t* sBhT = reinterpret_cast<bf16_t*>(smem + L::OFF_BHT);
    bf16_t* sAbT = reinterpret_cast<bf16_t*>(smem + L::OFF_ABT);
    bf16_t* sKtT = reinterpret_cast<bf16_t*>(smem + L::OFF_KTT);
    bf16_t* sVT = reinterpret_cast<bf16_t*>(smem + L::OFF_VT);
    float* RA = reinterpret_cast<float*>(smem + L::OFF_RA);
    bf16_t* sQA = reinterpret_cast<bf16_t*>(smem + L::OFF_QA);
    bf16_t* sXT = reinterpret_cast<bf16_t*>(smem + L::OFF_XT);
    bf16_t* sQK = reinterpret_cast<bf16_t*>(smem + L::OFF_QK);
    bf16_t* sBK = reinterpret_cast<bf16_t*>(smem + L::OFF_BK);
    bf16_t* RT = reinterpret_cast<bf16_t*>(smem + L::OFF_RT);
    float* s_gam = reinterpret_cast<float*>(smem + L::OFF_GAM);
    float* s_one = reinterpret_cast<float*>(smem + L::OFF_ONE);

    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int nchunks = (T + C - 1) / C;
    const int nblk = (nchunks + DPLR_PREP_CHUNKS - 1) / DPLR_PREP_CHUNKS;
    const int head = blockIdx.x / nblk;
    const int n_first = (blockIdx.x % nblk) * DPLR_PREP_CHUNKS;
    const int n_end = min(n_first + DPLR_PREP_CHUNKS, nchunks);
    const int bb = head / H, h = head % H;
    const size_t tokstride = (size_t)H * DK;
    const size_t hbase = ((size_t)bb * T * H + h) * DK;
    const int c0 = 16 * wave;                 // elementwise work: channels c0 .. c0 + 15, token row = lane
    if (threadIdx.x < C) s_one[threadIdx.x] = 1.f;

    DplrIn in;
    auto load = [&](int n, int r) {
        const int tok = n * C + r;
        const bool ok = tok < T;
        const size_t at = hbase + (size_t)min(tok, T - 1) * tokstride + c0;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            in.q[i] = ok ? ld8(q + at + 8 * i) : bf16x8{};
            in.k[i] = ok ? ld8(k + at + 8 * i) : bf16x8{};
            in.a[i] = ok ? ld8(a + at + 8 * i) : bf16x8{};
            in.b[i] = ok ? ld8(b + at + 8 * i) : bf16x8{};
            in.v[i] = ok ? ld8(v + at + 8 * i) : bf16x8{};
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
            in.g[i] = ok ? *reinterpret_cast<const f32x4*>(g + at + 4 * i) : f32x4{0.f, 0.f, 0.f, 0.f};
    };
    if (n_first < n_end) load(n_first, (int)threadIdx.x & 63);

    for (int n = n_first; n < n_end; ++n) {
        // Lane indices are re-derived every chunk from a value the compiler
        // cannot see through, so that the many per-lane addresses below are
        // recomputed here instead of being hoisted out of the loop and spilled.
        int t = threadIdx.x;
        asm volatile("" : "+v"(t));
        const int lane = t & 63, ln = lane & 15, lg = lane >> 4, r = lane;
        const size_t cidx = (size_t)head * nchunks + n;
        char* blk = blocks + cidx * WS_CHUNK;

        // ===== G: inclusive prefix over the 64 rows (= lanes) of the wave =====
        // within each 16-lane row by DPP row shifts (zero shifted in), then the
        // totals of the rows before, read as wave-uniform values
        float G[16], egc[16];
#pragma unroll
        for (int x = 0; x < 16; ++x) {
            float v = in.g[x >> 2][x & 3] * LOG2E;                 // log2 units
            v += row_shr<1>(v);
            v += row_shr<2>(v);
            v += row_shr<4>(v);
            v += row_shr<8>(v);
            const float t0 = readlane(v, 15), t1 = readlane(v, 31), t2 = readlane(v, 47), t3 = readlane(v, 63);
            G[x] = v + (lg >= 1 ? t0 : 0.f) + (lg >= 2 ? t1 : 0.f) + (lg >= 3 ? t2 : 0.f);
            egc[x] = __builtin_amdgcn_exp2f(t0 + t1 + t2 + t3);       // e^{G_64}
        }
#pragma unroll
        for (int x = 0; x < 16; ++x)
            if (lane == x) s_gam[c0 + x] = egc[x];

        // ===== decay-scaled rows: LDS operands, Qh and Ab^T exported =====
        bf16x8 bhv[2], ktv[2], abv[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            bf16x8 oq, okb;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int x = 8 * i + j;
                const float eg = __builtin_amdgcn_exp2f(G[x]), eng = __builtin_amdgcn_exp2f(-G[x]);
                const float egp = __builtin_amdgcn_exp2f(G[x] - in.g[x >> 2][x & 3] * LOG2E);
                const float kbar = (float)in.k[i][j] * eng;
                oq[j] = (bf16_t)((float)in.q[i][j] * eg);
                okb[j] = (bf16_t)kbar;
                abv[i][j] = (bf16_t)((float)in.a[i][j] * eng);
                bhv[i][j] = (bf16_t)((float)in.b[i][j] * egp);
                ktv[i][j] = (bf16_t)(kbar * egc[x]);
            }
            *reinterpret_cast<bf16x8*>(sQ + r * L::P128 + c0 + 8 * i) = oq;
            *reinterpret_cast<bf16x8*>(sKb + r * L::P128 + c0 + 8 * i) = okb;
            *reinterpret_cast<bf16x8*>(sAb + r * L::P128 + c0 + 8 * i) = abv[i];
            *reinterpret_cast<bf16x8*>(sBh + r * L::P128 + c0 + 8 * i) = bhv[i];
            *reinterpret_cast<bf16x8*>(blk + WS_QT + (r * WS_P128 + c0 + 8 * i) * 2) = oq;
        }
        // the channel-major operands K~^T and V^T: for each channel the 64
        // lanes write one 128-byte row
#pragma unroll
        for (int x = 0; x < 16; ++x) {
            sKtT[(c0 + x) * L::P64 + r] = ktv[x >> 3][x & 7];
            sVT[(c0 + x) * L::P64 + r] = in.v[x >> 3][x & 7];
        }
        lds_barrier();

        // ===== the four 64 x 64 products (lower block triangle) =====
        for (int u = wave; u < 40; u += 8) {
            const int mat = u / 10, tl = u % 10;
            const int mb = tl >= 6 ? 3 : tl >= 3 ? 2 : tl >= 1 ? 1 : 0, nb = tl - mb * (mb + 1) / 2;
            const f32x4 d = tile<4>(mat < 2 ? sQ : sBh, L::P128, 16 * mb, (mat & 1) ? sAb : sKb, L::P128,
                                    16 * nb, ln, lg);
            const int r0 = 16 * mb + 4 * lg, i = 16 * nb + ln;
            const bool incl = mat < 2;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float x = (incl ? i <= r0 + e : i < r0 + e) ? d[e] : 0.f;
                if (mat == 3) RA[(r0 + e) * L::PA + i] = x;
                else (mat == 0 ? sQK : mat == 1 ? sQA : sBK)[(r0 + e) * L::P64 + i] = (bf16_t)x;
            }
        }
        // zero blocks above the diagonal of A_qk, A_qa, A_bk (16-byte units)
        for (int u = t; u < 3 * 6 * 32; u += 512) {
            const int mat = u / 192, tl = (u / 32) % 6, w = u % 32;
            bf16_t* m = mat == 0 ? sQK : mat == 1 ? sQA : sBK;
            *reinterpret_cast<bf16x8*>(m + (16 * upper_m(tl) + w / 2) * L::P64 + 16 * upper_n(tl) + 8 * (w & 1)) =
                bf16x8{};
        }
        lds_barrier();

        // ===== diagonal blocks of T (wave 0) | A_qa and e^{G_64} exports (waves 1-7) =====
        if (wave == 0) {
            // column m of (I + A_bb)^{-1}, right-looking substitution; the wave's
            // reads all precede its writes
            const int blkd = lane >> 4, m = lane & 15;
            float* A = RA + 16 * blkd * L::PA + 16 * blkd;
            float x[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) x[i] = (i == m) ? 1.f : 0.f;
#pragma unroll
            for (int j = 0; j < 15; ++j) {
#pragma unroll
                for (int i = j + 1; i < 16; ++i) x[i] -= A[i * L::PA + j] * x[j];
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) A[i * L::PA + m] = x[i];
        } else {
            typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;
            const int u0i = t - 64, NU = 512 - 64;
            for (int u = u0i; u < L::CC / 16; u += NU)
                reinterpret_cast<i32x4*>(blk + WS_QK)[u] = reinterpret_cast<const i32x4*>(sQA)[u];
            if (u0i < DK / 4)
                reinterpret_cast<f32x4*>(blk + WS_GAM)[u0i] = reinterpret_cast<const f32x4*>(s_gam)[u0i];
        }
        lds_barrier();

        // ===== Bh^T and Ab^T (region X is free) | off-diagonal blocks of T =====
        // lanes = consecutive rows: each write is one 128-byte row segment;
        // Ab^T in the scan's swizzled layout, copied out below
#pragma unroll
        for (int x = 0; x < 16; ++x) {
            sBhT[(c0 + x) * L::P64 + r] = bhv[x >> 3][x & 7];
            sAbT[kbt_swz(c0 + x, r)] = abv[x >> 3][x & 7];
        }
        if (wave == 0) ut_offdiag_column<0, L::PA, L::P64>(RA, RT, s_one, lane);
        else if (wave == 1) ut_offdiag_column<1, L::PA, L::P64>(RA, RT, s_one, lane);
        else if (wave == 2) ut_offdiag_column<2, L::PA, L::P64>(RA, RT, s_one, lane);
        else if (wave == 3) {
#pragma unroll
            for (int blkd = 0; blkd < 4; ++blkd)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int rr2 = 16 * blkd + 4 * lg + e;
                    RT[rr2 * L::P64 + 16 * blkd + ln] = (bf16_t)RA[rr2 * L::PA + 16 * blkd + ln];
                }
        } else {
            for (int u = wave - 4; u < 6; u += 4)           // zero blocks above the diagonal
                st4(RT + (16 * upper_m(u) + ln) * L::P64 + 16 * upper_n(u) + 4 * lg, f32x4{0.f, 0.f, 0.f, 0.f});
        }
        lds_barrier();

        {   // Ab^T -> the Kb^T slot of the block, 16 bytes per lane
            typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;
            for (int u = t; u < L::T128 / 16; u += 512)
                reinterpret_cast<i32x4*>(blk + WS_KBT)[u] = reinterpret_cast<const i32x4*>(sAbT)[u];
        }
        // the next chunk's inputs load during the products below
        if (n + 1 < n_end) load(n + 1, r);

        // ===== 64-deep products; wave w owns block w of the value (or key) columns =====
        const int jb = wave;
        bf16x8 fv[2], fb[2];                        // V^T rows of block jb, Bh^T rows
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            fv[s] = ld8(sVT + (16 * jb + ln) * L::P64 + 32 * s + 8 * lg);
            fb[s] = ld8(sBhT + (16 * jb + ln) * L::P64 + 32 * s + 8 * lg);
        }
        auto prod = [&](const bf16x8 (&x)[2], const bf16_t* Y, int y0) {   // X rows fixed, Y rows y0..
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 2; ++s) acc = mma(x[s], ld8(Y + (y0 + ln) * L::P64 + 32 * s + 8 * lg), acc);
            return acc;
        };
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
            const int tr = n * C + 16 * rb + ln;
            // W = T Bh -> the Kh slot of the block: lane holds W[16rb + ln][16jb + 4lg ..]
            f32x4 d = prod(fb, RT, 16 * rb);
            st4(reinterpret_cast<bf16_t*>(blk + WS_KH) + (16 * rb + ln) * WS_P128 + 16 * jb + 4 * lg, d);
            // X = A_bk V -> X^T in LDS: lane holds X[16rb + 4lg ..][16jb + ln]
            d = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 2; ++s)
                d = mma(ld8(sBK + (16 * rb + ln) * L::P64 + 32 * s + 8 * lg), fv[s], d);
            st4(sXT + (16 * jb + ln) * L::P64 + 16 * rb + 4 * lg, d);
            // O0 = A_qk V -> token-major rows.  Rows past T go to a sink row so
            // that every chunk issues the same stores: the wait for the next
            // chunk's inputs then need not cover them.
            d = prod(fv, sQK, 16 * rb);
            st4((tr < T ? o0 + hbase + (size_t)tr * tokstride : sink) + 16 * jb + 4 * lg, d);
        }
        // H0 = (e^{G_64 - G} k)^T V: rows = key channels, columns = value columns
        bf16_t* hp = h0 + cidx * DK * DK;
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) st4(hp + (16 * cb + ln) * DK + 16 * jb + 4 * lg, prod(fv, sKtT, 16 * cb));
        lds_barrier();
        // U0 = -T X -> token-major rows
        bf16x8 fx[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) fx[s] = ld8(sXT + (16 * jb + ln) * L::P64 + 32 * s + 8 * lg);
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
            const f32x4 d = prod(fx, RT, 16 * rb);
            const int tr = n * C + 16 * rb + ln;
            st4((tr < T ? u0 + hbase + (size_t)tr * tokstride : sink) + 16 * jb + 4 * lg, d, -1.f);
        }
        lds_barrier();                             // LDS reused by the next chunk
    }
}

}  // namespace

size_t dplr_ws_layout(long long B, long long T, long long H, size_t* off)
{
    const size_t units = (size_t)B * (size_t)H * (size_t)((T + C - 1) / C);
    const size_t tok = (size_t)B * (size_t)T * (size_t)H;
    size_t o[KDA_DPLR_WS_REGIONS + 1];
    o[KDA_DPLR_WS_BLK] = 0;
    o[KDA_DPLR_WS_H0] = units * WS_CHUNK;
    o[KDA_DPLR_WS_U0] = o[KDA_DPLR_WS_H0] + units * DK * DK * 2;
    o[KDA_DPLR_WS_O0] = o[KDA_DPLR_WS_U0] + (tok * DK * 2 + 255) / 256 * 256;
    o[KDA_DPLR_WS_SINK] = o[KDA_DPLR_WS_O0] + (tok * DK * 2 + 255) / 256 * 256;
    o[KDA_DPLR_WS_REGIONS] = o[KDA_DPLR_WS_SINK] + 256;
    if (off)
        for (int i = 0; i < KDA_DPLR_WS_REGIONS; ++i) off[i] = o[i];
    return o[KDA_DPLR_WS_REGIONS];
}

hipError_t launch_dplr_chunk_fwd(const void* q, const void* k, const void* v, const void* a, const void* b,
                                 const float* g, const float* S0, void* o, float* S_T, int B, int T, int H,
                                 char* ws, hipStream_t stream)
{
    size_t off[KDA_DPLR_WS_REGIONS];
    dplr_ws_layout(B, T, H, off);
    char* blocks = ws + off[KDA_DPLR_WS_BLK];
    bf16_t* h0 = reinterpret_cast<bf16_t*>(ws + off[KDA_DPLR_WS_H0]);
    bf16_t* u0 = reinterpret_cast<bf16_t*>(ws + off[KDA_DPLR_WS_U0]);
    bf16_t* o0 = reinterpret_cast<bf16_t*>(ws + off[KDA_DPLR_WS_O0]);
    bf16_t* sink = reinterpret_cast<bf16_t*>(ws + off[KDA_DPLR_WS_SINK]);
    const long long nblk = ((T + C - 1) / C + DPLR_PREP_CHUNKS - 1) / DPLR_PREP_CHUNKS;
    hipLaunchKernelGGL(dplr_prep_kernel, dim3((unsigned)((long long)B * H * nblk)), dim3(512), 0, stream,
                       (const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v, (const bf16_t*)a,
                       (const bf16_t*)b, g, T, H, blocks, h0, u0, o0, sink);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    return launch_dplr_scan(blocks, u0, h0, o0, S0, o, S_T, B, T, H, stream);
}

}  // namespace kda
