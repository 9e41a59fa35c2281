// kda_prefill.hip -- chunkwise KDA prefill for gfx950 (one fused kernel).
//
// Method: page "Kimi Linear：高效注意力机制在长序列处理中的创新应用", sections
// 2.1-2.3 (Proposition S_r = P_r S_0 + H_r, WY representation, chunks of 64,
// forward substitution) and page "Kimi K3论文：Kimi Linear", section 4 (intra-
// chunk matrix products, UT transform, chunk-to-chunk state recurrence).
// For a chunk of C = 64 tokens with entry state S (d_k x d_v, fp32), and
// G = in-chunk cumulative sum of g = log(alpha):
//
//   Qt = e^{G} * Q,  Kh = e^{G} * K,  Kb = e^{-G} * K                  [64 x 128]
//   Aqk = Qt Kb^T   (kept for i <= r)                                  [64 x 64]
//   Akk = Diag(beta) Kh Kb^T   (kept for i < r)
//   Tm  = (I + Akk)^{-1}                         (UT transform)
//   Vn  = Tm Diag(beta) (V - Kh S)               (= U - W S with the WY factors
//                                                  W = Tm Diag(beta) Kh, U = Tm Diag(beta) V)
//   O   = Qt S + Aqk Vn
//   S  <- Diag(e^{G_64}) (S + Kb^T Vn)           (= Diag(e^{G_64}) S + (e^{G_64 - G} * K)^T Vn)
//
// The decay e^{G_r - G_i} is split into a row factor e^{G_r} and a column
// factor e^{-G_i} (reference point: the chunk start); this is exact up to
// rounding while every |G| in a chunk stays below ~80.  The WY factor W is
// never formed: Tm is applied to the residual V - Kh S instead, which is the
// same product reassociated and saves one 64x64x128 product and its buffer.
//
// Tm is built blockwise: the four 16x16 diagonal blocks by forward
// substitution in registers (one column per lane), then the off-diagonal
// blocks X_RI = -X_RR sum_J Akk_RJ X_JI column by column.
//
// Work decomposition.  The state recurrence is sequential over chunks, so one
// workgroup (8 waves) owns one head and walks its chunks in order with the
// fp32 state resident in MFMA accumulators.  Everything after Tm is
// independent per value column, so the 128 value columns are split into
// slices of DV columns, each its own workgroup (the key-side work -- G, Aqk,
// Akk, Tm -- is recomputed per slice).  Slices of one head are placed on one
// XCD so that their reads of q, k, g share an L2.  All operands live in LDS in
// the layout their MFMA fetch wants (contraction index contiguous, rows padded
// by 16 B against bank conflicts); nothing but the inputs, o and the final
// state touches HBM.
//
// Two instantiations: bf16 inputs use v_mfma_f32_16x16x32_bf16 (fp32
// accumulate) with bf16 LDS operands; fp32 inputs use v_mfma_f32_16x16x4_f32
// with fp32 LDS operands, so fp32 workloads keep fp32 products.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int C = 64;     // chunk length
constexpr int DK = 128;   // key / value head dimension
constexpr int NW = 8;     // waves per workgroup
constexpr int NT = 64 * NW;
constexpr int RPT = C / NW;   // rows per thread in the elementwise phase (8)

// Barrier that orders LDS traffic only: global loads stay in flight.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ---- MFMA wrappers -------------------------------------------------------
// A 16 x 16 output tile D = A B.  `frag_kc` fetches an operand from a row-major
// LDS matrix whose rows are the tile's M (or N) index and whose columns are the
// contraction index (pitch `ld`); `frag_mc` (fp32 only) fetches it from the
// transposed layout.  Both operands of one product use the same per-lane
// contraction slots, so the product is a plain sum over k.
// Output: acc[e] holds D[4 * (lane / 16) + e][lane % 16].
template <typename E> struct Mma;

template <> struct Mma<bf16_t> {
    static constexpr int KS = 32;
    typedef bf16x8 frag_t;
    __device__ static frag_t frag_kc(const bf16_t* p, int ld, int row0, int k0, int lane) {
        return *reinterpret_cast<const bf16x8*>(p + (row0 + (lane & 15)) * ld + k0 + 8 * (lane >> 4));
    }
    __device__ static f32x4 mma(frag_t a, frag_t b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};

template <> struct Mma<float> {
    static constexpr int KS = 4;
    typedef float frag_t;
    __device__ static frag_t frag_kc(const float* p, int ld, int row0, int k0, int lane) {
        return p[(row0 + (lane & 15)) * ld + k0 + (lane >> 4)];
    }
    __device__ static frag_t frag_mc(const float* p, int ld, int row0, int k0, int lane) {
        return p[(k0 + (lane >> 4)) * ld + row0 + (lane & 15)];
    }
    __device__ static f32x4 mma(frag_t a, frag_t b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
};

// acc[t] += A[arow0.., K] * B[brow[t].., K]^T over k in [0, K); A fragments are
// loaded once and reused for the NB output tiles.
template <typename E, int K, int NB>
__device__ __forceinline__ void mma_rows(f32x4 (&acc)[NB], const E* A, int lda, int arow0,
                                         const E* B, int ldb, const int (&brow)[NB], int lane) {
    constexpr int UNR = (K / Mma<E>::KS) < 8 ? (K / Mma<E>::KS) : 8;
#pragma unroll UNR
    for (int k = 0; k < K; k += Mma<E>::KS) {
        const auto a = Mma<E>::frag_kc(A, lda, arow0, k, lane);
#pragma unroll
        for (int t = 0; t < NB; ++t) acc[t] = Mma<E>::mma(a, Mma<E>::frag_kc(B, ldb, brow[t], k, lane), acc[t]);
    }
}

// ---- element pairs and runs ------------------------------------------------
template <typename E> struct Pair;
template <> struct Pair<bf16_t> { typedef bf16x2 type; };
template <> struct Pair<float> { typedef float2 type; };

__device__ __forceinline__ float2 unpack(bf16x2 x) { return make_float2((float)x[0], (float)x[1]); }
__device__ __forceinline__ float2 unpack(float2 x) { return x; }
template <typename E> __device__ __forceinline__ typename Pair<E>::type pack(float a, float b);
template <> __device__ __forceinline__ bf16x2 pack<bf16_t>(float a, float b) {
    bf16x2 r; r[0] = (bf16_t)a; r[1] = (bf16_t)b; return r;
}
template <> __device__ __forceinline__ float2 pack<float>(float a, float b) { return make_float2(a, b); }

template <typename E> __device__ __forceinline__ void store_vec4(E* p, f32x4 x);
template <> __device__ __forceinline__ void store_vec4<bf16_t>(bf16_t* p, f32x4 x) {
    bf16x4 v; v[0] = (bf16_t)x[0]; v[1] = (bf16_t)x[1]; v[2] = (bf16_t)x[2]; v[3] = (bf16_t)x[3];
    *reinterpret_cast<bf16x4*>(p) = v;
}
template <> __device__ __forceinline__ void store_vec4<float>(float* p, f32x4 x) {
    *reinterpret_cast<f32x4*>(p) = x;
}
template <typename E> __device__ __forceinline__ f32x4 load_vec4(const E* p);
template <> __device__ __forceinline__ f32x4 load_vec4<bf16_t>(const bf16_t* p) {
    const bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
    return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
template <> __device__ __forceinline__ f32x4 load_vec4<float>(const float* p) {
    return *reinterpret_cast<const f32x4*>(p);
}

// Store N contiguous values (N = 1, 2, 4, 8, ...).
template <typename E, int N>
__device__ __forceinline__ void store_run(E* p, const float* x) {
    if constexpr (N == 1) {
        *p = (E)x[0];
    } else if constexpr (N == 2) {
        *reinterpret_cast<typename Pair<E>::type*>(p) = pack<E>(x[0], x[1]);
    } else {
#pragma unroll
        for (int i = 0; i < N; i += 4) store_vec4<E>(p + i, f32x4{x[i], x[i + 1], x[i + 2], x[i + 3]});
    }
}

// ---- UT transform, off-diagonal blocks of one block column -------------------
// Column I of X = (I + A)^{-1} (A strictly lower, 4x4 blocks of 16, diagonal
// blocks X_RR already inverted in place in RA):  X_RI = -X_RR sum_{J=I}^{R-1}
// A_RJ X_JI.  The products are 16x16x16 bf16 MFMAs chained through registers:
// the D layout of one product (lane holds rows 4*(lane/16)+e of column
// lane%16) is exactly the B-operand layout of the next.  Each X_RI is written
// to RT scaled by beta of its column.
__device__ __forceinline__ bf16x4 to_bf16x4(const f32x4& x) {
    bf16x4 r; r[0] = (bf16_t)x[0]; r[1] = (bf16_t)x[1]; r[2] = (bf16_t)x[2]; r[3] = (bf16_t)x[3];
    return r;
}

template <int I, int PA, int PT>
__device__ __forceinline__ void ut_offdiag_column(const float* RA, bf16_t* RT, const float* s_beta, int lane) {
    const int ln = lane & 15, lg = lane >> 4;
    auto a_op = [&](int R, int J) {   // A operand: block (R, J) of RA, row-major
        return to_bf16x4(*reinterpret_cast<const f32x4*>(RA + (16 * R + ln) * PA + 16 * J + 4 * lg));
    };
    f32x4 X[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) X[I][e] = RA[(16 * I + 4 * lg + e) * PA + 16 * I + ln];
    const float bcol = s_beta[16 * I + ln];
#pragma unroll
    for (int R = I + 1; R < 4; ++R) {
        f32x4 Y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int J = I; J < R; ++J)
            Y = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a_op(R, J), to_bf16x4(X[J]), Y, 0, 0, 0);
        X[R] = -__builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a_op(R, R), to_bf16x4(Y),
                                                          f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) RT[(16 * R + 4 * lg + e) * PT + 16 * I + ln] = (bf16_t)(bcol * X[R][e]);
    }
}

// ---- LDS layout -------------------------------------------------------------
template <typename E, int DV>
struct Layout {
    static constexpr int ES = sizeof(E);
    static constexpr bool kF32 = (ES == 4);
    static constexpr int PAD = 16 / ES;
    static constexpr int P128 = DK + PAD;   // token-major [64][128] rows
    static constexpr int P64 = C + PAD;     // channel-major [*][64] rows
    static constexpr int PA = C + 4;        // fp32 [64][64] rows (== P64 when E is fp32)
    static constexpr int SZ_TOK = C * P128 * ES;
    static constexpr int OFF_QT = 0;                                  // Qt = e^G q
    static constexpr int OFF_KH = OFF_QT + SZ_TOK;                    // Kh = e^G k
    static constexpr int OFF_KB = OFF_KH + SZ_TOK;                    // Kb = e^-G k
    static constexpr int OFF_KBT = OFF_KB + SZ_TOK;                   // Kb^T (bf16 only)
    static constexpr int OFF_RA = OFF_KBT + (kF32 ? 0 : DK * P64 * ES);   // Akk -> Tm (fp32)
    static constexpr int OFF_RT = OFF_RA + C * PA * 4;               // Tm Diag(beta) in E (bf16 only)
    static constexpr int OFF_QK = OFF_RT + (kF32 ? 0 : C * P64 * ES);    // Aqk
    static constexpr int OFF_VT = OFF_QK + C * P64 * ES;             // V^T slice
    static constexpr int OFF_ST = OFF_VT + DV * P64 * ES;            // S^T slice in E
    static constexpr int OFF_ZT = OFF_ST + DV * P128 * ES;           // (V - Kh S)^T
    static constexpr int OFF_VN = OFF_ZT + DV * P64 * ES;            // Vn^T
    static constexpr int OFF_GAM = OFF_VN + DV * P64 * ES;           // e^{G_64}
    static constexpr int OFF_BETA = OFF_GAM + DK * 4;
    static constexpr int OFF_TOT = OFF_BETA + C * 4;                 // per-wave column sums of g
    static constexpr int TOTAL = OFF_TOT + NW * DK * 4;
    static_assert(TOTAL <= 160 * 1024, "LDS budget");
    static_assert(!kF32 || P64 == PA, "fp32 Tm aliases Akk");
};

// Per-thread registers of one chunk's inputs (prefetched one chunk ahead).
//   q/k/g: channels 2cp, 2cp+1, rows RPT*wave .. RPT*wave + RPT-1
//   v    : channels 2jp, 2jp+1 of the slice, rows RVR*rgv .. +RVR-1
template <typename E, int DV>
struct ChunkIn {
    static constexpr int RVR = DV / 16;
    float2 g[RPT];
    typename Pair<E>::type q[RPT], k[RPT];
    typename Pair<E>::type v[RVR];
    float beta;
};

template <typename E, int DV>
__global__ void __launch_bounds__(NT)
chunk_fwd_kernel(const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
                 const float* __restrict__ g, const E* __restrict__ beta,
                 const float* __restrict__ S0, E* __restrict__ o, float* __restrict__ S_T,
                 int T, int H, int nsplit)
{
    using L = Layout<E, DV>;
    using In = ChunkIn<E, DV>;
    using PairT = typename Pair<E>::type;
    using M = Mma<E>;
    constexpr int NJ = DV / 16;             // value-column tiles in the slice
    constexpr int RVR = In::RVR;
    constexpr int VP = DV / 2;              // value channel pairs

    __shared__ __attribute__((aligned(16))) char smem[L::TOTAL];
    E* sQt = reinterpret_cast<E*>(smem + L::OFF_QT);
    E* sKh = reinterpret_cast<E*>(smem + L::OFF_KH);
    E* sKb = reinterpret_cast<E*>(smem + L::OFF_KB);
    E* sKbT = reinterpret_cast<E*>(smem + L::OFF_KBT);
    float* RA = reinterpret_cast<float*>(smem + L::OFF_RA);
    E* RT = reinterpret_cast<E*>(smem + (L::kF32 ? L::OFF_RA : L::OFF_RT));
    E* sQK = reinterpret_cast<E*>(smem + L::OFF_QK);
    E* sVT = reinterpret_cast<E*>(smem + L::OFF_VT);
    E* sST = reinterpret_cast<E*>(smem + L::OFF_ST);
    E* sZT = reinterpret_cast<E*>(smem + L::OFF_ZT);
    E* sVN = reinterpret_cast<E*>(smem + L::OFF_VN);
    float* s_gam = reinterpret_cast<float*>(smem + L::OFF_GAM);
    float* s_beta = reinterpret_cast<float*>(smem + L::OFF_BETA);
    float* s_tot = reinterpret_cast<float*>(smem + L::OFF_TOT);

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int cp = t & 63;                  // channel pair for q/k/g work
    const int jp = t % VP, rgv = t / VP;    // value pair / row group for v
    const int ln = lane & 15, lg = lane >> 4;

    // Workgroup -> (head, slice), keeping the slices of a head on one XCD
    // (workgroups are dealt to the 8 XCDs round-robin).
    const int nwg = gridDim.x, w = blockIdx.x;
    const int lid = (nwg % 8 == 0) ? (w % 8) * (nwg / 8) + w / 8 : w;
    const int head = lid / nsplit, slice = lid % nsplit;
    const int b = head / H, h = head % H;
    const int j0 = slice * DV;

    const size_t tokstride = (size_t)H * DK;                       // one token, all heads
    const size_t hbase = ((size_t)b * T * H + h) * DK;             // (b, t=0, h, 0)
    const size_t sbase = (size_t)head * DK * DK;                   // state of this head
    const int nchunks = (T + C - 1) / C;

    auto load_chunk = [&](int n, In& in) {
        const int tok0 = n * C;
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int tok = tok0 + RPT * wave + i;
            if (tok < T) {
                const size_t off = hbase + (size_t)tok * tokstride + 2 * cp;
                in.g[i] = *reinterpret_cast<const float2*>(g + off);
                in.q[i] = *reinterpret_cast<const PairT*>(q + off);
                in.k[i] = *reinterpret_cast<const PairT*>(k + off);
            } else {
                in.g[i] = make_float2(0.f, 0.f);
                in.q[i] = pack<E>(0.f, 0.f);
                in.k[i] = pack<E>(0.f, 0.f);
            }
        }
#pragma unroll
        for (int i = 0; i < RVR; ++i) {
            const int tok = tok0 + RVR * rgv + i;
            in.v[i] = tok < T ? *reinterpret_cast<const PairT*>(v + hbase + (size_t)tok * tokstride + j0 + 2 * jp)
                              : pack<E>(0.f, 0.f);
        }
        if (t < C) {
            const int tok = tok0 + t;
            in.beta = tok < T ? to_f32(beta[((size_t)b * T + tok) * H + h]) : 0.f;
        }
    };

    // ---- state slice in accumulators: wave w owns rows 16w..16w+15 ------------
    f32x4 acc_s[NJ];
#pragma unroll
    for (int jb = 0; jb < NJ; ++jb) {
        const int c = 16 * wave + 4 * lg, j = j0 + 16 * jb + ln;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc_s[jb][e] = S0 ? S0[sbase + (size_t)(c + e) * DK + j] : 0.f;
    }
    auto write_state_lds = [&]() {
#pragma unroll
        for (int jb = 0; jb < NJ; ++jb)
            store_vec4<E>(sST + (16 * jb + ln) * L::P128 + 16 * wave + 4 * lg, acc_s[jb]);
    };
    write_state_lds();

    In in;
    load_chunk(0, in);

    for (int n = 0; n < nchunks; ++n) {
        // ===== E: cumulative log-decay and the decay-scaled operands =====
        float G0[RPT], G1[RPT];
        {
            float r0 = 0.f, r1 = 0.f;
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                r0 += in.g[i].x; r1 += in.g[i].y;
                G0[i] = r0; G1[i] = r1;
            }
            s_tot[wave * DK + 2 * cp] = r0;
            s_tot[wave * DK + 2 * cp + 1] = r1;
            if (t < C) s_beta[t] = in.beta;
        }
        lds_barrier();
        {
            float off0 = 0.f, off1 = 0.f, tot0 = 0.f, tot1 = 0.f;
#pragma unroll
            for (int w2 = 0; w2 < NW; ++w2) {
                const float a0 = s_tot[w2 * DK + 2 * cp], a1 = s_tot[w2 * DK + 2 * cp + 1];
                if (w2 < wave) { off0 += a0; off1 += a1; }
                tot0 += a0; tot1 += a1;
            }
            if (wave == 0) { s_gam[2 * cp] = exp_fast(tot0); s_gam[2 * cp + 1] = exp_fast(tot1); }
            float kb0[RPT], kb1[RPT];
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const int r = RPT * wave + i;
                const float Ga = G0[i] + off0, Gb = G1[i] + off1;
                const float e0 = exp_fast(Ga), e1 = exp_fast(Gb);
                const float n0 = exp_fast(-Ga), n1 = exp_fast(-Gb);
                const float2 qf = unpack(in.q[i]), kf = unpack(in.k[i]);
                kb0[i] = kf.x * n0; kb1[i] = kf.y * n1;
                *reinterpret_cast<PairT*>(sQt + r * L::P128 + 2 * cp) = pack<E>(qf.x * e0, qf.y * e1);
                *reinterpret_cast<PairT*>(sKh + r * L::P128 + 2 * cp) = pack<E>(kf.x * e0, kf.y * e1);
                *reinterpret_cast<PairT*>(sKb + r * L::P128 + 2 * cp) = pack<E>(kb0[i], kb1[i]);
            }
            if constexpr (!L::kF32) {
                store_run<E, RPT>(sKbT + (2 * cp) * L::P64 + RPT * wave, kb0);
                store_run<E, RPT>(sKbT + (2 * cp + 1) * L::P64 + RPT * wave, kb1);
            }
            float va[RVR], vb[RVR];
#pragma unroll
            for (int i = 0; i < RVR; ++i) {
                const float2 vf = unpack(in.v[i]);
                va[i] = vf.x; vb[i] = vf.y;
            }
            store_run<E, RVR>(sVT + (2 * jp) * L::P64 + RVR * rgv, va);
            store_run<E, RVR>(sVT + (2 * jp + 1) * L::P64 + RVR * rgv, vb);
        }
        lds_barrier();

        // prefetch the next chunk while this one is computed
        if (n + 1 < nchunks) load_chunk(n + 1, in);

        // ===== M1 (waves 0-3): Aqk, Akk.  P (waves 4-7): Kh S, then Z = V - Kh S =====
        if (wave < 4) {
            // Aqk^T / Akk^T tiles (rows i in block I, columns r in block R >= I);
            // the A operand (Kb rows of block I) is shared by the wave's tiles.
            auto epilogue = [&](const f32x4& acc, int I, int R, bool kk) {
                const int r = 16 * R + ln, i0 = 16 * I + 4 * lg;
                f32x4 val;
                const float bt = kk ? s_beta[r] : 1.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) val[e] = (kk ? (i0 + e < r) : (i0 + e <= r)) ? bt * acc[e] : 0.f;
                if (kk) *reinterpret_cast<f32x4*>(RA + r * L::PA + i0) = val;
                else store_vec4<E>(sQK + r * L::P64 + i0, val);
            };
            const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
            if (wave < 2) {               // I = 0, R = 0..3, one matrix per wave
                const bool kk = wave == 1;
                f32x4 acc[4] = {z4, z4, z4, z4};
                const int br[4] = {0, 16, 32, 48};
                mma_rows<E, DK, 4>(acc, sKb, L::P128, 0, kk ? sKh : sQt, L::P128, br, lane);
#pragma unroll
                for (int R = 0; R < 4; ++R) epilogue(acc[R], 0, R, kk);
            } else if (wave == 2) {       // I = 1, R = 1..3, both matrices
                f32x4 acc[6] = {z4, z4, z4, z4, z4, z4};
                {
                    f32x4 a3[3] = {z4, z4, z4};
                    const int br[3] = {16, 32, 48};
                    mma_rows<E, DK, 3>(a3, sKb, L::P128, 16, sQt, L::P128, br, lane);
                    acc[0] = a3[0]; acc[1] = a3[1]; acc[2] = a3[2];
                    f32x4 b3[3] = {z4, z4, z4};
                    mma_rows<E, DK, 3>(b3, sKb, L::P128, 16, sKh, L::P128, br, lane);
                    acc[3] = b3[0]; acc[4] = b3[1]; acc[5] = b3[2];
                }
#pragma unroll
                for (int R = 1; R < 4; ++R) { epilogue(acc[R - 1], 1, R, false); epilogue(acc[R + 2], 1, R, true); }
            } else {                      // I = 2 (R = 2, 3) and I = 3 (R = 3), both matrices
                f32x4 a2[2] = {z4, z4}, b2[2] = {z4, z4};
                const int br[2] = {32, 48};
                mma_rows<E, DK, 2>(a2, sKb, L::P128, 32, sQt, L::P128, br, lane);
                mma_rows<E, DK, 2>(b2, sKb, L::P128, 32, sKh, L::P128, br, lane);
                f32x4 a1[1] = {z4}, b1[1] = {z4};
                const int br1[1] = {48};
                mma_rows<E, DK, 1>(a1, sKb, L::P128, 48, sQt, L::P128, br1, lane);
                mma_rows<E, DK, 1>(b1, sKb, L::P128, 48, sKh, L::P128, br1, lane);
                epilogue(a2[0], 2, 2, false); epilogue(a2[1], 2, 3, false);
                epilogue(b2[0], 2, 2, true); epilogue(b2[1], 2, 3, true);
                epilogue(a1[0], 3, 3, false); epilogue(b1[0], 3, 3, true);
                // zero the upper tiles (I > R) of Aqk and Akk
                for (int u = 0; u < 6; ++u) {
                    const int I = u < 3 ? u + 1 : (u < 5 ? u - 1 : 3);
                    const int R = u < 3 ? 0 : (u < 5 ? 1 : 2);
                    const int r = 16 * R + ln, i0 = 16 * I + 4 * lg;
                    *reinterpret_cast<f32x4*>(RA + r * L::PA + i0) = z4;
                    store_vec4<E>(sQK + r * L::P64 + i0, z4);
                }
            }
        }
        f32x4 pacc[NJ];
        if (wave >= 4) {                  // P tiles (R = wave - 4, all column blocks)
            const int R = wave - 4;
            int br[NJ];
#pragma unroll
            for (int jb = 0; jb < NJ; ++jb) { pacc[jb] = f32x4{0.f, 0.f, 0.f, 0.f}; br[jb] = 16 * jb; }
            mma_rows<E, DK, NJ>(pacc, sKh, L::P128, 16 * R, sST, L::P128, br, lane);
        }
        lds_barrier();

        // ===== UT transform, diagonal blocks (wave 0) | Z = V - Kh S (waves 4-7) =====
        if (wave == 0) {
            // column m of X = (I + A_bb)^{-1} for block bb, right-looking substitution
            const int bb = lane >> 4, m = lane & 15;
            float* A = RA + 16 * bb * L::PA + 16 * bb;
            float x[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) x[i] = (i == m) ? 1.f : 0.f;
#pragma unroll
            for (int j = 0; j < 15; ++j) {
#pragma unroll
                for (int i = j + 1; i < 16; ++i) x[i] -= A[i * L::PA + j] * x[j];
                __builtin_amdgcn_sched_barrier(0);   // keep one column of loads in flight
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) A[i * L::PA + m] = x[i];
        } else if (wave >= 4) {
            const int R = wave - 4;
#pragma unroll
            for (int jb = 0; jb < NJ; ++jb) {
                const int j = 16 * jb + ln, r = 16 * R + 4 * lg;
                const f32x4 vv = load_vec4<E>(sVT + j * L::P64 + r);
                store_vec4<E>(sZT + j * L::P64 + r, vv - pacc[jb]);
            }
        }
        lds_barrier();

        // ===== UT transform, off-diagonal blocks; then Tm Diag(beta) in E =====
        if constexpr (!L::kF32) {
            // Column I = wave (0..2): X_RI = -X_RR sum_{J=I}^{R-1} A_RJ X_JI, chained
            // through registers with 16x16x16 bf16 MFMAs (the D layout of one
            // product is the B layout of the next).  Results go straight to RT,
            // scaled by beta of their column.  Wave 3 writes the diagonal blocks,
            // waves 4-7 clear the upper blocks of RT.
            if (wave == 0) ut_offdiag_column<0, L::PA, L::P64>(RA, RT, s_beta, lane);
            else if (wave == 1) ut_offdiag_column<1, L::PA, L::P64>(RA, RT, s_beta, lane);
            else if (wave == 2) ut_offdiag_column<2, L::PA, L::P64>(RA, RT, s_beta, lane);
            else if (wave == 3) {
#pragma unroll
                for (int bb = 0; bb < 4; ++bb) {
                    const int r = 16 * bb + 4 * lg;
                    const float bcol = s_beta[16 * bb + ln];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        RT[(r + e) * L::P64 + 16 * bb + ln] = (E)(bcol * RA[(r + e) * L::PA + 16 * bb + ln]);
                }
            } else {
                for (int u = wave - 4; u < 6; u += 4) {
                    const int I = u < 3 ? u + 1 : (u < 5 ? u - 1 : 3);
                    const int R = u < 3 ? 0 : (u < 5 ? 1 : 2);
                    store_vec4<E>(RT + (16 * R + ln) * L::P64 + 16 * I + 4 * lg, f32x4{0.f, 0.f, 0.f, 0.f});
                }
            }
            lds_barrier();
        } else {
            // fp32: block rows R = 1..3 by plain dot products, in place in RA,
            // then scale the columns by beta.
            float* s_z = reinterpret_cast<float*>(sVN);   // Vn^T is not in use yet
            static_assert(16 * 48 * 4 <= DV * L::P64 * L::ES, "scratch fits in the Vn^T buffer");
            for (int R = 1; R < 4; ++R) {
                const int w16 = 16 * R;
                for (int e = t; e < 16 * w16; e += NT) {   // Z = -sum_J A_RJ X_J.
                    const int r = e / w16, i = e % w16;
                    const float* arow = RA + (w16 + r) * L::PA;
                    float s = 0.f;
                    for (int j = i; j < w16; ++j) s += arow[j] * RA[j * L::PA + i];
                    s_z[e] = -s;
                }
                lds_barrier();
                for (int e = t; e < 16 * w16; e += NT) {   // X_R. = X_RR Z
                    const int r = e / w16, i = e % w16;
                    const float* xrow = RA + (w16 + r) * L::PA + w16;
                    float s = 0.f;
                    for (int rp = 0; rp <= r; ++rp) s += xrow[rp] * s_z[rp * w16 + i];
                    RA[(w16 + r) * L::PA + i] = s;
                }
                lds_barrier();
            }
            for (int e = t; e < C * C; e += NT) {
                const int r = e >> 6, i = e & 63;
                RA[r * L::PA + i] *= s_beta[i];
            }
            lds_barrier();
        }

        // ===== Vn = Tm Diag(beta) Z; tiles (R, jb), A operand shared per wave =====
        {
            constexpr int NVT = 4 * NJ;            // tiles
            constexpr int PER = (NVT + NW - 1) / NW;
            if (wave < NVT) {
                const int R = wave % 4;
                f32x4 acc[PER];
                int br[PER];
#pragma unroll
                for (int u = 0; u < PER; ++u) {
                    acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
                    const int jb = (wave / 4) + 2 * u;
                    br[u] = 16 * (jb < NJ ? jb : 0);
                }
                mma_rows<E, C, PER>(acc, RT, L::P64, 16 * R, sZT, L::P64, br, lane);
#pragma unroll
                for (int u = 0; u < PER; ++u) {
                    const int jb = (wave / 4) + 2 * u;
                    if (jb < NJ) store_vec4<E>(sVN + (16 * jb + ln) * L::P64 + 16 * R + 4 * lg, acc[u]);
                }
            }
        }
        lds_barrier();

        // ===== O = Qt S + Aqk Vn (to HBM) | S <- Diag(gamma) (S + Kb^T Vn) =====
        {
            constexpr int NOT = 4 * NJ;
            constexpr int PER = (NOT + NW - 1) / NW;
            const int ot0 = PER * wave;
            if (ot0 < NOT) {
                const int jb = ot0 / 4;
                f32x4 acc[PER];
                int br[PER];
#pragma unroll
                for (int u = 0; u < PER; ++u) { acc[u] = f32x4{0.f, 0.f, 0.f, 0.f}; br[u] = 16 * ((ot0 + u) % 4); }
                mma_rows<E, DK, PER>(acc, sST, L::P128, 16 * jb, sQt, L::P128, br, lane);
                mma_rows<E, C, PER>(acc, sVN, L::P64, 16 * jb, sQK, L::P64, br, lane);
#pragma unroll
                for (int u = 0; u < PER; ++u) {
                    const int r = br[u] + ln, tok = n * C + r;
                    if (tok < T) store_vec4<E>(o + hbase + (size_t)tok * tokstride + j0 + 16 * jb + 4 * lg, acc[u]);
                }
            }
            int br[NJ];
#pragma unroll
            for (int jb = 0; jb < NJ; ++jb) br[jb] = 16 * jb;
            if constexpr (L::kF32) {
                // A operand Kb^T read from the token-major Kb
#pragma unroll
                for (int kk = 0; kk < C; kk += M::KS) {
                    const float a = M::frag_mc(sKb, L::P128, 16 * wave, kk, lane);
#pragma unroll
                    for (int jb = 0; jb < NJ; ++jb)
                        acc_s[jb] = M::mma(a, M::frag_kc(sVN, L::P64, br[jb], kk, lane), acc_s[jb]);
                }
            } else {
                mma_rows<E, C, NJ>(acc_s, sKbT, L::P64, 16 * wave, sVN, L::P64, br, lane);
            }
            const int c = 16 * wave + 4 * lg;
#pragma unroll
            for (int jb = 0; jb < NJ; ++jb)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc_s[jb][e] *= s_gam[c + e];
        }
        lds_barrier();
        write_state_lds();
    }

    if (S_T) {
#pragma unroll
        for (int jb = 0; jb < NJ; ++jb) {
            const int c = 16 * wave + 4 * lg, j = j0 + 16 * jb + ln;
#pragma unroll
            for (int e = 0; e < 4; ++e) S_T[sbase + (size_t)(c + e) * DK + j] = acc_s[jb][e];
        }
    }
}

template <typename E, int DV>
void launch_one(const void* q, const void* k, const void* v, const float* g, const void* beta,
                const float* S0, void* o, float* S_T, int B, int T, int H, hipStream_t stream)
{
    const int nsplit = DK / DV;
    const unsigned nwg = (unsigned)((long long)B * H * nsplit);
    hipLaunchKernelGGL((chunk_fwd_kernel<E, DV>), dim3(nwg), dim3(NT), 0, stream,
                       (const E*)q, (const E*)k, (const E*)v, g, (const E*)beta, S0, (E*)o, S_T,
                       T, H, nsplit);
}

}  // namespace

hipError_t launch_chunk_fwd(const void* q, const void* k, const void* v, const float* g,
                            const void* beta, const float* S0, void* o, float* S_T,
                            int B, int T, int H, int dtype, hipStream_t stream)
{
    const long long heads = (long long)B * H;
    if (dtype == 0) {
        // fp32 operands need the narrowest slice to fit the LDS budget
        launch_one<float, 16>(q, k, v, g, beta, S0, o, S_T, B, T, H, stream);
    } else if (heads * 2 >= 256) {
        launch_one<bf16_t, 64>(q, k, v, g, beta, S0, o, S_T, B, T, H, stream);
    } else if (heads * 4 >= 256) {
        launch_one<bf16_t, 32>(q, k, v, g, beta, S0, o, S_T, B, T, H, stream);
    } else {
        launch_one<bf16_t, 16>(q, k, v, g, beta, S0, o, S_T, B, T, H, stream);
    }
    return hipGetLastError();
}

}  // namespace kda
