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
#include "kda_chunk_common.h"
#include "kda_device.h"
#include "kda_internal.h"

#include <type_traits>

namespace kda {
namespace {

constexpr int NW = 8;     // waves per workgroup (two per SIMD)
constexpr int NT = 64 * NW;
constexpr int RPT = C / NW;   // rows per wave in the elementwise phase (8)
constexpr int RPL = RPT / 4;  // rows per lane in the elementwise phase (2)

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
    static constexpr int OFF_KH = OFF_QT + SZ_TOK;                    // Kh = e^G k (right after Qt)
    static constexpr int OFF_KB = OFF_KH + SZ_TOK;                    // Kb = e^-G k
    static constexpr int OFF_KBT = OFF_KB + SZ_TOK;                   // Kb^T (bf16 only)
    static constexpr int OFF_RA = OFF_KBT + (kF32 ? 0 : DK * P64 * ES);   // Akk -> Tm (fp32)
    static constexpr int OFF_RT = OFF_RA + C * PA * 4;               // Tm Diag(beta) in E (bf16 only)
    static constexpr int OFF_QK = OFF_RT + (kF32 ? 0 : C * P64 * ES);    // Aqk
    static constexpr int PV = DV + PAD;     // token-major [64][DV] rows
    static constexpr int OFF_V = OFF_QK + C * P64 * ES;              // V slice, token-major
    static constexpr int OFF_ST = OFF_V + C * PV * ES;               // S^T slice in E
    static constexpr int OFF_ZT = OFF_ST + DV * P128 * ES;           // (V - Kh S)^T
    static constexpr int OFF_VN = OFF_ZT + DV * P64 * ES;            // Vn^T
    static constexpr int OFF_GAM = OFF_VN + DV * P64 * ES;           // e^{G_64}
    static constexpr int OFF_BETA = OFF_GAM + DK * 4;
    static constexpr int OFF_TOT = OFF_BETA + C * 4;                 // per-wave column sums of g
    static constexpr int TOTAL = OFF_TOT + NW * DK * 4;
    static_assert(TOTAL <= 160 * 1024, "LDS budget");
    static_assert(!kF32 || P64 == PA, "fp32 Tm aliases Akk");
    // Kb^T (channel-major, 64 tokens per row) is stored with its 8-token
    // blocks XOR-swizzled by bits 3..5 of the channel, so that the elementwise
    // phase (lanes 8 channels apart) writes it without bank conflicts while the
    // MFMA fetch (8 consecutive channels, one 8-token block) stays conflict-free.
    static constexpr int PDT = 16 + 4;      // fp32 rows of the transposed diagonal blocks
    static_assert(4 * (DV / 16) * 64 * 16 <= SZ_TOK, "parked output tiles fit in the Kh buffer");
    static_assert(kF32 || C * PDT * 4 <= C * P64 * ES, "transposed blocks fit in the Tm buffer");
    __device__ static constexpr int kbt(int c, int i) {
        return c * P64 + ((((i >> 3) ^ ((c >> 3) & 7)) << 3) | (i & 7));
    }
};

// Per-thread registers of one chunk's inputs (prefetched one chunk ahead),
// all fetched with 16-byte loads:
//   q/k/g: channels 8cg .. 8cg+7, rows RPT*wave + RPL*rq + i (i < RPL)
//   v    : channels 8vg .. 8vg+7 of the slice, rows RVR*vr + i (i < RVR)
template <typename E, int DV>
struct ChunkIn {
    static constexpr int VL = DV / 8;                   // lanes per value row
    static constexpr int RVR = (64 * VL + NT - 1) / NT; // value rows per thread
    Raw8f g[RPL];
    Raw8<E> q[RPL], k[RPL];
    Raw8<E> v[RVR];
    E beta;
};

// Workspace block of one chunk, written by the prep instantiation of the
// kernel below and read by chunk_scan_kernel (bf16 only).  Byte offsets:
constexpr int WS_QT = 0;                       // Qt   [64][128] bf16, token-major
constexpr int WS_KH = WS_QT + C * DK * 2;      // Kh   [64][128] bf16, token-major
constexpr int WS_KBT = WS_KH + C * DK * 2;     // Kb^T [128][64] bf16, channel-major
constexpr int WS_TM = WS_KBT + DK * C * 2;     // Tm Diag(beta) [64][64] bf16
constexpr int WS_QK = WS_TM + C * C * 2;       // Aqk  [64][64] bf16
constexpr int WS_GAM = WS_QK + C * C * 2;      // e^{G_64} [128] fp32
constexpr int WS_CHUNK = WS_GAM + DK * 4;      // 66,048 bytes

// The fused kernel (PREP = false): one workgroup per (head, value slice)
// walks all chunks of its head.  The prep instantiation (PREP = true): one
// workgroup per (head, chunk) runs only the key-side work -- decay, Aqk, Akk,
// Tm -- and exports it to the workspace for chunk_scan_kernel.
template <typename E, int DV, bool PREP>
__global__ void __launch_bounds__(NT)
chunk_fwd_kernel(const E* q, const E* k, const E* v, const float* g, const E* beta,
                 const float* S0, E* o, float* S_T, int T, int H, int nsplit, char* ws)
{
    // (No __restrict__ on the inputs: the LDS barriers are asm statements with
    // a memory clobber, and without restrict the compiler keeps the prefetch
    // loads where they are written instead of sinking them towards their use.)
    using L = Layout<E, DV>;
    using In = ChunkIn<E, DV>;
    using PairT = typename Pair<E>::type;
    using M = Mma<E>;
    constexpr int NJ = DV / 16;             // value-column tiles in the slice
    constexpr int RVR = In::RVR;
    constexpr int NO = 4 * NJ;              // output tiles (jb, R)
    constexpr int MO = (NO + NW - 2) / (NW - 1);   // output tiles per wave (waves 1..NW-1)

    __shared__ __attribute__((aligned(16))) char smem[L::TOTAL];
    E* sQt = reinterpret_cast<E*>(smem + L::OFF_QT);
    E* sKh = reinterpret_cast<E*>(smem + L::OFF_KH);
    E* sKb = reinterpret_cast<E*>(smem + L::OFF_KB);
    E* sKbT = reinterpret_cast<E*>(smem + L::OFF_KBT);
    float* RA = reinterpret_cast<float*>(smem + L::OFF_RA);
    E* RT = reinterpret_cast<E*>(smem + (L::kF32 ? L::OFF_RA : L::OFF_RT));
    // transposed diagonal blocks of Akk, [block][j][i] = Akk_block[i][j]; lives
    // in the Tm buffer, which is only written after the substitution
    float* sDT = reinterpret_cast<float*>(smem + L::OFF_RT);
    // inter-chunk output tiles Qt S (fp32, one f32x4 per lane per tile), parked
    // in the Kh buffer, which is dead once Akk and Kh S are formed
    float* sOI = reinterpret_cast<float*>(smem + L::OFF_KH);
    E* sQK = reinterpret_cast<E*>(smem + L::OFF_QK);
    E* sV = reinterpret_cast<E*>(smem + L::OFF_V);
    E* sST = reinterpret_cast<E*>(smem + L::OFF_ST);
    E* sZT = reinterpret_cast<E*>(smem + L::OFF_ZT);
    E* sVN = reinterpret_cast<E*>(smem + L::OFF_VN);
    float* s_gam = reinterpret_cast<float*>(smem + L::OFF_GAM);
    float* s_beta = reinterpret_cast<float*>(smem + L::OFF_BETA);
    float* s_tot = reinterpret_cast<float*>(smem + L::OFF_TOT);

    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);   // uniform per wave
    const int cg = lane & 15, rq = lane >> 4;   // 8-channel group and row quad for q/k/g
    const int vg = t % In::VL, vr = t / In::VL; // 8-channel group and row group for v
    const int ln = lane & 15, lg = lane >> 4;

    const int nchunks = (T + C - 1) / C;
    // Workgroup -> (head, slice), keeping the slices of a head on one XCD
    // (workgroups are dealt to the 8 XCDs round-robin); prep: (head, chunk).
    const int nwg = gridDim.x, w = blockIdx.x;
    const int lid = (!PREP && nwg % 8 == 0) ? (w % 8) * (nwg / 8) + w / 8 : w;
    const int head = PREP ? lid / nchunks : lid / nsplit;
    const int slice = PREP ? 0 : lid % nsplit;
    const int b = head / H, h = head % H;
    const int j0 = slice * DV;
    const int n_first = PREP ? lid % nchunks : 0;
    const int n_end = PREP ? n_first + 1 : nchunks;

    const size_t tokstride = (size_t)H * DK;                       // one token, all heads
    const size_t hbase = ((size_t)b * T * H + h) * DK;             // (b, t=0, h, 0)
    const size_t sbase = (size_t)head * DK * DK;                   // state of this head

    // Prefetch of one chunk into registers.  Branch-free: rows past T read the
    // last valid token (always in bounds) and are zeroed when consumed, so no
    // load result is needed before the next chunk starts.
    const E* betap = beta + (size_t)b * T * H + h;
    auto load_chunk = [&](int n, In& in) {
        const int tok0 = n * C;
#pragma unroll
        for (int i = 0; i < RPL; ++i) {
            const int tok = min(tok0 + RPT * wave + RPL * rq + i, T - 1);
            const size_t off = hbase + (size_t)tok * tokstride + 8 * cg;
            in.g[i].load(g + off);
            in.q[i].load(q + off);
            in.k[i].load(k + off);
        }
        if constexpr (!PREP) {
#pragma unroll
            for (int i = 0; i < RVR; ++i) {
                const int tok = min(tok0 + RVR * vr + i, T - 1);
                if (RVR * vr + i < C)
                    in.v[i].load(v + hbase + (size_t)tok * tokstride + j0 + 8 * vg);
            }
        }
        in.beta = betap[(size_t)min(tok0 + lane, T - 1) * H];
    };

    // ---- state slice in accumulators: wave w owns rows 16w .. 16w+15 ----------
    f32x4 acc_s[NJ];
    if constexpr (!PREP)
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
    if constexpr (!PREP) write_state_lds();

    In in;
    load_chunk(n_first, in);
    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};

    for (int n = n_first; n < n_end; ++n) {
        const bool full = (n + 1) * C <= T;     // uniform: no row of this chunk is past T

        // ===== E: cumulative log2-decay and the decay-scaled operands =====
        // G is kept in log2 units so that 2^G = e^{sum g}.  Each lane owns
        // 8 channels x 2 consecutive rows; the prefix over rows is local, then
        // across the 4 row pairs of a wave (row-swap exchanges), then across
        // waves (LDS).
        // Full chunks take a path without per-row masking.
        auto ephase = [&](auto masked_t) {
            constexpr bool MASKED = decltype(masked_t)::value;
            auto row_ok = [&](int r) { return !MASKED || n * C + r < T; };
            const int r0 = RPT * wave + RPL * rq;
            float G[RPL][8];
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                float run = 0.f;
#pragma unroll
                for (int i = 0; i < RPL; ++i) {
                    const float gi = in.g[i][c] * LOG2E;
                    run += row_ok(r0 + i) ? gi : 0.f;
                    G[i][c] = run;
                }
                // inclusive scan over rq: pairs (0,1), (2,3), then the lower
                // pair's total into the upper pair
                const float p16 = lane_xor16(run, lane);
                const float p32 = lane_xor32(run + p16, lane);   // other pair's total
                const float inc = run + ((rq & 1) ? p16 : 0.f) + ((rq & 2) ? p32 : 0.f);
                const float excl = inc - run;
#pragma unroll
                for (int i = 0; i < RPL; ++i) G[i][c] += excl;
                if (rq == 3) s_tot[wave * DK + 8 * cg + c] = inc;
            }
            if (wave == 0) s_beta[lane] = row_ok(lane) ? to_f32(in.beta) : 0.f;
            lds_barrier();
            // per channel: exclusive prefix of the wave totals, in place, and e^{G_64}
            if (t < DK) {
                float acc = 0.f;
#pragma unroll
                for (int w2 = 0; w2 < NW; ++w2) {
                    const float a = s_tot[w2 * DK + t];
                    s_tot[w2 * DK + t] = acc;
                    acc += a;
                }
                s_gam[t] = __builtin_amdgcn_exp2f(acc);
            }
            lds_barrier();
            {
                const f32x4 o0 = *reinterpret_cast<const f32x4*>(s_tot + wave * DK + 8 * cg);
                const f32x4 o1 = *reinterpret_cast<const f32x4*>(s_tot + wave * DK + 8 * cg + 4);
#pragma unroll
                for (int i = 0; i < RPL; ++i)
#pragma unroll
                    for (int c = 0; c < 4; ++c) { G[i][c] += o0[c]; G[i][c + 4] += o1[c]; }
            }
            float kb[RPL][8];
#pragma unroll
            for (int i = 0; i < RPL; ++i) {
                const int r = r0 + i;
                const bool ok = row_ok(r);
                float qe[8], ke[8];
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    const float e = __builtin_amdgcn_exp2f(G[i][c]), ne = __builtin_amdgcn_exp2f(-G[i][c]);
                    const float qv = ok ? in.q[i][c] : 0.f, kv = ok ? in.k[i][c] : 0.f;
                    qe[c] = qv * e; ke[c] = kv * e; kb[i][c] = kv * ne;
                }
                store8<E>(sQt + r * L::P128 + 8 * cg, qe);
                store8<E>(sKh + r * L::P128 + 8 * cg, ke);
                store8<E>(sKb + r * L::P128 + 8 * cg, kb[i]);
            }
            if constexpr (!L::kF32) {
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    float col[RPL];
#pragma unroll
                    for (int i = 0; i < RPL; ++i) col[i] = kb[i][c];
                    store_run<E, RPL>(sKbT + L::kbt(8 * cg + c, r0), col);
                }
            }
            if (!PREP && RVR * vr < C) {
#pragma unroll
                for (int i = 0; i < RVR; ++i) {
                    const bool ok = row_ok(RVR * vr + i);
                    float row[8];
#pragma unroll
                    for (int c = 0; c < 8; ++c) row[c] = ok ? in.v[i][c] : 0.f;
                    store8<E>(sV + (RVR * vr + i) * L::PV + 8 * vg, row);
                }
            }
        };
        if (full) ephase(std::false_type{});
        else ephase(std::true_type{});
        lds_barrier();

        // ===== M1: Aqk, Akk (waves 0-3) | P = Kh S, Z = V - P (waves 4-7) =====
        {
            // Aqk^T / Akk^T tiles: rows i in block I (A operand = Kb rows, shared
            // by the wave's tiles), columns r in block R >= I.  Kh sits right
            // after Qt in LDS, so Kh row r is row 64 + r of the Qt base.
            auto epilogue = [&](const f32x4& acc, int I, int R, bool kk) {
                const int r = 16 * R + ln, i0 = 16 * I + 4 * lg;
                f32x4 val;
                const float bt = kk ? s_beta[r] : 1.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) val[e] = (kk ? (i0 + e < r) : (i0 + e <= r)) ? bt * acc[e] : 0.f;
                if (kk) *reinterpret_cast<f32x4*>(RA + r * L::PA + i0) = val;
                else store_vec4<E>(sQK + r * L::P64 + i0, val);
                if constexpr (!L::kF32) {
                    // diagonal Akk blocks again, transposed, for the substitution
                    if (kk && I == R) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) sDT[(16 * R + 4 * lg + e) * L::PDT + ln] = val[e];
                    }
                }
            };
            // 20 tiles over waves 0-3 (Kh row r is row 64 + r of the Qt base).
            if (wave == 0) {          // I = 0: Aqk R = 0..3, Akk R = 0
                f32x4 acc[5] = {z4, z4, z4, z4, z4};
                const int br[5] = {0, 16, 32, 48, 64};
                mma_rows<E, DK, 5>(acc, sKb, L::P128, 0, sQt, L::P128, br, lane);
#pragma unroll
                for (int R = 0; R < 4; ++R) epilogue(acc[R], 0, R, false);
                epilogue(acc[4], 0, 0, true);
            } else if (wave == 1) {   // I = 0: Akk R = 1..3;  I = 1: Aqk R = 1, 2
                f32x4 acc[3] = {z4, z4, z4};
                const int br[3] = {80, 96, 112};
                mma_rows<E, DK, 3>(acc, sKb, L::P128, 0, sQt, L::P128, br, lane);
                f32x4 acc2[2] = {z4, z4};
                const int br2[2] = {16, 32};
                mma_rows<E, DK, 2>(acc2, sKb, L::P128, 16, sQt, L::P128, br2, lane);
#pragma unroll
                for (int R = 1; R < 4; ++R) epilogue(acc[R - 1], 0, R, true);
                epilogue(acc2[0], 1, 1, false); epilogue(acc2[1], 1, 2, false);
            } else if (wave == 2) {   // I = 1: Aqk R = 3, Akk R = 1..3
                f32x4 acc[4] = {z4, z4, z4, z4};
                const int br[4] = {48, 80, 96, 112};
                mma_rows<E, DK, 4>(acc, sKb, L::P128, 16, sQt, L::P128, br, lane);
                epilogue(acc[0], 1, 3, false);
#pragma unroll
                for (int R = 1; R < 4; ++R) epilogue(acc[R], 1, R, true);
            } else if (wave == 3) {   // I = 2, 3 for both, and the zero upper tiles
                f32x4 acc[4] = {z4, z4, z4, z4};
                const int br[4] = {32, 48, 96, 112};
                mma_rows<E, DK, 4>(acc, sKb, L::P128, 32, sQt, L::P128, br, lane);
                f32x4 acc3[2] = {z4, z4};
                const int br3[2] = {48, 112};
                mma_rows<E, DK, 2>(acc3, sKb, L::P128, 48, sQt, L::P128, br3, lane);
                epilogue(acc[0], 2, 2, false); epilogue(acc[1], 2, 3, false);
                epilogue(acc[2], 2, 2, true); epilogue(acc[3], 2, 3, true);
                epilogue(acc3[0], 3, 3, false); epilogue(acc3[1], 3, 3, true);
#pragma unroll
                for (int u = 0; u < 6; ++u) {       // zero the upper tiles (I > R)
                    const int I = u < 3 ? u + 1 : (u < 5 ? u - 1 : 3);
                    const int R = u < 3 ? 0 : (u < 5 ? 1 : 2);
                    const int r = 16 * R + ln, i0 = 16 * I + 4 * lg;
                    // (bf16: only the lower blocks of Akk are ever read; fp32
                    // turns Akk into Tm in place, whose upper blocks are read)
                    if constexpr (L::kF32) *reinterpret_cast<f32x4*>(RA + r * L::PA + i0) = z4;
                    store_vec4<E>(sQK + r * L::P64 + i0, z4);
                }
            }
            // P tiles for token block R = wave - 4 (waves 4-7)
            auto p_block = [&](int R) {
                f32x4 pacc[NJ];
                int br[NJ];
#pragma unroll
                for (int jb = 0; jb < NJ; ++jb) { pacc[jb] = z4; br[jb] = 16 * jb; }
                mma_rows<E, DK, NJ>(pacc, sKh, L::P128, 16 * R, sST, L::P128, br, lane);
#pragma unroll
                for (int jb = 0; jb < NJ; ++jb) {
                    const int j = 16 * jb + ln, r = 16 * R + 4 * lg;
                    f32x4 vv;
#pragma unroll
                    for (int e = 0; e < 4; ++e) vv[e] = to_f32(sV[(r + e) * L::PV + j]);
                    store_vec4<E>(sZT + j * L::P64 + r, vv - pacc[jb]);
                }
            };
            if (!PREP && wave >= 4) p_block(wave - 4);
        }
        lds_barrier();

        // ===== UT diagonal blocks (wave 0) | inter-chunk output Qt S (waves 1-7) =====
        if (wave == 0) {
            // column m of X = (I + A_bb)^{-1} for block bb, right-looking substitution
            const int bb = lane >> 4, m = lane & 15;
            float* A = RA + 16 * bb * L::PA + 16 * bb;
            float x[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) x[i] = (i == m) ? 1.f : 0.f;
            // right-looking: once x[j] is final, column j of the block updates x[i > j]
            if constexpr (!L::kF32) {
                // column j is row j of the transposed block: four 16-byte loads,
                // fetched one step ahead
                const float* D = sDT + 16 * bb * L::PDT;
                f32x4 col[2][4];
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) col[0][q4] = *reinterpret_cast<const f32x4*>(D + 4 * q4);
#pragma unroll
                for (int j = 0; j < 15; ++j) {
                    if (j + 1 < 15) {
#pragma unroll
                        for (int q4 = 0; q4 < 4; ++q4)
                            col[(j + 1) & 1][q4] = *reinterpret_cast<const f32x4*>(D + (j + 1) * L::PDT + 4 * q4);
                    }
#pragma unroll
                    for (int i = j + 1; i < 16; ++i) x[i] -= col[j & 1][i >> 2][i & 3] * x[j];
                    __builtin_amdgcn_sched_barrier(0);
                }
            } else {
#pragma unroll
                for (int j = 0; j < 15; ++j) {
#pragma unroll
                    for (int i = j + 1; i < 16; ++i) x[i] -= A[i * L::PA + j] * x[j];
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) A[i * L::PA + m] = x[i];
        } else if constexpr (!PREP) {
            // output tiles t = (wave - 1) + (NW - 1) m: (jb = t / 4, R = t % 4)
#pragma unroll
            for (int m = 0; m < MO; ++m) {
                const int tt = (wave - 1) + (NW - 1) * m;
                if (tt < NO) {
                    f32x4 one[1] = {z4};
                    const int br[1] = {16 * (tt % 4)};
                    mma_rows<E, DK, 1>(one, sST, L::P128, 16 * (tt / 4), sQt, L::P128, br, lane);
                    *reinterpret_cast<f32x4*>(sOI + (tt * 64 + lane) * 4) = one[0];
                }
            }
        }
        lds_barrier();

        // Prefetch the next chunk while the rest of this one is computed.  It is
        // issued here, not earlier, so that its registers are free during the
        // register-heavy Akk/Aqk products and diagonal-block substitution.
        // Waves 3-7, which have little work in the off-diagonal step, issue
        // first; waves 0-2 issue after their substitution chains, so that the
        // chains do not queue behind the address unit.
        if (!PREP && wave >= 3 && n + 1 < nchunks) load_chunk(n + 1, in);

        // ===== UT off-diagonal blocks; Tm Diag(beta) in E =====
        if constexpr (!L::kF32) {
            if (wave == 0) ut_offdiag_column<0, L::PA, L::P64>(RA, RT, s_beta, lane);
            else if (wave == 1) ut_offdiag_column<1, L::PA, L::P64>(RA, RT, s_beta, lane);
            else if (wave == 2) ut_offdiag_column<2, L::PA, L::P64>(RA, RT, s_beta, lane);
            else if (wave == 3) {
                // diagonal blocks, scaled by beta of their column
#pragma unroll
                for (int bb = 0; bb < 4; ++bb) {
                    const int r = 16 * bb + 4 * lg;
                    const float bcol = s_beta[16 * bb + ln];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        RT[(r + e) * L::P64 + 16 * bb + ln] = (E)(bcol * RA[(r + e) * L::PA + 16 * bb + ln]);
                }
            } else {
                for (int u = wave - 4; u < 6; u += 4) {   // zero upper blocks of RT
                    const int I = u < 3 ? u + 1 : (u < 5 ? u - 1 : 3);
                    const int R = u < 3 ? 0 : (u < 5 ? 1 : 2);
                    store_vec4<E>(RT + (16 * R + ln) * L::P64 + 16 * I + 4 * lg, z4);
                }
            }
            if (!PREP && wave < 3 && n + 1 < nchunks) load_chunk(n + 1, in);
            lds_barrier();
        } else {
            if (!PREP && wave < 3 && n + 1 < nchunks) load_chunk(n + 1, in);
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

        if constexpr (PREP) {
            // ===== export the key-side operands of this chunk =====
            char* blk = ws + ((size_t)head * nchunks + n) * WS_CHUNK;
            typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;
            for (int u = t; u < C * DK / 8; u += NT) {            // Qt, Kh: [64][128]
                const int r = u >> 4, cb = u & 15;
                reinterpret_cast<i32x4*>(blk + WS_QT)[u] = *reinterpret_cast<const i32x4*>(sQt + r * L::P128 + 8 * cb);
                reinterpret_cast<i32x4*>(blk + WS_KH)[u] = *reinterpret_cast<const i32x4*>(sKh + r * L::P128 + 8 * cb);
            }
            for (int u = t; u < DK * C / 8; u += NT) {            // Kb^T: [128][64], unswizzled
                const int c = u >> 3, b8 = u & 7;
                reinterpret_cast<i32x4*>(blk + WS_KBT)[u] = *reinterpret_cast<const i32x4*>(sKbT + L::kbt(c, 8 * b8));
            }
            for (int u = t; u < C * C / 8; u += NT) {             // Tm Diag(beta), Aqk: [64][64]
                const int r = u >> 3, b8 = u & 7;
                reinterpret_cast<i32x4*>(blk + WS_TM)[u] = *reinterpret_cast<const i32x4*>(RT + r * L::P64 + 8 * b8);
                reinterpret_cast<i32x4*>(blk + WS_QK)[u] = *reinterpret_cast<const i32x4*>(sQK + r * L::P64 + 8 * b8);
            }
            if (t < DK / 4)
                reinterpret_cast<f32x4*>(blk + WS_GAM)[t] = reinterpret_cast<const f32x4*>(s_gam)[t];
            continue;
        }

        // ===== Vn = Tm Diag(beta) Z: wave w -> token block R = w % 4, column blocks w / 4 + 2u =====
        {
            constexpr int PER = (NJ + 1) / 2;
            const int R = wave % 4;
            if (wave / 4 < NJ) {
                f32x4 acc[PER];
                int br[PER];
#pragma unroll
                for (int u = 0; u < PER; ++u) {
                    acc[u] = z4;
                    const int jb = wave / 4 + 2 * u;
                    br[u] = 16 * (jb < NJ ? jb : 0);
                }
                mma_rows<E, C, PER>(acc, RT, L::P64, 16 * R, sZT, L::P64, br, lane);
#pragma unroll
                for (int u = 0; u < PER; ++u) {
                    const int jb = wave / 4 + 2 * u;
                    if (jb < NJ) store_vec4<E>(sVN + (16 * jb + ln) * L::P64 + 16 * R + 4 * lg, acc[u]);
                }
            }
        }
        lds_barrier();

        // ===== O += Aqk Vn (to HBM; the parked Qt S tiles, spread over all
        // waves) | S <- Diag(gamma) (S + Kb^T Vn) =====
        {
#pragma unroll
            for (int m = 0; m < (NO + NW - 1) / NW; ++m) {
                const int tt = wave + NW * m;
                if (tt < NO) {
                    const int jb = tt / 4, R = tt % 4;
                    f32x4 one[1] = {*reinterpret_cast<const f32x4*>(sOI + (tt * 64 + lane) * 4)};
                    const int br[1] = {16 * R};
                    mma_rows<E, C, 1>(one, sVN, L::P64, 16 * jb, sQK, L::P64, br, lane);
                    const int tok = n * C + 16 * R + ln;
                    if (full || tok < T)
                        store_vec4<E>(o + hbase + (size_t)tok * tokstride + j0 + 16 * jb + 4 * lg, one[0]);
                }
            }
        }
        {
            int br[NJ];
#pragma unroll
            for (int jb = 0; jb < NJ; ++jb) br[jb] = 16 * jb;
            const int Cb = wave;
            if constexpr (L::kF32) {
                // A operand Kb^T read from the token-major Kb
#pragma unroll 4
                for (int kk = 0; kk < C; kk += M::KS) {
                    const float a = M::frag_mc(sKb, L::P128, 16 * Cb, kk, lane);
#pragma unroll
                    for (int jb = 0; jb < NJ; ++jb)
                        acc_s[jb] = M::mma(a, M::frag_kc(sVN, L::P64, br[jb], kk, lane), acc_s[jb]);
                }
            } else {
                const int row = 16 * Cb + ln;
#pragma unroll
                for (int kk = 0; kk < C; kk += M::KS) {
                    const int blk = ((kk >> 3) + lg) ^ ((row >> 3) & 7);
                    const auto a = *reinterpret_cast<const bf16x8*>(sKbT + row * L::P64 + (blk << 3));
#pragma unroll
                    for (int jb = 0; jb < NJ; ++jb)
                        acc_s[jb] = M::mma(a, M::frag_kc(sVN, L::P64, br[jb], kk, lane), acc_s[jb]);
                }
            }
            const int c = 16 * Cb + 4 * lg;
#pragma unroll
            for (int jb = 0; jb < NJ; ++jb)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc_s[jb][e] *= s_gam[c + e];
        }
        // S^T for the next chunk: nobody reads S^T in this phase, and the next
        // chunk's first barrier orders these writes before its readers.
        write_state_lds();
    }

    if (!PREP && S_T) {
#pragma unroll
        for (int jb = 0; jb < NJ; ++jb) {
            const int c = 16 * wave + 4 * lg, j = j0 + 16 * jb + ln;
#pragma unroll
            for (int e = 0; e < 4; ++e) S_T[sbase + (size_t)(c + e) * DK + j] = acc_s[jb][e];
        }
    }
}


// ---- serial scan over chunks from the workspace (bf16) --------------------
// One workgroup per (head, value slice), 8 waves.  For every chunk it loads
// the key-side operands that chunk_fwd_kernel<.., PREP = true> exported (the
// slices of one head read the same bytes, shared through L2) and the V slice,
// and runs only the state-dependent products:
//   Z = V - Kh S;  Vn = Tm Diag(beta) Z;  O = Qt S + Aqk Vn;
//   S <- Diag(gamma) (S + Kb^T Vn).
// The next chunk's operands are fetched into registers while the current one
// is computed.
template <int DV>
struct ScanLayout {
    typedef bf16_t E;
    static constexpr int ES = 2, PAD = 8;
    static constexpr int P128 = DK + PAD, P64 = C + PAD, PV = DV + PAD;
    static constexpr int OFF_QT = 0;
    static constexpr int OFF_KH = OFF_QT + C * P128 * ES;
    static constexpr int OFF_KBT = OFF_KH + C * P128 * ES;
    static constexpr int OFF_TM = OFF_KBT + DK * P64 * ES;
    static constexpr int OFF_QK = OFF_TM + C * P64 * ES;
    static constexpr int OFF_V = OFF_QK + C * P64 * ES;
    static constexpr int OFF_ST = OFF_V + C * PV * ES;
    static constexpr int OFF_ZT = OFF_ST + DV * P128 * ES;
    static constexpr int OFF_VN = OFF_ZT + DV * P64 * ES;
    static constexpr int OFF_GAM = OFF_VN + DV * P64 * ES;
    static constexpr int TOTAL = OFF_GAM + DK * 4;
    static_assert(TOTAL <= 160 * 1024, "LDS budget");
    __device__ static constexpr int kbt(int c, int i) {
        return c * P64 + ((((i >> 3) ^ ((c >> 3) & 7)) << 3) | (i & 7));
    }
};

template <int DV>
__global__ void __launch_bounds__(NT)
chunk_scan_kernel(const char* ws, const bf16_t* v, const float* S0, bf16_t* o, float* S_T,
                  int T, int H, int nsplit)
{
    typedef bf16_t E;
    using L = ScanLayout<DV>;
    using M = Mma<E>;
    typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;
    constexpr int NJ = DV / 16;
    constexpr int VL = DV / 8;              // lanes per value row (16 bytes each)

    __shared__ __attribute__((aligned(16))) char smem[L::TOTAL];
    E* sQt = reinterpret_cast<E*>(smem + L::OFF_QT);
    E* sKh = reinterpret_cast<E*>(smem + L::OFF_KH);
    E* sKbT = reinterpret_cast<E*>(smem + L::OFF_KBT);
    E* sTM = reinterpret_cast<E*>(smem + L::OFF_TM);
    E* sQK = reinterpret_cast<E*>(smem + L::OFF_QK);
    E* sV = reinterpret_cast<E*>(smem + L::OFF_V);
    E* sST = reinterpret_cast<E*>(smem + L::OFF_ST);
    E* sZT = reinterpret_cast<E*>(smem + L::OFF_ZT);
    E* sVN = reinterpret_cast<E*>(smem + L::OFF_VN);
    float* s_gam = reinterpret_cast<float*>(smem + L::OFF_GAM);

    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int ln = lane & 15, lg = lane >> 4;
    const int nchunks = (T + C - 1) / C;
    const int nwg = gridDim.x, w = blockIdx.x;
    const int lid = (nwg % 8 == 0) ? (w % 8) * (nwg / 8) + w / 8 : w;
    const int head = lid / nsplit, slice = lid % nsplit;
    const int b = head / H, h = head % H;
    const int j0 = slice * DV;
    const size_t tokstride = (size_t)H * DK;
    const size_t hbase = ((size_t)b * T * H + h) * DK;
    const size_t sbase = (size_t)head * DK * DK;
    const char* wsh = ws + (size_t)head * nchunks * WS_CHUNK;
    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};

    // registers of one chunk: 8 x 16 bytes of the workspace block per thread
    // (the first 64 KiB), e^{G_64} (threads 0-31) and one value row segment
    struct Pre { i32x4 blk[8]; f32x4 gam; Raw8<E> v; };
    const int vg = t % VL, vr = t / VL;
    auto load = [&](int n, Pre& pr) {
        const char* src = wsh + (size_t)n * WS_CHUNK;
#pragma unroll
        for (int m = 0; m < 8; ++m) pr.blk[m] = reinterpret_cast<const i32x4*>(src)[t + NT * m];
        if (t < DK / 4) pr.gam = reinterpret_cast<const f32x4*>(src + WS_GAM)[t];
        if (vr < C) pr.v.load(v + hbase + (size_t)min(n * C + vr, T - 1) * tokstride + j0 + 8 * vg);
    };
    auto store = [&](int n, const Pre& pr) {
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const int u = t + NT * m;                       // 16-byte unit in the block
            i32x4* dst;
            if (m < 2) dst = reinterpret_cast<i32x4*>(sQt + (u >> 4) * L::P128 + 8 * (u & 15));
            else if (m < 4) { const int x = u - 1024; dst = reinterpret_cast<i32x4*>(sKh + (x >> 4) * L::P128 + 8 * (x & 15)); }
            else if (m < 6) { const int x = u - 2048; dst = reinterpret_cast<i32x4*>(sKbT + L::kbt(x >> 3, 8 * (x & 7))); }
            else if (m < 7) { const int x = u - 3072; dst = reinterpret_cast<i32x4*>(sTM + (x >> 3) * L::P64 + 8 * (x & 7)); }
            else { const int x = u - 3584; dst = reinterpret_cast<i32x4*>(sQK + (x >> 3) * L::P64 + 8 * (x & 7)); }
            *dst = pr.blk[m];
        }
        if (t < DK / 4) reinterpret_cast<f32x4*>(s_gam)[t] = pr.gam;
        if (vr < C) {
            const bool ok = n * C + vr < T;
            float row[8];
#pragma unroll
            for (int c = 0; c < 8; ++c) row[c] = ok ? pr.v[c] : 0.f;
            store8<E>(sV + vr * L::PV + 8 * vg, row);
        }
    };

    // state rows 16w .. 16w+15 of the slice in accumulators
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

    Pre pre;
    load(0, pre);
    for (int n = 0; n < nchunks; ++n) {
        store(n, pre);
        if (n + 1 < nchunks) load(n + 1, pre);
        lds_barrier();

        // ---- waves 0-3: Z = V - Kh S for token block R = wave | waves 4-7: Qt S
        f32x4 oacc[NJ];
        if (wave < 4) {
            const int R = wave;
            f32x4 pacc[NJ];
            int br[NJ];
#pragma unroll
            for (int jb = 0; jb < NJ; ++jb) { pacc[jb] = z4; br[jb] = 16 * jb; }
            mma_rows<E, DK, NJ>(pacc, sKh, L::P128, 16 * R, sST, L::P128, br, lane);
#pragma unroll
            for (int jb = 0; jb < NJ; ++jb) {
                const int j = 16 * jb + ln, r = 16 * R + 4 * lg;
                f32x4 vv;
#pragma unroll
                for (int e = 0; e < 4; ++e) vv[e] = (float)sV[(r + e) * L::PV + j];
                store_vec4<E>(sZT + j * L::P64 + r, vv - pacc[jb]);
            }
        } else {
            // output tiles (jb, R = wave - 4): A = S^T rows jb, B = Qt rows R
            const int R = wave - 4;
#pragma unroll
            for (int jb = 0; jb < NJ; ++jb) {
                f32x4 one[1] = {z4};
                const int br[1] = {16 * R};
                mma_rows<E, DK, 1>(one, sST, L::P128, 16 * jb, sQt, L::P128, br, lane);
                oacc[jb] = one[0];
            }
        }
        lds_barrier();

        // ---- Vn = Tm Diag(beta) Z: wave -> token block R = wave % 4, column blocks wave / 4 + 2u
        {
            constexpr int PER = (NJ + 1) / 2;
            const int R = wave % 4;
            if (wave / 4 < NJ) {
                f32x4 acc[PER];
                int br[PER];
#pragma unroll
                for (int u = 0; u < PER; ++u) {
                    acc[u] = z4;
                    const int jb = wave / 4 + 2 * u;
                    br[u] = 16 * (jb < NJ ? jb : 0);
                }
                mma_rows<E, C, PER>(acc, sTM, L::P64, 16 * R, sZT, L::P64, br, lane);
#pragma unroll
                for (int u = 0; u < PER; ++u) {
                    const int jb = wave / 4 + 2 * u;
                    if (jb < NJ) store_vec4<E>(sVN + (16 * jb + ln) * L::P64 + 16 * R + 4 * lg, acc[u]);
                }
            }
        }
        lds_barrier();

        // ---- O = Qt S + Aqk Vn (waves 4-7) | S <- Diag(gamma) (S + Kb^T Vn) (all)
        if (wave >= 4) {
            const int R = wave - 4;
            const int tok = n * C + 16 * R + ln;
#pragma unroll
            for (int jb = 0; jb < NJ; ++jb) {
                f32x4 one[1] = {oacc[jb]};
                const int br[1] = {16 * R};
                mma_rows<E, C, 1>(one, sVN, L::P64, 16 * jb, sQK, L::P64, br, lane);
                if (tok < T) store_vec4<E>(o + hbase + (size_t)tok * tokstride + j0 + 16 * jb + 4 * lg, one[0]);
            }
        }
        {
            int br[NJ];
#pragma unroll
            for (int jb = 0; jb < NJ; ++jb) br[jb] = 16 * jb;
            const int row = 16 * wave + ln;
#pragma unroll
            for (int kk = 0; kk < C; kk += M::KS) {
                const int blk = ((kk >> 3) + lg) ^ ((row >> 3) & 7);
                const auto a = *reinterpret_cast<const bf16x8*>(sKbT + row * L::P64 + (blk << 3));
#pragma unroll
                for (int jb = 0; jb < NJ; ++jb)
                    acc_s[jb] = M::mma(a, M::frag_kc(sVN, L::P64, br[jb], kk, lane), acc_s[jb]);
            }
            const int c = 16 * wave + 4 * lg;
#pragma unroll
            for (int jb = 0; jb < NJ; ++jb)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc_s[jb][e] *= s_gam[c + e];
        }
        lds_barrier();      // everyone is done with this chunk's operands and S^T
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
    hipLaunchKernelGGL((chunk_fwd_kernel<E, DV, false>), dim3(nwg), dim3(NT), 0, stream,
                       (const E*)q, (const E*)k, (const E*)v, g, (const E*)beta, S0, (E*)o, S_T,
                       T, H, nsplit, (char*)nullptr);
}

}  // namespace

size_t chunk_ws_bytes(long long B, long long T, long long H)
{
    return (size_t)B * (size_t)H * (size_t)((T + C - 1) / C) * (size_t)WS_CHUNK;
}

bool chunk_prefers_two_kernel(long long B, long long T, long long H, int dtype)
{
    // The fused kernel recomputes the key-side work once per value slice; with
    // fewer than 128 heads it needs 4 or 8 slices to fill the machine, and the
    // precomputed operands (about 1 KiB per token) cost less than the recompute.
    return dtype == 1 && B * H < 128 && T > C;
}

hipError_t launch_chunk_fwd(const void* q, const void* k, const void* v, const float* g,
                            const void* beta, const float* S0, void* o, float* S_T,
                            int B, int T, int H, int dtype, void* ws, hipStream_t stream)
{
    const long long heads = (long long)B * H;
    if (dtype == 0) {
        // fp32 operands need the narrowest slice to fit the LDS budget
        launch_one<float, 16>(q, k, v, g, beta, S0, o, S_T, B, T, H, stream);
    } else if (ws) {
        const int nchunks = (T + C - 1) / C;
        hipLaunchKernelGGL((chunk_fwd_kernel<bf16_t, 16, true>), dim3((unsigned)(heads * nchunks)), dim3(NT),
                           0, stream, (const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v, g,
                           (const bf16_t*)beta, S0, (bf16_t*)o, S_T, T, H, 1, (char*)ws);
        // value slices: enough workgroups to cover the machine
        const int dv = heads * 2 >= 256 ? 64 : (heads * 4 >= 256 ? 32 : 16);
        const int nsplit = DK / dv;
        const dim3 grid((unsigned)(heads * nsplit));
        if (dv == 64)
            hipLaunchKernelGGL(chunk_scan_kernel<64>, grid, dim3(NT), 0, stream, (const char*)ws,
                               (const bf16_t*)v, S0, (bf16_t*)o, S_T, T, H, nsplit);
        else if (dv == 32)
            hipLaunchKernelGGL(chunk_scan_kernel<32>, grid, dim3(NT), 0, stream, (const char*)ws,
                               (const bf16_t*)v, S0, (bf16_t*)o, S_T, T, H, nsplit);
        else
            hipLaunchKernelGGL(chunk_scan_kernel<16>, grid, dim3(NT), 0, stream, (const char*)ws,
                               (const bf16_t*)v, S0, (bf16_t*)o, S_T, T, H, nsplit);
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
