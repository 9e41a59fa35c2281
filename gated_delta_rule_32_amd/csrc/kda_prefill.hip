// kda_prefill.hip -- chunkwise KDA prefill for gfx950 (one fused kernel).
//
// Method: page "Kimi Linear：高效注意力机制在长序列处理中的创新应用", sections
// 2.1-2.3 (Proposition S_r = P_r S_0 + H_r, WY representation, chunks of 64,
// forward substitution) and page "Kimi K3论文：Kimi Linear", section 4 (intra-
// chunk matrix products, UT transform, chunk-to-chunk state recurrence).
// For a chunk of C = 64 tokens with entry state S (d_k x d_v, fp32), and
// G = in-chunk cumulative sum of g = log(alpha):
//
//   Qt = e^{G} * Q,  Kh = e^{G} * K,  Kt = e^{G_64 - G} * K             [64 x 128]
//   Aqk[r,i] = sum_c q_r[c] k_i[c] e^{G_r[c] - G_i[c]}   (kept for i <= r) [64 x 64]
//   Akk[r,i] = beta_r sum_c k_r[c] k_i[c] e^{G_r[c] - G_i[c]}   (kept for i < r)
//   Tm  = (I + Akk)^{-1}                         (UT transform)
//   Vn  = Tm Diag(beta) (V - Kh S)               (= U - W S with the WY factors
//                                                  W = Tm Diag(beta) Kh, U = Tm Diag(beta) V)
//   O   = Qt S + Aqk Vn
//   S  <- Diag(e^{G_64}) S + Kt^T Vn
//
// Aqk and Akk are products of decay-scaled operands: the decay e^{G_r - G_i}
// is split at a reference point into a row factor and a column factor.  A
// chunk whose decay stays in range (every channel's G_64 above -FAST_LIM in
// log2 units) takes the chunk start: Aqk = Qt Kb^T, Akk = Diag(beta) Kh Kb^T
// with Kb = e^{-G} * K.  Any other chunk takes the ends of its four 16-token
// sub-chunks (the secondary chunking of page "Kimi K3论文：Kimi Linear",
// section 4): its 16 x 16 blocks are products of operands referenced to the
// end of their own sub-chunk, the blocks below the diagonal scaled by the
// decay between the two sub-chunk ends (m1_subchunk), so that no factor grows
// with the chunk's total decay; only each sub-chunk's decay must stay in fp32
// range.  Kt, the state update's operand, is bounded by one on both paths.
// The WY factor W is never formed: Tm is applied to the residual V - Kh S
// instead, which is the same product reassociated and saves one 64x64x128
// product and its buffer.
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

#include <algorithm>
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
    static constexpr int OFF_KBT = OFF_KB + SZ_TOK;                   // Kt^T (bf16 only)
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
    static constexpr int OFF_GTOT = OFF_TOT + NW * DK * 4;           // G_64 per channel (log2)
    static constexpr int TOTAL = OFF_GTOT + DK * 4;
    static_assert(TOTAL <= 160 * 1024, "LDS budget");
    static_assert(!kF32 || P64 == PA, "fp32 Tm aliases Akk");
    // Kt^T (channel-major, 64 tokens per row) is stored with its 8-token
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
    Raw8f g[RPL];                                       // per-channel gate
    float gh[RPL];                                      // per-head gate
    Raw8<E> q[RPL], k[RPL];
    Raw8<E> v[RVR];
    E beta;
};

constexpr int PREP_CHUNKS = 4;                      // chunks per prep workgroup

// Largest log2-decay magnitude over one chunk (per channel) for which the
// chunk-start factorisation 2^{G_r} 2^{-G_i} keeps every factor a normal
// number with room to spare (fp32 and bf16 share the 8-bit exponent).
constexpr float FAST_LIM = 96.f;

// Intra-chunk matrices of a chunk whose decay exceeds the fast path's range
// (secondary chunking; page "Kimi K3论文：Kimi Linear", section 4, on chunking
// below the chunk because of the cumulative decay's reciprocal).  On entry the
// LDS holds, for row r of sub-chunk s = r / 16 with B_{s+1} the cumulative
// log2-decay at the end of that sub-chunk (prefix totals in s_tot, G_64 in
// s_gtot):
//   Qt = 2^{G_r - B_{s+1}} q_r, Kh = 2^{G_r - B_{s+1}} k_r   (>= 1, bounded by
//   the sub-chunk's decay),  Kb = 2^{B_{s+1} - G_r} k_r   (<= 1).
// Tile (I, R), R >= I, of Aqk^T / Akk^T takes A = Kb rows of block I and B =
// the Qt / Kh rows of block R; their product carries 2^{G_r - G_i} times
// 2^{B_{I+1} - B_{R+1}}, so for R > I the B fragment is scaled by
// F = 2^{B_{R+1} - B_{I+1}} (<= 1, per channel) first: every operand then
// stays at or below one off the diagonal, and the diagonal tiles need no
// factor.  The tiles are written as the fast path writes them (Akk in RA with
// beta, Aqk in sQK, the transposed diagonal Akk blocks in sDT, zero upper
// tiles).  Then Qt and Kh are rebased to the chunk start (times 2^{B_{s+1}} <=
// 1), and for fp32, which keeps no Kt^T tile, Kb becomes Kt = 2^{G_64 - G_r}
// k_r.
template <typename E, int DV>
__device__ __forceinline__ void m1_subchunk(char* smem, int t)
{
    using L = Layout<E, DV>;
    using M = Mma<E>;
    const int lane = t & 63, wave = t >> 6, ln = lane & 15, lg = lane >> 4;
    E* sQt = reinterpret_cast<E*>(smem + L::OFF_QT);
    E* sKh = reinterpret_cast<E*>(smem + L::OFF_KH);
    E* sKb = reinterpret_cast<E*>(smem + L::OFF_KB);
    float* RA = reinterpret_cast<float*>(smem + L::OFF_RA);
    float* sDT = reinterpret_cast<float*>(smem + L::OFF_RT);
    E* sQK = reinterpret_cast<E*>(smem + L::OFF_QK);
    const float* s_beta = reinterpret_cast<const float*>(smem + L::OFF_BETA);
    const float* s_tot = reinterpret_cast<const float*>(smem + L::OFF_TOT);
    const float* s_gtot = reinterpret_cast<const float*>(smem + L::OFF_GTOT);
    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
    auto bnd_of = [&](int j, int c) { return j < 4 ? s_tot[2 * j * DK + c] : s_gtot[c]; };   // B_j, j = 1..4
    // 20 product tiles (10 of Aqk, 10 of Akk) and 6 zero upper tiles over the 8 waves
#pragma unroll 1
    for (int u = wave; u < 26; u += NW) {
        if (u < 20) {
            const bool kk = u >= 10;
            const int v10 = u % 10;   // (I, R): (0,0..3), (1,1..3), (2,2..3), (3,3)
            const int I = v10 < 4 ? 0 : (v10 < 7 ? 1 : (v10 < 9 ? 2 : 3));
            const int R = I + (v10 < 4 ? v10 : (v10 < 7 ? v10 - 4 : (v10 < 9 ? v10 - 7 : 0)));
            const E* Bm = kk ? sKh : sQt;
            f32x4 acc = z4;
#pragma unroll 1
            for (int k0 = 0; k0 < DK; k0 += M::KS) {
                const auto fa = M::frag_kc(sKb, L::P128, 16 * I, k0, lane);
                auto fb = M::frag_kc(Bm, L::P128, 16 * R, k0, lane);
                if (R > I) {
                    if constexpr (L::kF32) {
                        const int c = k0 + (lane >> 4);
                        fb *= __builtin_amdgcn_exp2f(bnd_of(R + 1, c) - bnd_of(I + 1, c));
                    } else {
                        const int c0 = k0 + 8 * (lane >> 4);
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            fb[e] = (bf16_t)((float)fb[e] *
                                             __builtin_amdgcn_exp2f(bnd_of(R + 1, c0 + e) - bnd_of(I + 1, c0 + e)));
                    }
                }
                acc = M::mma(fa, fb, acc);
            }
            // epilogue: mask, beta of the row for Akk, store (as the fast path)
            const int r = 16 * R + ln, i0 = 16 * I + 4 * lg;
            f32x4 val;
            const float bt = kk ? s_beta[r] : 1.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) val[e] = (kk ? (i0 + e < r) : (i0 + e <= r)) ? bt * acc[e] : 0.f;
            if (kk) *reinterpret_cast<f32x4*>(RA + r * L::PA + i0) = val;
            else store_vec4<E>(sQK + r * L::P64 + i0, val);
            if constexpr (!L::kF32) {
                if (kk && I == R) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) sDT[(16 * R + 4 * lg + e) * L::PDT + ln] = val[e];
                }
            }
        } else {
            const int v6 = u - 20;
            const int I = v6 < 3 ? v6 + 1 : (v6 < 5 ? v6 - 1 : 3);
            const int R = v6 < 3 ? 0 : (v6 < 5 ? 1 : 2);
            const int r = 16 * R + ln, i0 = 16 * I + 4 * lg;
            if constexpr (L::kF32) *reinterpret_cast<f32x4*>(RA + r * L::PA + i0) = z4;
            store_vec4<E>(sQK + r * L::P64 + i0, z4);
        }
    }
    lds_barrier();
    // rebase: Qt, Kh times 2^{B_{s+1}}; fp32 Kb times 2^{G_64 - B_{s+1}}
    constexpr int NTILE = L::kF32 ? 3 : 2;
#pragma unroll 1
    for (int gi = t; gi < NTILE * C * 16; gi += NT) {
        const int tile = gi / (C * 16), r = (gi / 16) % C, c0 = 8 * (gi % 16);
        E* row = (tile == 0 ? sQt : tile == 1 ? sKh : sKb) + r * L::P128 + c0;
        const int s = r >> 4;
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float bs = bnd_of(s + 1, c0 + e);
            x[e] = to_f32(row[e]) * __builtin_amdgcn_exp2f(tile < 2 ? bs : s_gtot[c0 + e] - bs);
        }
        store8<E>(row, x);
    }
    lds_barrier();
}

// The fused kernel (PREP = false): one workgroup per (head, value slice)
// walks all chunks of its head.  The prep instantiation (PREP = true): one
// workgroup per (head, chunk) runs only the key-side work -- decay, Aqk, Akk,
// Tm -- and exports it to the workspace for chunk_scan_kernel; with BWD it
// also exports to `wsb` the operands of the backward state scan (the
// transposes Aqk^T, Tm^T, Qt^T, Kh^T and Kt = e^{G_64 - G} k, layout
// WSB_* in kda_chunk_common.h).
//
// With cu_seqlens (fused kernel only), batch index b is a sequence packed
// along one token axis of T tokens: tokens cu_seqlens[b] .. cu_seqlens[b+1]
// (clamped to [0, T]), chunked from its own first token.
//
// GATE selects the forget gate: GATE_CHANNEL (KDA, g [B, T, H, 128]),
// GATE_HEAD (one decay per head and token, g [B, T, H]: Gated DeltaNet) or
// GATE_NONE (alpha = 1: DeltaNet, g unused).  With one decay per row the
// decay factors are computed once per row instead of once per channel.
//
// The body runs on LDS `smem` for the work item `lid` (a (head, slice) or
// (head, chunk group) index); with `flags` (prep only, the pipelined
// schedule) each exported block is followed by a ready flag, see
// chunk_pipe_kernel.
template <typename E, int DV, bool PREP, bool BWD = false, int GATE = GATE_CHANNEL>
__device__ __forceinline__ void
chunk_fwd_body(const E* q, const E* k, const E* v, const float* g, const E* beta,
               const float* S0, E* o, float* S_T, int T_axis, int H, int nsplit, char* ws,
               char* wsb, const int* cu_seqlens, char* smem, const int lid, int* flags)
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
    float* s_gtot = reinterpret_cast<float*>(smem + L::OFF_GTOT);
    // prep for the backward pass: Tm^T, unscaled, in the (unused) value-side
    // buffers; null otherwise
    static_assert(!BWD || (PREP && L::OFF_VN - L::OFF_V >= C * TMT_P * 2 && L::P64 == TMT_P),
                  "Tm^T fits in the value-side buffers");
    bf16_t* sTmT = BWD ? reinterpret_cast<bf16_t*>(smem + L::OFF_V) : nullptr;

    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);   // uniform per wave
    const int cg = lane & 15, rq = lane >> 4;   // 8-channel group and row quad for q/k/g
    const int vg = t % In::VL, vr = t / In::VL; // 8-channel group and row group for v
    const int ln = lane & 15, lg = lane >> 4;

    const int nblk = ((T_axis + C - 1) / C + PREP_CHUNKS - 1) / PREP_CHUNKS;   // prep: chunk groups per head
    const int head = PREP ? lid / nblk : lid / nsplit;
    const int slice = PREP ? 0 : lid % nsplit;
    const int b = head / H, h = head % H;
    const int j0 = slice * DV;
    // this head's tokens: T of them from token index seq0 of the token axis
    size_t seq0 = (size_t)b * T_axis;
    int T = T_axis;
    if (!PREP && cu_seqlens) {
        const int s0 = min(max(cu_seqlens[b], 0), T_axis);
        const int s1 = min(max(cu_seqlens[b + 1], s0), T_axis);
        seq0 = (size_t)s0;
        T = s1 - s0;
    }
    const int nchunks = (T + C - 1) / C;
    const int n_first = PREP ? (lid % nblk) * PREP_CHUNKS : 0;
    const int n_end = PREP ? min(n_first + PREP_CHUNKS, nchunks) : nchunks;

    const size_t tokstride = (size_t)H * DK;                       // one token, all heads
    const size_t hbase = (seq0 * H + h) * DK;                      // (b, t=0, h, 0)
    const size_t sbase = (size_t)head * DK * DK;                   // state of this head

    // Prefetch of one chunk into registers.  Branch-free: rows past T read the
    // last valid token (always in bounds) and are zeroed when consumed, so no
    // load result is needed before the next chunk starts.
    const E* betap = beta + seq0 * H + h;
    auto load_chunk = [&](int n, In& in) {
        const int tok0 = n * C;
#pragma unroll
        for (int i = 0; i < RPL; ++i) {
            const int tok = min(tok0 + RPT * wave + RPL * rq + i, T - 1);
            const size_t off = hbase + (size_t)tok * tokstride + 8 * cg;
            if constexpr (GATE == GATE_CHANNEL) in.g[i].load(g + off);
            else if constexpr (GATE == GATE_HEAD) in.gh[i] = g[(seq0 + tok) * H + h];
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
    if (n_first < n_end) load_chunk(n_first, in);   // (an empty sequence has no tokens to read)
    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};

    for (int n = n_first; n < n_end; ++n) {
        const bool full = (n + 1) * C <= T;     // uniform: no row of this chunk is past T

        // PREP: this chunk's operand block.  Its units are gathered from the
        // padded LDS rows, two 8-byte halves per 16-byte unit.  Qt, Kh and
        // Kt^T (not Qt for the backward pass, whose save-mode scan does not
        // read it) are exported by threads u0, u0 + du, ...
        char* blk = PREP ? ws + ((size_t)head * nchunks + n) * WSK_CHUNK : nullptr;
        typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;
        typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2;
        auto put = [&](int dst, const E* lo, const E* hi) {
            const i32x2 a = *reinterpret_cast<const i32x2*>(lo), c2 = *reinterpret_cast<const i32x2*>(hi);
            *reinterpret_cast<i32x4*>(blk + dst) = i32x4{a[0], a[1], c2[0], c2[1]};
        };
        auto export_tok = [&](int u0, int du) {
            // Qt, Kh: 64 rows of 16 units; unit u = 4p + lg of row r
            for (int u = (BWD ? C * 16 : 0) + u0; u < 2 * C * 16; u += du) {
                const int mat = u / (C * 16), r = (u >> 4) & (C - 1), uu = u & 15;
                const E* row = (mat ? sKh : sQt) + r * L::P128 + 32 * (uu >> 2) + 4 * (uu & 3);
                put((mat ? WSK_KH : WSK_QT) + 2 * wsk_tok_unit(r, uu), row, row + 16);
            }
            // Kt^T: 128 rows of 8 units (tokens from the swizzled LDS tile)
            for (int u = u0; u < DK * 8; u += du) {
                const int c = u >> 3, uu = u & 7, i0 = 32 * (uu >> 2) + 4 * (uu & 3);
                put(WSK_KBT + 2 * wsk_kbt_unit(c, uu), sKbT + L::kbt(c, i0), sKbT + L::kbt(c, i0 + 16));
            }
        };

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
            constexpr int NG = GATE == GATE_CHANNEL ? 8 : 1;   // distinct decays per lane row
            float G[RPL][NG];
#pragma unroll
            for (int c = 0; c < NG; ++c) {
                if constexpr (GATE == GATE_NONE) {
#pragma unroll
                    for (int i = 0; i < RPL; ++i) G[i][c] = 0.f;
                    if (rq == 3) {
#pragma unroll
                        for (int c2 = 0; c2 < 8; ++c2) s_tot[wave * DK + 8 * cg + c2] = 0.f;
                    }
                    continue;
                }
                float run = 0.f;
#pragma unroll
                for (int i = 0; i < RPL; ++i) {
                    const float gi = (GATE == GATE_CHANNEL ? in.g[i][c] : in.gh[i]) * LOG2E;
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
                if (rq == 3) {
                    if constexpr (NG == 8) s_tot[wave * DK + 8 * cg + c] = inc;
                    else {
#pragma unroll
                        for (int c2 = 0; c2 < 8; ++c2) s_tot[wave * DK + 8 * cg + c2] = inc;
                    }
                }
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
                s_gtot[t] = acc;
            }
            lds_barrier();
            // Decay range of this chunk (the same verdict in every wave).
            // While every channel's log2-decay over the chunk stays above
            // -FAST_LIM, the row and column factors 2^{G} and 2^{-G} referenced
            // to the chunk start are normal fp32 / bf16 numbers and the chunk
            // takes the fast path.  Otherwise its intra-chunk products are
            // referenced to the ends of the four 16-token sub-chunks (slow
            // path below), which needs only each sub-chunk's decay in range.
            bool slow_chunk = false;
            if constexpr (GATE != GATE_NONE) {
                const float ga = s_gtot[lane], gb = s_gtot[lane + 64];   // both read, no branch
                slow_chunk = __builtin_amdgcn_ballot_w64((ga < -FAST_LIM) | (gb < -FAST_LIM)) != 0;
            }
            {
                if constexpr (NG == 8) {
                    const f32x4 o0 = *reinterpret_cast<const f32x4*>(s_tot + wave * DK + 8 * cg);
                    const f32x4 o1 = *reinterpret_cast<const f32x4*>(s_tot + wave * DK + 8 * cg + 4);
#pragma unroll
                    for (int i = 0; i < RPL; ++i)
#pragma unroll
                        for (int c = 0; c < 4; ++c) { G[i][c] += o0[c]; G[i][c + 4] += o1[c]; }
                } else if constexpr (GATE == GATE_HEAD) {
                    const float o = s_tot[wave * DK + 8 * cg];
#pragma unroll
                    for (int i = 0; i < RPL; ++i) G[i][0] += o;
                }
            }
            // Operands, per row r and channel c, from factors a, b, c':
            //   Qt = a q, Kh = a k, Kb = b k, Kt = c' k  (Kt^T is the bf16 Kb^T tile)
            // with a = 2^{G_r - ref}, b = 2^{ref - G_r}, c' = 2^{G_64 - G_r}
            // = 2^{G_64 - ref} b.  Fast path: ref = 0 (the chunk start).  Slow
            // path: ref = B_{s+1}, the end of the row's sub-chunk s = r / 16
            // (a >= 1 and b <= 1 within the sub-chunk); its Qt and Kh are
            // rebased to the chunk start after the intra-chunk products, and Kt
            // is the same on both paths.  Both paths run the same code on G
            // shifted by ref.
            float mult[8];                       // 2^{G_64 - ref} per channel
            if (slow_chunk) {
                // sub-chunk s = wave / 2 (16 rows = two waves): its end is the
                // exclusive prefix at wave 2s + 2, or G_64 for the last one
                const float* bsrc = (wave >> 1) < 3 ? s_tot + ((wave >> 1) * 2 + 2) * DK + 8 * cg : s_gtot + 8 * cg;
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    const float ref = bsrc[c];
                    mult[c] = __builtin_amdgcn_exp2f(s_gtot[8 * cg + c] - ref);
                    if (c < NG) {
#pragma unroll
                        for (int i = 0; i < RPL; ++i) G[i][c] -= ref;
                    }
                }
            } else {
#pragma unroll
                for (int c = 0; c < 8; ++c) mult[c] = s_gam[8 * cg + c];
            }
            float kt[RPL][8];
#pragma unroll
            for (int i = 0; i < RPL; ++i) {
                const int r = r0 + i;
                const bool ok = row_ok(r);
                float qe[8], ke[8], kb[8], fa[NG], fb[NG];
#pragma unroll
                for (int c = 0; c < NG; ++c) {
                    fa[c] = GATE == GATE_NONE ? 1.f : __builtin_amdgcn_exp2f(G[i][c]);
                    fb[c] = GATE == GATE_NONE ? 1.f : __builtin_amdgcn_exp2f(-G[i][c]);
                }
#pragma unroll
                for (int c = 0; c < 8; ++c) kt[i][c] = mult[c] * fb[NG == 8 ? c : 0];
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    const float e = fa[NG == 8 ? c : 0], ne = fb[NG == 8 ? c : 0];
                    const float qv = ok ? in.q[i][c] : 0.f, kv = ok ? in.k[i][c] : 0.f;
                    qe[c] = qv * e; ke[c] = kv * e; kb[c] = kv * ne; kt[i][c] *= kv;
                }
                store8<E>(sQt + r * L::P128 + 8 * cg, qe);
                store8<E>(sKh + r * L::P128 + 8 * cg, ke);
                store8<E>(sKb + r * L::P128 + 8 * cg, kb);
            }
            if constexpr (!L::kF32) {
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    float col[RPL];
#pragma unroll
                    for (int i = 0; i < RPL; ++i) col[i] = kt[i][c];
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
            return slow_chunk;
        };
        const bool slow = full ? ephase(std::false_type{}) : ephase(std::true_type{});
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
            if (!slow) {
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
                } else if (wave == 2) {   // I = 1: Aqk R = 3, Akk R = 1..3;  I = 3: Akk R = 3
                    f32x4 acc[4] = {z4, z4, z4, z4};
                    const int br[4] = {48, 80, 96, 112};
                    mma_rows<E, DK, 4>(acc, sKb, L::P128, 16, sQt, L::P128, br, lane);
                    f32x4 acc3[1] = {z4};
                    const int br3[1] = {112};
                    mma_rows<E, DK, 1>(acc3, sKb, L::P128, 48, sQt, L::P128, br3, lane);
                    epilogue(acc[0], 1, 3, false);
    #pragma unroll
                    for (int R = 1; R < 4; ++R) epilogue(acc[R], 1, R, true);
                    epilogue(acc3[0], 3, 3, true);
                } else if (wave == 3) {   // I = 2 for both, I = 3: Aqk R = 3, and the zero upper tiles
                    f32x4 acc[4] = {z4, z4, z4, z4};
                    const int br[4] = {32, 48, 96, 112};
                    mma_rows<E, DK, 4>(acc, sKb, L::P128, 32, sQt, L::P128, br, lane);
                    f32x4 acc3[1] = {z4};
                    const int br3[1] = {48};
                    mma_rows<E, DK, 1>(acc3, sKb, L::P128, 48, sQt, L::P128, br3, lane);
                    epilogue(acc[0], 2, 2, false); epilogue(acc[1], 2, 3, false);
                    epilogue(acc[2], 2, 2, true); epilogue(acc[3], 2, 3, true);
                    epilogue(acc3[0], 3, 3, false);
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
                if (!PREP && wave >= 4) p_block(wave - 4);
                // prep: Qt, Kh and Kt^T are final after E on this path; the
                // waves without tiles export them while the tiles are formed
                if (PREP && wave >= 4) export_tok(t - 256, NT - 256);
            } else {
                m1_subchunk<E, DV>(smem, t);
                if (!PREP && wave >= 4) p_block(wave - 4);
            }
        }
        lds_barrier();

        // ===== UT diagonal blocks (wave 0) | inter-chunk output Qt S (waves 1-7;
        // backward prep: the transposed operands of the backward state scan) =====
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
        } else if constexpr (PREP && BWD) {
            // Aqk^T, Qt^T, Kh^T and Kt (final since the intra-chunk products)
            // for the backward state scan, by the seven waves that have no
            // substitution chain, transposed 16 x 16 blocks at a time on the
            // matrix cores: the A operand is 16 rows of the source (4
            // consecutive columns per lane, one 8-byte LDS read), B the
            // identity, so accumulator lane (ln, lg) holds source rows 4lg ..
            // 4lg+3 of column ln, i.e. 4 consecutive elements of row ln of the
            // transpose (bf16 times one, summed in fp32: exact).
            char* bb = wsb + ((size_t)head * nchunks + n) * WSB_CHUNK;
            bf16x4 ident;
#pragma unroll
            for (int e = 0; e < 4; ++e) ident[e] = (bf16_t)(4 * lg + e == ln ? 1.f : 0.f);
            // Blocks 0-31 Qt^T, 32-63 Kh^T ([128][64] from [64][128]), 64-95
            // Kt ([64][128] from the swizzled Kt^T tile, 4 consecutive tokens
            // contiguous), 96-105 the nonzero blocks of Aqk^T.  A lane's four
            // elements (row `row`, columns 32p + 16h + 4lg .. +3) are half h
            // of unit 4p + lg of that row in the block's layout.
            for (int bk = wave - 1; bk < 106; bk += NW - 1) {
                const int m = bk >> 5, b5 = bk & 31;
                int r0 = 16 * (b5 & 3), c0 = 16 * (b5 >> 2);
                if (m == 3) {                 // upper block (Ib, Rr), Rr >= Ib, of Aqk^T
                    const int Ib = b5 < 4 ? 0 : b5 < 7 ? 1 : b5 < 9 ? 2 : 3;
                    const int Rr = Ib + b5 - (Ib == 0 ? 0 : Ib == 1 ? 4 : Ib == 2 ? 7 : 9);
                    r0 = 16 * Rr; c0 = 16 * Ib;   // Aqk rows r0.., columns c0..
                }
                bf16x4 a;
                if (m < 2) a = *reinterpret_cast<const bf16x4*>((m ? sKh : sQt) + (r0 + ln) * L::P128 + c0 + 4 * lg);
                else if (m == 2) a = *reinterpret_cast<const bf16x4*>(sKbT + L::kbt(c0 + ln, r0 + 4 * lg));
                else a = *reinterpret_cast<const bf16x4*>(sQK + (r0 + ln) * L::P64 + c0 + 4 * lg);
                const bf16x4 d = to_bf16x4(__builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, ident, z4, 0, 0, 0));
                // transpose row, and its columns' pair p and half h
                const int row = (m == 2 ? r0 : c0) + ln, cc = m == 2 ? c0 : r0, p = cc >> 5, h = (cc >> 4) & 1;
                size_t off;
                if (m < 2) off = (m ? WSB_KHT : WSB_QTT) + 2 * wsk_kbt_unit(row, 4 * p + lg) + 8 * h;
                else if (m == 2) off = WSB_KT + 2 * wsk_tok_unit(row, 4 * p + lg) + 8 * h;
                else {
                    const int Ib = c0 >> 4;
                    off = WSB_AQKT + wsb_pair_off(Ib, p) +
                          (wsb_pair_full(Ib, p) ? 16 * (4 * ln + lg) + 8 * h : 8 * (4 * ln + lg));
                }
                *reinterpret_cast<bf16x4*>(bb + off) = d;
            }
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
        if (wave >= 3 && n + 1 < n_end) load_chunk(n + 1, in);

        // ===== UT off-diagonal blocks; Tm Diag(beta) in E =====
        if constexpr (!L::kF32) {
            if (wave == 0) ut_offdiag_column<0, L::PA, L::P64>(RA, RT, s_beta, lane, sTmT);
            else if (wave == 1) ut_offdiag_column<1, L::PA, L::P64>(RA, RT, s_beta, lane, sTmT);
            else if (wave == 2) ut_offdiag_column<2, L::PA, L::P64>(RA, RT, s_beta, lane, sTmT);
            else if (wave == 3) {
                // diagonal blocks, scaled by beta of their column
#pragma unroll
                for (int bb = 0; bb < 4; ++bb) {
                    const int r = 16 * bb + 4 * lg;
                    const float bcol = s_beta[16 * bb + ln];
                    f32x4 x;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        x[e] = RA[(r + e) * L::PA + 16 * bb + ln];
                        RT[(r + e) * L::P64 + 16 * bb + ln] = (E)(bcol * x[e]);
                    }
                    if (sTmT) store_vec4<bf16_t>(sTmT + (16 * bb + ln) * TMT_P + r, x);
                }
            } else {
                for (int u = wave - 4; u < 6; u += 4) {   // zero upper blocks of RT (lower of Tm^T)
                    const int I = u < 3 ? u + 1 : (u < 5 ? u - 1 : 3);
                    const int R = u < 3 ? 0 : (u < 5 ? 1 : 2);
                    store_vec4<E>(RT + (16 * R + ln) * L::P64 + 16 * I + 4 * lg, z4);
                    if (sTmT) store_vec4<bf16_t>(sTmT + (16 * I + ln) * TMT_P + 16 * R + 4 * lg, z4);
                }
            }
            if (wave < 3 && n + 1 < n_end) load_chunk(n + 1, in);
            lds_barrier();
        } else {
            if (wave < 3 && n + 1 < n_end) load_chunk(n + 1, in);
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
            // ===== export the rest of this chunk's operand block =====
            // (Qt, Kh and Kt^T here only on the sub-chunk path, which rebases
            // Qt and Kh after the intra-chunk products)
            if (slow) export_tok(t, NT);
            if (t < DK / 4)
                reinterpret_cast<f32x4*>(blk + WSK_GAM)[t] = reinterpret_cast<const f32x4*>(s_gam)[t];
            // Tm Diag(beta) and (not for the backward pass) Aqk: six operand
            // pairs of 64 units each (8-byte units for the two half pairs)
            for (int u = t; u < (BWD ? 1 : 2) * 6 * 64; u += NT) {
                const int mat = u / (6 * 64), k6 = (u >> 6) % 6, l = u & 63;
                const int Rb = k6 < 1 ? 0 : k6 < 2 ? 1 : k6 < 4 ? 2 : 3, pp = (k6 == 3 || k6 == 5) ? 1 : 0;
                const E* row = (mat ? sQK : RT) + (16 * Rb + (l >> 2)) * L::P64 + 32 * pp + 4 * (l & 3);
                const int off = (mat ? WSK_QK : WSK_TM) + wsk_pair_off(Rb, pp);
                if (wsk_pair_full(Rb, pp)) put(off + 16 * l, row, row + 16);
                else *reinterpret_cast<i32x2*>(blk + off + 8 * l) = *reinterpret_cast<const i32x2*>(row);
            }
            if constexpr (BWD) {
                // the rest of the backward state scan's operands (Aqk^T, Qt^T,
                // Kh^T and Kt went out during the diagonal UT step)
                char* bb = wsb + ((size_t)head * nchunks + n) * WSB_CHUNK;
                // Tm^T as the operand pairs of its nonzero blocks: 4 full pairs
                // of 64 units, then the two half pairs (second block only)
                for (int u = t; u < 6 * 64; u += NT) {
                    const int k6 = u >> 6, l = u & 63;
                    const int Rb = k6 < 2 ? 0 : k6 < 4 ? 1 : k6 < 5 ? 2 : 3, p = (k6 == 0 || k6 == 2) ? 0 : 1;
                    const bf16_t* row = sTmT + (16 * Rb + (l >> 2)) * TMT_P + 32 * p + 4 * (l & 3);
                    const int off = WSB_TMT + wsb_pair_off(Rb, p);
                    const i32x2 hi = *reinterpret_cast<const i32x2*>(row + 16);
                    if (wsb_pair_full(Rb, p)) {
                        const i32x2 lo = *reinterpret_cast<const i32x2*>(row);
                        *reinterpret_cast<i32x4*>(bb + off + 16 * l) = i32x4{lo[0], lo[1], hi[0], hi[1]};
                    } else {
                        *reinterpret_cast<i32x2*>(bb + off + 8 * l) = hi;
                    }
                }
                if (t < DK) reinterpret_cast<float*>(bb + WSB_GAM)[t] = s_gam[t];
                if (t < C) reinterpret_cast<float*>(bb + WSB_BETA)[t] = s_beta[t];
                // the next chunk's first LDS writes (beta, column totals) come
                // before its first barrier
                lds_barrier();
            }
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
        // waves) | S <- Diag(gamma) S + Kt^T Vn =====
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
            const int c = 16 * Cb + 4 * lg;
            // S <- Diag(gamma) S + Kt^T Vn, Kt = 2^{G_64 - G} k (bf16: the Kb^T
            // tile holds Kt^T; fp32: Kb holds Kt on the slow path, while the
            // fast path keeps Kb = 2^{-G} k and applies gamma after the sum)
            const bool gamma_first = !L::kF32 || slow;
            if (gamma_first) {
#pragma unroll
                for (int jb = 0; jb < NJ; ++jb)
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc_s[jb][e] *= s_gam[c + e];
            }
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
            if (!gamma_first) {
#pragma unroll
                for (int jb = 0; jb < NJ; ++jb)
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc_s[jb][e] *= s_gam[c + e];
            }
        }
        // S^T for the next chunk: nobody reads S^T in this phase, and the next
        // chunk's first barrier orders these writes before its readers.
        write_state_lds();
    }

    if (PREP && !BWD && flags && n_first < n_end) {
        // the blocks of this work item complete in L2 (every store is
        // acknowledged there), then their ready flags: one wait per item,
        // not per chunk.  The reader sits on the same XCD, so that L2 is
        // where it looks.
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        lds_barrier();
        if (t < n_end - n_first)
            __hip_atomic_store(flags + (size_t)head * nchunks + n_first + t, 1, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
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


template <typename E, int DV, bool PREP, bool BWD = false, int GATE = GATE_CHANNEL>
__global__ void __launch_bounds__(NT)
chunk_fwd_kernel(const E* q, const E* k, const E* v, const float* g, const E* beta,
                 const float* S0, E* o, float* S_T, int T_axis, int H, int nsplit, char* ws,
                 char* wsb, const int* cu_seqlens)
{
    __shared__ __attribute__((aligned(16))) char smem[Layout<E, DV>::TOTAL];
    // Workgroup -> (head, slice), keeping the slices of a head on one XCD
    // (workgroups are dealt to the 8 XCDs round-robin); prep: (head, chunk group).
    const int nwg = gridDim.x, w = blockIdx.x;
    const int lid = (!PREP && nwg % 8 == 0) ? (w % 8) * (nwg / 8) + w / 8 : w;
    chunk_fwd_body<E, DV, PREP, BWD, GATE>(q, k, v, g, beta, S0, o, S_T, T_axis, H, nsplit, ws, wsb,
                                           cu_seqlens, smem, lid, nullptr);
}

// ---- serial scan over chunks from the workspace (bf16) --------------------
// One workgroup per (head, 16 NCW value columns), eight waves:
//   waves 0 .. 7-NCW (loaders) move data: the next chunk's workspace block -- the
//     key-side operands Qt, Kh, Kt^T, Tm Diag(beta), Aqk, e^{G_64} of that
//     chunk, laid out as this kernel's LDS image -- is copied global -> LDS
//     directly (16-byte LDS-destination loads) into the other of two stages,
//     the V slice is written transposed next to it, and the previous chunk's
//     output is stored from an LDS staging tile to HBM with 16-byte stores;
//   the last NCW waves (consumers) each own 16 value columns and keep their 128 x 16
//     slice of the state in MFMA accumulators.  For chunk n they form
//       P = Kh S,  Qt S,  Z = V - P,  Vn = Tm Z,  O = Qt S + Aqk Vn (to LDS),
//       S <- Diag(e^{G_64}) S + Kt^T Vn
//     chaining every product through registers: the accumulator layout of one
//     product (lane holds rows 4*(lane/16)+e of column lane%16) is the
//     B-operand layout of the next.  Only A-operands are read from LDS, and
//     consumers issue no global memory operations inside the loop.
// One barrier per chunk.  The 16x16x32 MFMA takes eight contraction values per
// lane; the consumers feed it two 16-row blocks at once (four values from
// each), reading the A-operand with the same split, so each product is a
// plain sum over k.
constexpr int SEG_NONE = 0, SEG_SUMMARY = 1, SEG_OUTPUT = 2;   // chunk_scan_kernel segment modes

template <int NCW, bool SAVE = false> struct ScanCfg {   // NCW consumer waves
    static constexpr int DV = 16 * NCW;                   // value columns per workgroup
    static constexpr int NLW = 8 - NCW;                   // loader waves (two waves per SIMD)
    static constexpr int NT = 64 * (NLW + NCW);
    static constexpr int OFF_VT = 0;                      // V^T [DV cols][72] bf16
    static constexpr int OFF_BLK = DV * WS_P64 * 2;       // workspace image
    static constexpr int STAGE = OFF_BLK + WS_CHUNK;
    static constexpr int OFF_O = 2 * STAGE;               // output staging [2][64][DV] bf16 (not in SAVE mode)
    static constexpr int TOTAL = OFF_O + (SAVE ? 0 : 2 * C * DV * 2);
    static constexpr int VG = DV / 8;                     // 16-byte units per token row
    static constexpr int VPL = (C * VG + 255) / 256;      // V units per lane of the first four waves
    static_assert(TOTAL <= 160 * 1024, "LDS budget");
    static_assert(NLW >= 4, "the first four waves are loaders");
    static_assert(SAVE || VPL == 1, "one output unit per lane of the first four loader waves");
};

// SAVE (the forward part of the backward pass): no output (Qt S and Aqk Vn
// are skipped); instead each chunk's entry state S_n [128][128],
// Y = V - Kh S_n [64][128] and Vn [64][128] are written in bf16 to svS / svY /
// svVn, indexed (head, chunk).
//
// DPLR (the general diagonal-plus-low-rank transition, see kda_dplr.hip): the
// block holds Qt = e^G q, Kh = W, Kb^T = (e^{-G} a)^T and Aqk = A_qa, its Tm
// slot is not used, and `v` points at U0.  Per chunk the scan computes
// Vn = U0 - W S (no Tm product), O = Qt S + A_qa Vn + O0 and
// S <- Diag(gamma) (S + Kb^T Vn) + H0, with O0 [token][128] and
// H0 [head, chunk][128][128] (bf16) from the DPLR prep kernel: H0's slice of
// this workgroup's value columns is loaded into the Tm slot, and O0 is added
// by the loader lanes when they store the output.
//
// SEG (few heads: the chunks of a head are split into segments of seg_len
// chunks that run in parallel).  The chunk-to-chunk map is affine in the
// state, S' = A_n S + B_n, and acts on each state column alike, so a segment
// is summarised by its end state E from a zero entry state and its transition
// P = A_last ... A_first, the end state of the identity matrix run with zero
// values (the page's proposition S_r = P_r S_0 + H_r, taken per segment):
//   SEG_SUMMARY: every segment but the last, 2 x 128 columns per head: value
//     columns from S = 0, then identity columns with V = 0.  No output; the
//     end state goes to segbuf [head][segment][128][256] fp32 (E | P).
//   SEG_OUTPUT: every segment from its entry state segbuf [head][segment]
//     [128][128] (written by seg_combine_kernel, the first a copy of S0, so
//     that S_T may overwrite S0 in place), with the output; the last segment
//     writes S_T.
//
// The body runs on LDS `smem` for the work item `lid` ((head, segment,
// slice) index); with `flags` (the pipelined schedule) the loaders wait for
// each block's ready flag before copying it (see chunk_pipe_kernel).
template <int NCW, bool SAVE, bool DPLR = false, int SEG = SEG_NONE>
__device__ __forceinline__ void
chunk_scan_body(const char* ws, const bf16_t* v, const float* S0, bf16_t* o, float* S_T,
                int T, int H, bf16_t* svS, bf16_t* svY, bf16_t* svVn,
                const bf16_t* h0, const bf16_t* o0, int seg_len, float* segbuf, char* smem, const int lid,
                const int* flags)
{
    static_assert(!(SAVE && DPLR), "the backward pass is KDA only");
    static_assert(SEG == SEG_NONE || !(SAVE || DPLR), "segments: KDA forward only");
    typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;
    constexpr bool NOOUT = SAVE || SEG == SEG_SUMMARY;      // no output products or stores
    using SC = ScanCfg<NCW, NOOUT>;
    static_assert(SC::NT == 512, "eight waves (the launch bounds)");

    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const bool loader = wave < SC::NLW;
    const int ln = lane & 15, lg = lane >> 4;
    const int cw = wave - SC::NLW;
    constexpr int nsplit = (SEG == SEG_SUMMARY ? 2 * DK : DK) / SC::DV;
    const int nchunks = (T + C - 1) / C;
    // segments per head in this launch (1 without SEG)
    const int nsegs = SEG == SEG_NONE ? 1 : (nchunks + seg_len - 1) / seg_len - (SEG == SEG_SUMMARY ? 1 : 0);
    const int head = lid / (nsplit * nsegs), seg = lid / nsplit % nsegs, slice = lid % nsplit;
    const int c0 = SEG == SEG_NONE ? 0 : seg * seg_len;                  // chunks c0 .. c1-1
    const int c1 = SEG == SEG_NONE ? nchunks : min(nchunks, c0 + seg_len);
    const bool ident = SEG == SEG_SUMMARY && slice * SC::DV >= DK;       // identity columns, V = 0
    const int b = head / H, h = head % H;
    const int j0 = slice * SC::DV % DK;
    const size_t tokstride = (size_t)H * DK;
    const size_t hbase = ((size_t)b * T * H + h) * DK;
    const size_t sbase = (size_t)head * DK * DK;
    // block layout: the KDA block (swizzled rows, tiled Tm and Aqk) or the
    // DPLR block (padded rows)
    constexpr int B_QT = DPLR ? WS_QT : WSK_QT, B_KH = DPLR ? WS_KH : WSK_KH, B_KBT = DPLR ? WS_KBT : WSK_KBT;
    constexpr int B_TM = DPLR ? WS_TM : WSK_TM, B_QK = DPLR ? WS_QK : WSK_QK, B_GAM = DPLR ? WS_GAM : WSK_GAM;
    constexpr int B_CHUNK = DPLR ? WS_CHUNK : WSK_CHUNK, B_KIB = B_CHUNK / 1024;
    const char* wsh = ws + (size_t)head * nchunks * B_CHUNK;
    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};

    // ---- loader side: lane pt moves V / output unit (token ut, columns 8 ug ..)
    const int pt = t & 255, ug = pt % SC::VG, ut = pt / SC::VG;
    const bool ulane = t < 256 && ut < C;     // lanes of the first four loader waves
    bf16x8 vrow[SC::VPL], o0row = bf16x8{};   // unit i of a lane: pt + 256 i
    // DPLR: the H0 slice [128][DV] (unpadded) replaces the Tm pages
    constexpr int TM_P0 = B_TM / 1024, TM_P1 = B_QK / 1024;
    constexpr int HPR = SC::DV / 8;                       // 16-byte pieces per H0 row
    constexpr int HRPP = 64 / HPR;                        // H0 rows per 1 KiB page
    constexpr int HPAGES = DK / HRPP;
    static_assert(!DPLR || (B_TM % 1024 == 0 && B_QK % 1024 == 0 && HPAGES <= TM_P1 - TM_P0),
                  "H0 slice fits the Tm slot");
    constexpr int QT_P1 = B_KH / 1024, QK_P0 = B_QK / 1024, QK_P1 = B_GAM / 1024;
    static_assert(B_QT == 0 && B_KH % 1024 == 0 && B_QK % 1024 == 0 && B_GAM % 1024 == 0,
                  "Qt and Aqk occupy whole pages");
    // The block is copied in two groups: G1, the pages of Qt and Kh, which the
    // consumers read first, and G2, the rest.  In step n the loaders issue G2
    // of block n + 1 (and its V rows) at the start; once the consumers have
    // passed their first phase (a second barrier per step) they wait for
    // those, write V^T, store the previous output tile and then issue G1 of
    // block n + 2 into the G1 pages of this step's stage, which stays in
    // flight until the middle of step n + 1.  (Every LDS access of a loader
    // comes after that wait, so no wait for the DMA in flight falls into the
    // part of a step before the middle barrier.)
    constexpr int G1_P0 = NOOUT ? QT_P1 : 0, G1_P1 = B_KBT / 1024;      // G1 pages [G1_P0, G1_P1)
    static_assert(B_KBT % 1024 == 0, "G1 pages");
    auto load_g1 = [&](int n) {               // G1 of block n -> stage n % 2
        const char* src = wsh + (size_t)n * B_CHUNK;
        char* dst = smem + (n & 1) * SC::STAGE + SC::OFF_BLK;
        for (int u = G1_P0 + wave; u < G1_P1; u += SC::NLW)
            __builtin_amdgcn_global_load_lds(src + (size_t)u * 1024 + lane * 16,
                                             (__attribute__((address_space(3))) void*)(dst + u * 1024), 16, 0, 0);
    };
    auto load_block = [&](int n) {            // G2 of workspace block n -> stage n % 2
        const char* src = wsh + (size_t)n * B_CHUNK;
        char* dst = smem + (n & 1) * SC::STAGE + SC::OFF_BLK;
        for (int u = G1_P1 + wave; u < B_KIB; u += SC::NLW) {
            // without output, the Aqk pages are not read: not copied
            if (NOOUT && u >= QK_P0 && u < QK_P1) continue;
            const char* from = src + (size_t)u * 1024 + lane * 16;
            if constexpr (DPLR) {
                if (u >= TM_P0 && u < TM_P1) {
                    const int hp = u - TM_P0;
                    if (hp >= HPAGES) continue;
                    const int row = HRPP * hp + lane / HPR;
                    from = reinterpret_cast<const char*>(
                        h0 + (((size_t)head * nchunks + n) * DK + row) * DK + j0 + 8 * (lane % HPR));
                }
            }
            __builtin_amdgcn_global_load_lds(from, (__attribute__((address_space(3))) void*)(dst + u * 1024),
                                             16, 0, 0);
        }
    };
    // pipelined schedule: block n is copied only once its ready flag is set.
    // The producers never wait, so every wait ends; the spin budget (shared
    // by all waits of the wave, about a second in all) only guards against a
    // launch that cannot make progress: once spent, the wave stops waiting.
    // The flag is read with a scalar load that bypasses the scalar cache
    // (glc), waited for in the same statement: it does not count against the
    // vector-memory counter, so a poll does not wait for the copies in flight.
    int spin_budget = 1 << 20;
    auto wait_ready = [&](int n) {
        if (!flags) return;
        const int* f = flags + (size_t)head * nchunks + n;
        while (spin_budget > 0) {
            int fv;
            asm volatile("s_load_dword %0, %1, 0x0 glc\n\ts_waitcnt lgkmcnt(0)" : "=s"(fv) : "s"(f) : "memory");
            if (fv != 0) break;
            __builtin_amdgcn_s_sleep(1);
            --spin_budget;
        }
    };
    auto load_v = [&](int n) {
        if (t >= 256 || ident) return;
#pragma unroll
        for (int i = 0; i < SC::VPL; ++i) {
            const int u = pt + 256 * i, uu = u / SC::VG, ug2 = u % SC::VG;
            if (uu >= C) continue;
            const int tok = min(n * C + uu, T - 1);
            vrow[i] = *reinterpret_cast<const bf16x8*>(v + hbase + (size_t)tok * tokstride + j0 + 8 * ug2);
        }
    };
    auto write_vt = [&](int n) {              // V^T of chunk n into stage n % 2
        bf16_t* vt = reinterpret_cast<bf16_t*>(smem + (n & 1) * SC::STAGE + SC::OFF_VT);
        if (t >= 256) return;
#pragma unroll
        for (int i = 0; i < SC::VPL; ++i) {
            const int u = pt + 256 * i, uu = u / SC::VG, ug2 = u % SC::VG;
            if (uu >= C) continue;
            const bool ok = !ident && n * C + uu < T;
#pragma unroll
            for (int c = 0; c < 8; ++c) vt[(8 * ug2 + c) * WS_P64 + uu] = ok ? vrow[i][c] : bf16_t{};
        }
    };
    auto load_o0 = [&](int n) {               // DPLR: O0 row of chunk n, stored with it next step
        if (!ulane) return;
        const int tok = min(n * C + ut, T - 1);
        o0row = *reinterpret_cast<const bf16x8*>(o0 + hbase + (size_t)tok * tokstride + j0 + 8 * ug);
    };
    auto store_out = [&](int n) {             // output tile of chunk n: LDS -> HBM
        const bf16_t* ot = reinterpret_cast<const bf16_t*>(smem + SC::OFF_O + (n & 1) * C * SC::DV * 2);
        if (ulane && n * C + ut < T) {
            bf16x8 x = *reinterpret_cast<const bf16x8*>(ot + ut * SC::DV + 8 * ug);
            if constexpr (DPLR) {
#pragma unroll
                for (int c = 0; c < 8; ++c) x[c] = (bf16_t)((float)x[c] + (float)o0row[c]);
            }
            *reinterpret_cast<bf16x8*>(o + hbase + (size_t)(n * C + ut) * tokstride + j0 + 8 * ug) = x;
        }
    };

    // ---- consumer side: S[16cb + 4lg + e][j0 + jc] in acc_s[cb][e] ----
    const int jc = 16 * cw + ln;
    f32x4 acc_s[8];
    if (!loader) {
        // entry state: S0, zero or the identity (summary), or the segment's
        // entry state from seg_combine_kernel
        const float* sin = S0 ? S0 + sbase : nullptr;
        if (SEG == SEG_OUTPUT) sin = segbuf + ((size_t)head * nsegs + seg) * DK * DK;
        if (SEG == SEG_SUMMARY) sin = nullptr;
#pragma unroll
        for (int cb = 0; cb < 8; ++cb)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * cb + 4 * lg + e;
                acc_s[cb][e] = sin ? sin[(size_t)r * DK + j0 + jc] : (ident && r == j0 + jc ? 1.f : 0.f);
            }
    } else {
        wait_ready(c0);
        load_g1(c0);
        load_block(c0);
        load_v(c0);
        __builtin_amdgcn_s_waitcnt(0);        // vmcnt, lgkmcnt and expcnt all zero
        write_vt(c0);
        if (c0 + 1 < c1) { wait_ready(c0 + 1); load_g1(c0 + 1); }   // lands during step c0
    }
    lds_barrier();

    for (int n = c0; n < c1; ++n) {
        if (loader) {
            // the ready flag of block n + 2, read early (a vector load that
            // lands with the copies below); polled only if it was not set
            int ready2 = 1;
            if (flags && n + 2 < c1)
                ready2 = __hip_atomic_load(flags + (size_t)head * nchunks + n + 2, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
            // G2 (and V) of block n + 1; its G1 is in flight since step n - 1
            if (n + 1 < c1) { load_block(n + 1); load_v(n + 1); }
            lds_barrier();                    // the consumers are done with G1 of block n
            __builtin_amdgcn_s_waitcnt(0);    // block n + 1 complete (G1, G2), V rows in registers
            if (n + 1 < c1) write_vt(n + 1);
            if (!NOOUT && n > c0) store_out(n - 1);
            if constexpr (DPLR) load_o0(n);   // (after the store of chunk n - 1, which adds O0 of n - 1)
            if (n + 2 < c1) {
                if (__builtin_amdgcn_readfirstlane(ready2) == 0) wait_ready(n + 2);
                load_g1(n + 2);               // into the G1 pages of this step's stage
            }
        } else {
            const char* st = smem + (n & 1) * SC::STAGE;
            const bf16_t* sQt = reinterpret_cast<const bf16_t*>(st + SC::OFF_BLK + B_QT);
            const bf16_t* sKh = reinterpret_cast<const bf16_t*>(st + SC::OFF_BLK + B_KH);
            const bf16_t* sKbT = reinterpret_cast<const bf16_t*>(st + SC::OFF_BLK + B_KBT);
            const bf16_t* sTm = reinterpret_cast<const bf16_t*>(st + SC::OFF_BLK + B_TM);
            const bf16_t* sQK = reinterpret_cast<const bf16_t*>(st + SC::OFF_BLK + B_QK);
            const float* sGam = reinterpret_cast<const float*>(st + SC::OFF_BLK + B_GAM);
            // A-operand pair p of row block Rb of Tm or Aqk (lower part only)
            auto tri_pair = [&](const bf16_t* m, int Rb, int p) {
                if constexpr (DPLR) return a_pair(m + (16 * Rb + ln) * WS_P64, p, lg, 2 * p + 1 <= Rb);
                else {
                    const char* q = reinterpret_cast<const char*>(m) + wsk_pair_off(Rb, p);
                    if (wsk_pair_full(Rb, p)) return *reinterpret_cast<const bf16x8*>(q + 16 * (4 * ln + lg));
                    return cat8(*reinterpret_cast<const bf16x4*>(q + 8 * (4 * ln + lg)), bf16x4{});
                }
            };
            const bf16_t* sVT = reinterpret_cast<const bf16_t*>(st + SC::OFF_VT);
            bf16_t* sO = reinterpret_cast<bf16_t*>(smem + SC::OFF_O + (n & 1) * C * SC::DV * 2);
            const size_t cidx = (size_t)head * nchunks + n;
            // saved tiles (SAVE): neighbouring lanes pair up so that each store
            // is a 4-byte column pair (see pair_rows_bf16).  S (the state
            // entering the chunk), Y and Vn are stored at the end of the step:
            // issued earlier they queue behind the loader waves' block copy and
            // hold up the dependent MFMA chain.
            const int prow = 4 * lg + 2 * (ln & 1), pcol = j0 + 16 * cw + (ln & ~1);
            bf16x2 s_pr[SAVE ? 8 : 1][2], y_pr[SAVE ? 4 : 1][2], w_pr[SAVE ? 4 : 1][2];
            if constexpr (SAVE) {
#pragma unroll
                for (int cb = 0; cb < 8; ++cb) pair_rows_bf16(acc_s[cb], lane, s_pr[cb][0], s_pr[cb][1]);
            }

            // P = Kh S and Qt S; a block's eight operand loads go out before its
            // products, the next block's while they run
            bf16x8 sb[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) sb[p] = cat8(to_bf16x4(acc_s[2 * p]), to_bf16x4(acc_s[2 * p + 1]));
            constexpr int NF = NOOUT ? 4 : 8;         // Kh (and Qt) fragments per block
            bf16x8 fa[2][NF];
            // A-operand pair p of rows 16 Rb + ln of Kh or Qt: padded rows
            // (DPLR), or one 16-byte unit (KDA)
            auto tok_pair = [&](const bf16_t* m, int Rb, int p) {
                if constexpr (DPLR) return a_pair(m + (16 * Rb + ln) * WS_P128, p, lg, true);
                else return *reinterpret_cast<const bf16x8*>(m + wsk_tok_unit(16 * Rb + ln, 4 * p + lg));
            };
            auto frags = [&](int Rb, bf16x8 (&f)[NF]) {
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    f[p] = tok_pair(sKh, Rb, p);
                    if constexpr (!NOOUT) f[4 + p] = tok_pair(sQt, Rb, p);
                }
            };
            f32x4 pk[4], qs[4];
            frags(0, fa[0]);
#pragma unroll
            for (int Rb = 0; Rb < 4; ++Rb) {
                if (Rb + 1 < 4) frags(Rb + 1, fa[(Rb + 1) & 1]);
                f32x4 a = z4, c2 = z4;
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[Rb & 1][p], sb[p], a, 0, 0, 0);
                    if constexpr (!NOOUT)
                        c2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[Rb & 1][4 + p], sb[p], c2, 0, 0, 0);
                }
                pk[Rb] = a;
                qs[Rb] = c2;
                if (Rb + 1 < 4) __builtin_amdgcn_sched_group_barrier(0x100, NF, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, NF, 0);
            }
            // the G1 pages of this stage (Qt, Kh) are read: the loaders may
            // refill them with block n + 2
            lds_barrier();

            // Z = V - P (V^T read in the B layout), Vn = Tm Z (lower blocks only)
            f32x4 zt[4], vn[4];
#pragma unroll
            for (int Rb = 0; Rb < 4; ++Rb) {
                const bf16x4 vv = ld4(sVT + jc * WS_P64 + 16 * Rb + 4 * lg);
#pragma unroll
                for (int e = 0; e < 4; ++e) zt[Rb][e] = (float)vv[e] - pk[Rb][e];
            }
#pragma unroll
            for (int Rb = 0; Rb < 4; ++Rb) {
                if constexpr (DPLR) {
                    vn[Rb] = zt[Rb];
                    continue;
                }
                f32x4 a = z4;
#pragma unroll
                for (int p = 0; p < 2; ++p)
                    if (2 * p <= Rb)
                        a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            tri_pair(sTm, Rb, p), cat8(to_bf16x4(zt[2 * p]), to_bf16x4(zt[2 * p + 1])), a, 0, 0, 0);
                vn[Rb] = a;
            }
            if constexpr (SAVE) {
#pragma unroll
                for (int Rb = 0; Rb < 4; ++Rb) {
                    pair_rows_bf16(zt[Rb], lane, y_pr[Rb][0], y_pr[Rb][1]);
                    pair_rows_bf16(vn[Rb], lane, w_pr[Rb][0], w_pr[Rb][1]);
                }
            }

            // O = Qt S + Aqk Vn -> LDS staging (stored to HBM by the loaders)
            if constexpr (!NOOUT)
#pragma unroll
            for (int Rb = 0; Rb < 4; ++Rb) {
                f32x4 a = qs[Rb];
#pragma unroll
                for (int p = 0; p < 2; ++p)
                    if (2 * p <= Rb)
                        a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            tri_pair(sQK, Rb, p), cat8(to_bf16x4(vn[2 * p]), to_bf16x4(vn[2 * p + 1])), a, 0, 0, 0);
#pragma unroll
                for (int e = 0; e < 4; ++e) sO[(16 * Rb + 4 * lg + e) * SC::DV + jc] = (bf16_t)a[e];
            }

            // KDA: S <- Diag(gamma) S + Kt^T Vn with Kt = e^{G_64 - G} k (the
            // block's Kb^T slot holds Kt^T); DPLR: S <- Diag(gamma) (S + Ab^T Vn)
            // + H0 (the slot holds (e^{-G} a)^T).  kbt(16cb + ln, 32p + 16hh + 4lg)
            // splits into a lane part and a compile-time part: the swizzle bits
            // 1-2 depend on (cb, p, hh) only.
            bf16x8 vb[2];
#pragma unroll
            for (int p = 0; p < 2; ++p) vb[p] = cat8(to_bf16x4(vn[2 * p]), to_bf16x4(vn[2 * p + 1]));
            // DPLR block: rows of 72 with the 8-token blocks XOR-permuted by
            // bits 3..5 of the channel (two 8-byte halves per operand); KDA
            // block: one 16-byte unit per operand
            const bf16_t* kl = sKbT + ln * WS_P64 + ((((lg >> 1) ^ (ln >> 3)) & 1) << 3) + 4 * (lg & 1);
            auto kbt_at = [&](int cb, int p, int hh) {
                return kl + 16 * cb * WS_P64 + ((p ^ ((cb >> 1) & 1)) << 5) + ((hh ^ (cb & 1)) << 4);
            };
            auto kbt_pair = [&](int cb, int p) {
                if constexpr (DPLR) return cat8(ld4(kbt_at(cb, p, 0)), ld4(kbt_at(cb, p, 1)));
                else return *reinterpret_cast<const bf16x8*>(sKbT + wsk_kbt_unit(16 * cb + ln, 4 * p + lg));
            };
#pragma unroll
            for (int cb = 0; cb < 8; ++cb) {
                const f32x4 gv = *reinterpret_cast<const f32x4*>(sGam + 16 * cb + 4 * lg);
                if constexpr (!DPLR) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc_s[cb][e] *= gv[e];
                }
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    const bf16x8 a = kbt_pair(cb, p);
                    acc_s[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, vb[p], acc_s[cb], 0, 0, 0);
                }
                if constexpr (DPLR) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc_s[cb][e] *= gv[e];
                }
                if constexpr (DPLR) {
                    const bf16_t* sH0 = sTm;          // [128][DV] in the Tm slot
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc_s[cb][e] += (float)sH0[(16 * cb + 4 * lg + e) * SC::DV + jc];
                }
            }
            if constexpr (SAVE) {
#pragma unroll
                for (int cb = 0; cb < 8; ++cb) {
                    *reinterpret_cast<bf16x2*>(svS + sv_at(cidx, DK, 16 * cb + prow, pcol)) = s_pr[cb][0];
                    *reinterpret_cast<bf16x2*>(svS + sv_at(cidx, DK, 16 * cb + prow + 1, pcol)) = s_pr[cb][1];
                }
#pragma unroll
                for (int Rb = 0; Rb < 4; ++Rb) {
                    const size_t a0 = sv_at(cidx, C, 16 * Rb + prow, pcol), a1 = sv_at(cidx, C, 16 * Rb + prow + 1, pcol);
                    *reinterpret_cast<bf16x2*>(svY + a0) = y_pr[Rb][0];
                    *reinterpret_cast<bf16x2*>(svY + a1) = y_pr[Rb][1];
                    *reinterpret_cast<bf16x2*>(svVn + a0) = w_pr[Rb][0];
                    *reinterpret_cast<bf16x2*>(svVn + a1) = w_pr[Rb][1];
                }
            }
        }
        lds_barrier();
    }

    if (loader) {
        if (!NOOUT) store_out(c1 - 1);
    } else if (SEG == SEG_SUMMARY) {
        float* dst = segbuf + ((size_t)head * nsegs + seg) * DK * 2 * DK + slice * SC::DV + jc;
#pragma unroll
        for (int cb = 0; cb < 8; ++cb)
#pragma unroll
            for (int e = 0; e < 4; ++e) dst[(size_t)(16 * cb + 4 * lg + e) * 2 * DK] = acc_s[cb][e];
    } else if (S_T && (SEG == SEG_NONE || seg == nsegs - 1)) {
#pragma unroll
        for (int cb = 0; cb < 8; ++cb)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                S_T[sbase + (size_t)(16 * cb + 4 * lg + e) * DK + j0 + jc] = acc_s[cb][e];
    }
}

template <int NCW, bool SAVE, bool DPLR = false, int SEG = SEG_NONE>
__global__ void __launch_bounds__(512)
chunk_scan_kernel(const char* ws, const bf16_t* v, const float* S0, bf16_t* o, float* S_T,
                  int T, int H, bf16_t* svS, bf16_t* svY, bf16_t* svVn,
                  const bf16_t* h0, const bf16_t* o0, int seg_len, float* segbuf)
{
    __shared__ __attribute__((aligned(1024))) char smem[ScanCfg<NCW, SAVE || SEG == SEG_SUMMARY>::TOTAL];
    const int nwg = gridDim.x, w = blockIdx.x;
    const int lid = (nwg % 8 == 0) ? (w % 8) * (nwg / 8) + w / 8 : w;   // slices of a head on one XCD
    chunk_scan_body<NCW, SAVE, DPLR, SEG>(ws, v, S0, o, S_T, T, H, svS, svY, svVn, h0, o0, seg_len, segbuf, smem,
                                          lid, nullptr);
}

// Entry states of the segments of SEG_OUTPUT, entry [head][j][128][128]:
// with E_j | P_j the summary of segment j (end state from zero, transition),
// S_{j+1} = P_j S_j + E_j from S_0 = S0 (or zero), in fp32.  One workgroup
// per (head, 16 state columns); thread t computes row t / 2, columns
// 8 (t % 2) .. +7.
__global__ void __launch_bounds__(256)
seg_combine_kernel(const float* summ, const float* S0, float* entry, int nseg)
{
    __shared__ float cur[DK][16];
    const int head = blockIdx.x / (DK / 16), j0 = blockIdx.x % (DK / 16) * 16;
    const int t = threadIdx.x, r = t >> 1, c8 = (t & 1) * 8;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const float x = S0 ? S0[((size_t)head * DK + r) * DK + j0 + c8 + c] : 0.f;
        cur[r][c8 + c] = x;
        entry[((size_t)head * nseg * DK + r) * DK + j0 + c8 + c] = x;
    }
    __syncthreads();
    for (int j = 0; j + 1 < nseg; ++j) {
        const float* sm = summ + (((size_t)head * (nseg - 1) + j) * DK + r) * 2 * DK;   // row r of E_j | P_j
        float acc[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] = sm[j0 + c8 + c];
        // the row of P_j in registers first (its 32 loads in flight together)
        f32x4 prow[DK / 4];
#pragma unroll
        for (int i = 0; i < DK / 4; ++i) prow[i] = *reinterpret_cast<const f32x4*>(sm + DK + 4 * i);
#pragma unroll
        for (int i = 0; i < DK / 4; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int c = 0; c < 8; ++c) acc[c] = fmaf(prow[i][e], cur[4 * i + e][c8 + c], acc[c]);
        __syncthreads();
        float* out = entry + (((size_t)head * nseg + j + 1) * DK + r) * DK + j0 + c8;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            cur[r][c8 + c] = acc[c];
            out[c] = acc[c];
        }
        __syncthreads();
    }
}

// ---- prep and scan in one launch (pipelined two-kernel schedule) -------------
// For 24 to 48 heads (a multiple of 8, bf16): the prep role's chunk blocks are
// consumed by the scan role while the prep is still running, so the key-side
// work of later chunks overlaps the serial state scan, and each block is read
// from the L2 it was just written to instead of from HBM.  One workgroup per
// CU, 32 per XCD: on each XCD the first `nprep` workgroups to arrive become
// producers, the others consumers (one per head of that XCD and 32 value
// columns).  The heads of XCD x are x, x + 8, ...; producers walk their
// XCD's chunk groups group-major (all heads' group 0, then group 1, ...) and
// set a ready flag per block; consumers run chunk_scan_body, whose loaders
// wait for each block's flag.  Producer and consumer of a block share the
// XCD's L2, where the flag and the block meet (the producer waits for its
// stores' acknowledgements before setting the flag).  Roles come from the
// hardware XCD id and a per-XCD arrival counter, so the pairing does not
// depend on how workgroups are dealt to XCDs; producers never wait, and
// consumers arrive after them, so the launch always progresses.  The flags
// and counters are cleared by pipe_clear_kernel before the launch.
constexpr int PIPE_NCW = 2;                                // consumer: 32 value columns
constexpr int PIPE_LDS = Layout<bf16_t, 16>::TOTAL > ScanCfg<PIPE_NCW>::TOTAL ? Layout<bf16_t, 16>::TOTAL
                                                                               : ScanCfg<PIPE_NCW>::TOTAL;
constexpr int PIPE_PER_XCD = 32;                           // workgroups per XCD (256 CUs / 8)

__device__ __forceinline__ int xcc_id() {
    // HW_REG_XCC_ID (hardware register 20), bits 3:0
    return __builtin_amdgcn_s_getreg((20) | (0 << 6) | (3 << 11)) & 7;
}

__global__ void __launch_bounds__(256)
pipe_clear_kernel(int* p, int n)
{
    for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = 0;
}

template <int GATE>
__global__ void __launch_bounds__(512)
chunk_pipe_kernel(const bf16_t* q, const bf16_t* k, const bf16_t* v, const float* g, const bf16_t* beta,
                  const float* S0, bf16_t* o, float* S_T, int T, int H, int heads, char* ws, int* flags,
                  int* counters)
{
    __shared__ __attribute__((aligned(1024))) char smem[PIPE_LDS];
    constexpr int NSL = DK / ScanCfg<PIPE_NCW>::DV;        // consumers per head
    const int x = xcc_id();
    // arrival index on this XCD (passed through the first LDS word, which the
    // roles overwrite only after the second barrier)
    if (threadIdx.x == 0) *reinterpret_cast<int*>(smem) = atomicAdd(counters + x, 1);
    __syncthreads();
    const int j = *reinterpret_cast<const int*>(smem);
    __syncthreads();
    const int hx = heads / 8;                              // heads per XCD
    const int nprep = PIPE_PER_XCD - NSL * hx;
    const int nchunks = (T + C - 1) / C;
    const int nblk = (nchunks + PREP_CHUNKS - 1) / PREP_CHUNKS;
    if (j < nprep) {
        for (int i = j; i < hx * nblk; i += nprep) {
            const int grp = i / hx, head = x + 8 * (i % hx);
            chunk_fwd_body<bf16_t, 16, true, false, GATE>(q, k, v, g, beta, S0, nullptr, nullptr, T, H, 1, ws,
                                                          nullptr, nullptr, smem, head * nblk + grp, flags);
        }
    } else if (j < PIPE_PER_XCD) {
        const int js = j - nprep, head = x + 8 * (js / NSL), slice = js % NSL;
        chunk_scan_body<PIPE_NCW, false>(ws, v, S0, o, S_T, T, H, nullptr, nullptr, nullptr, nullptr, nullptr, 0,
                                         nullptr, smem, head * NSL + slice, flags);
    }
}

template <typename E, int DV, int GATE>
void launch_one(const void* q, const void* k, const void* v, const float* g, const void* beta,
                const float* S0, void* o, float* S_T, int B, int T, int H, hipStream_t stream,
                const int* cu_seqlens = nullptr)
{
    const int nsplit = DK / DV;
    const unsigned nwg = (unsigned)((long long)B * H * nsplit);
    hipLaunchKernelGGL((chunk_fwd_kernel<E, DV, false, false, GATE>), dim3(nwg), dim3(NT), 0, stream,
                       (const E*)q, (const E*)k, (const E*)v, g, (const E*)beta, S0, (E*)o, S_T,
                       T, H, nsplit, (char*)nullptr, (char*)nullptr, cu_seqlens);
}

template <int GATE>
void launch_gate(const void* q, const void* k, const void* v, const float* g, const void* beta,
                 const float* S0, void* o, float* S_T, int B, int T, int H, int dtype, void* ws,
                 hipStream_t stream, const int* cu, bool seg)
{
    const long long heads = (long long)B * H;
    if (dtype == 0) {
        // fp32 operands need the narrowest slice to fit the LDS budget
        launch_one<float, 16, GATE>(q, k, v, g, beta, S0, o, S_T, B, T, H, stream, cu);
    } else if (ws) {
        const int nchunks = (T + C - 1) / C;
        const int nblk = (nchunks + PREP_CHUNKS - 1) / PREP_CHUNKS;
        if (seg && chunk_uses_pipe(B, T, H)) {
            // prep and scan in one launch; flags and arrival counters after the blocks
            int* flags = reinterpret_cast<int*>((char*)ws + chunk_ws_bytes(B, T, H));
            int* counters = flags + heads * nchunks;
            const int nclear = (int)(heads * nchunks + 8);
            hipLaunchKernelGGL(pipe_clear_kernel, dim3((unsigned)std::min(1024, (nclear + 255) / 256)), dim3(256),
                               0, stream, flags, nclear);
            hipLaunchKernelGGL((chunk_pipe_kernel<GATE>), dim3(8 * PIPE_PER_XCD), dim3(512), 0, stream,
                               (const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v, g, (const bf16_t*)beta, S0,
                               (bf16_t*)o, S_T, T, H, (int)heads, (char*)ws, flags, counters);
            return;
        }
        hipLaunchKernelGGL((chunk_fwd_kernel<bf16_t, 16, true, false, GATE>), dim3((unsigned)(heads * nblk)),
                           dim3(NT), 0, stream, (const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v, g,
                           (const bf16_t*)beta, S0, (bf16_t*)o, S_T, T, H, 1, (char*)ws, (char*)nullptr,
                           (const int*)nullptr);
        const int nseg0 = seg ? chunk_seg_count(B, T, H) : 1;
        const int L = (nchunks + nseg0 - 1) / nseg0;          // chunks per segment
        const int nseg = (nchunks + L - 1) / L;                // as the kernels count them (<= nseg0)
        if (nseg > 1) {
            // few heads: segments in parallel (summaries, combine, outputs)
            float* summ = reinterpret_cast<float*>((char*)ws + chunk_ws_bytes(B, T, H));
            float* entry = summ + (size_t)heads * (nseg - 1) * DK * 2 * DK;
            hipLaunchKernelGGL((chunk_scan_kernel<4, false, false, SEG_SUMMARY>),
                               dim3((unsigned)(heads * (nseg - 1) * (2 * DK / ScanCfg<4, true>::DV))),
                               dim3(ScanCfg<4, true>::NT), 0, stream, (const char*)ws, (const bf16_t*)v,
                               (const float*)nullptr, (bf16_t*)nullptr, (float*)nullptr, T, H, (bf16_t*)nullptr,
                               (bf16_t*)nullptr, (bf16_t*)nullptr, (const bf16_t*)nullptr, (const bf16_t*)nullptr,
                               L, summ);
            hipLaunchKernelGGL(seg_combine_kernel, dim3((unsigned)(heads * (DK / 16))), dim3(256), 0, stream,
                               (const float*)summ, S0, entry, nseg);
            hipLaunchKernelGGL((chunk_scan_kernel<2, false, false, SEG_OUTPUT>),
                               dim3((unsigned)(heads * nseg * (DK / ScanCfg<2>::DV))), dim3(ScanCfg<2>::NT), 0,
                               stream, (const char*)ws, (const bf16_t*)v, S0, (bf16_t*)o, S_T, T, H,
                               (bf16_t*)nullptr, (bf16_t*)nullptr, (bf16_t*)nullptr, (const bf16_t*)nullptr,
                               (const bf16_t*)nullptr, L, entry);
            return;
        }
        // value columns per scan workgroup: enough workgroups to cover the machine
        const int ncw = heads * 4 >= 256 ? 2 : 1;
#define KDA_SCAN(NCW) hipLaunchKernelGGL((chunk_scan_kernel<NCW, false>), dim3((unsigned)(heads * (DK / ScanCfg<NCW>::DV))), \
                                         dim3(ScanCfg<NCW>::NT), 0, stream, (const char*)ws, (const bf16_t*)v, S0, \
                                         (bf16_t*)o, S_T, T, H, (bf16_t*)nullptr, (bf16_t*)nullptr, (bf16_t*)nullptr, \
                                         (const bf16_t*)nullptr, (const bf16_t*)nullptr, 0, (float*)nullptr)
        if (ncw == 2) KDA_SCAN(2);
        else KDA_SCAN(1);
#undef KDA_SCAN
    } else if (heads * 2 >= 256) {
        launch_one<bf16_t, 64, GATE>(q, k, v, g, beta, S0, o, S_T, B, T, H, stream, cu);
    } else if (heads * 4 >= 256) {
        launch_one<bf16_t, 32, GATE>(q, k, v, g, beta, S0, o, S_T, B, T, H, stream, cu);
    } else {
        launch_one<bf16_t, 16, GATE>(q, k, v, g, beta, S0, o, S_T, B, T, H, stream, cu);
    }
}

}  // namespace

size_t chunk_ws_bytes(long long B, long long T, long long H)
{
    return (size_t)B * (size_t)H * (size_t)((T + C - 1) / C) * (size_t)WSK_CHUNK;
}

int chunk_seg_count(long long B, long long T, long long H)
{
    // With 16 heads or fewer, one workgroup per 16 value columns leaves CUs
    // idle; segments of each head then run in parallel (4 value-column
    // workgroups per segment, about 256 workgroups in all), each segment at
    // least two chunks long.
    const long long heads = B * H, nchunks = (T + C - 1) / C;
    if (heads > 16) return 1;
    long long nseg = std::min<long long>(16, 64 / heads);
    nseg = std::min(nseg, nchunks / 2);
    if (nseg < 2) return 1;
    const long long L = (nchunks + nseg - 1) / nseg;
    return (int)((nchunks + L - 1) / L);     // no empty trailing segment
}

bool chunk_uses_pipe(long long B, long long T, long long H)
{
    // 24 to 48 heads, a multiple of 8 (whole heads per XCD): 12 to 24 scan
    // workgroups of 32 columns per XCD, the rest producers
    const long long heads = B * H;
    return heads % 8 == 0 && heads >= 24 && heads <= 48 && (T + C - 1) / C >= 2;
}

size_t chunk_fwd_ws_bytes(long long B, long long T, long long H)
{
    if (chunk_uses_pipe(B, T, H))   // blocks, then a ready flag per block and 8 arrival counters
        return chunk_ws_bytes(B, T, H) + ((size_t)B * H * ((T + C - 1) / C) + 8) * 4;
    const int nseg = chunk_seg_count(B, T, H);
    // summaries [nseg - 1][128][256] and entry states [nseg][128][128] per head
    const size_t seg = nseg > 1 ? (size_t)B * H * (3 * (nseg - 1) + 1) * DK * DK * 4 : 0;
    return chunk_ws_bytes(B, T, H) + seg;
}

bool chunk_prefers_two_kernel(long long B, long long T, long long H, int dtype)
{
    // The fused kernel recomputes the key-side work once per value slice; with
    // fewer than 128 heads it needs 4 or 8 slices to fill the machine, and the
    // precomputed operands (about 1 KiB per token) cost less than the recompute.
    return dtype == 1 && B * H < 128 && T > C;
}

hipError_t launch_bwd_forward_part(const void* q, const void* k, const void* v, const float* g,
                                  const void* beta, const float* S0, int B, int T, int H,
                                  char* ws_fwd, char* ws_bwd, bf16_t* svS, bf16_t* svY, bf16_t* svVn,
                                  hipStream_t stream, int gate)
{
    const long long heads = (long long)B * H;
    const int nchunks = (T + C - 1) / C;
    const int nblk = (nchunks + PREP_CHUNKS - 1) / PREP_CHUNKS;
#define KDA_PREP(GT) hipLaunchKernelGGL((chunk_fwd_kernel<bf16_t, 16, true, true, GT>), dim3((unsigned)(heads * nblk)),   \
                                      dim3(NT), 0, stream, (const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v, g,     \
                                      (const bf16_t*)beta, S0, (bf16_t*)nullptr, (float*)nullptr, T, H, 1, ws_fwd,     \
                                      ws_bwd, (const int*)nullptr)
    if (gate == GATE_HEAD) KDA_PREP(GATE_HEAD);
    else if (gate == GATE_NONE) KDA_PREP(GATE_NONE);
    else KDA_PREP(GATE_CHANNEL);
#undef KDA_PREP
    // (save mode has no output staging, so 64-column slices fit: one round of
    // workgroups from 128 heads on)
    const int ncw = heads * 2 >= 256 ? 4 : heads * 4 >= 256 ? 2 : 1;
#define KDA_SCAN(NCW) hipLaunchKernelGGL((chunk_scan_kernel<NCW, true>), dim3((unsigned)(heads * (DK / ScanCfg<NCW, true>::DV))), \
                                         dim3(ScanCfg<NCW, true>::NT), 0, stream, (const char*)ws_fwd, (const bf16_t*)v, S0, \
                                         (bf16_t*)nullptr, (float*)nullptr, T, H, svS, svY, svVn, \
                                         (const bf16_t*)nullptr, (const bf16_t*)nullptr, 0, (float*)nullptr)
    if (ncw == 4) KDA_SCAN(4);
    else if (ncw == 2) KDA_SCAN(2);
    else KDA_SCAN(1);
#undef KDA_SCAN
    return hipGetLastError();
}

hipError_t launch_dplr_scan(const char* blocks, const bf16_t* u0, const bf16_t* h0, const bf16_t* o0,
                            const float* S0, void* o, float* S_T, int B, int T, int H, hipStream_t stream)
{
    const long long heads = (long long)B * H;
    const int ncw = heads * 4 >= 256 ? 2 : 1;
#define KDA_SCAN(NCW) hipLaunchKernelGGL((chunk_scan_kernel<NCW, false, true>),                                   \
                                         dim3((unsigned)(heads * (DK / ScanCfg<NCW>::DV))), dim3(ScanCfg<NCW>::NT), \
                                         0, stream, blocks, u0, S0, (bf16_t*)o, S_T, T, H, (bf16_t*)nullptr,       \
                                         (bf16_t*)nullptr, (bf16_t*)nullptr, h0, o0, 0, (float*)nullptr)
    if (ncw == 2) KDA_SCAN(2);
    else KDA_SCAN(1);
#undef KDA_SCAN
    return hipGetLastError();
}

hipError_t launch_chunk_fwd(const void* q, const void* k, const void* v, const float* g,
                            const void* beta, const float* S0, void* o, float* S_T,
                            int B, int T, int H, int dtype, void* ws, hipStream_t stream, int gate,
                            const int* cu_seqlens, bool seg)
{
    if (cu_seqlens) ws = nullptr;   // packed sequences: fused kernel
    if (gate == GATE_HEAD)
        launch_gate<GATE_HEAD>(q, k, v, g, beta, S0, o, S_T, B, T, H, dtype, ws, stream, cu_seqlens, seg);
    else if (gate == GATE_NONE)
        launch_gate<GATE_NONE>(q, k, v, g, beta, S0, o, S_T, B, T, H, dtype, ws, stream, cu_seqlens, seg);
    else
        launch_gate<GATE_CHANNEL>(q, k, v, g, beta, S0, o, S_T, B, T, H, dtype, ws, stream, cu_seqlens, seg);
    return hipGetLastError();
}

}  // namespace kda
