// kda_backward.hip -- backward pass of the chunked KDA prefill for gfx950.
//
// The forward pass is the chunkwise algorithm of page "Kimi Linear：高效注意力
// 机制在长序列处理中的创新应用" (sections 2.1-2.3) and page "Kimi K3论文：Kimi
// Linear" (section 4).  Per chunk of 64 tokens, with S the state entering it,
// G the in-chunk cumulative log-decay and gamma = e^{G_64}:
//
//   Qt = e^G q,  Kh = e^G k,  Kb = e^-G k,  Kt = e^{G_64 - G} k
//   Aqk = tril(Qt Kb^T),  Akk = Diag(beta) stril(Kh Kb^T),  Tm = (I + Akk)^-1
//   Y = V - Kh S,  Vn = Tm Diag(beta) Y
//   O = Qt S + Aqk Vn,   S' = Diag(gamma) S + Kt^T Vn
//
// Reverse mode through these lines, given dO and dS' (the gradient of the
// state leaving the chunk), is
//
//   dVn = Aqk^T dO + Kt dS'          dZ = Tm^T dVn        dV = Diag(beta) dZ
//   dS  = Diag(gamma) dS' + Qt^T dO - Kh^T dV                    (to chunk n-1)
//   dAqk = tril(dO Vn^T)             dAkk = -stril(dZ Vn^T),  dA' = Diag(beta) dAkk
//   dQt = dO S^T + dAqk Kb           dKh = -dV S^T + dA' Kb
//   dKb = dAqk^T Qt + dA'^T Kh       dKt = Vn dS'^T
//   dbeta_r = sum_j Y[r,j] dZ[r,j] + sum_i dAkk[r,i] (Kh Kb^T)[r,i]
//   dq = e^G dQt,  dk = e^G dKh + e^-G dKb + e^{G_64-G} dKt
//   dG = Qt.dQt + Kh.dKh - Kb.dKb - Kt.dKt (elementwise)
// (the gradient kernel evaluates these with every decay factor referenced to
// the end of a 16-token sub-chunk rather than to the chunk start, so that no
// factor grows with the chunk's total decay; see chunk_bwd_grad_kernel)
//   dG_64 += e^{G_64} sum_j S[c,j] dS'[c,j] + sum_r Kt[r,c] dKt[r,c]
//   dg = reverse cumulative sum of dG over the chunk's tokens.
//
// The pass runs four kernels:
//   1. the forward prep kernel, which also writes the operands of the reverse
//      scan (Aqk^T, Tm^T, Qt^T, Kh^T, Kt, gamma, beta) per chunk;
//   2. the forward scan in save mode: S, Y and Vn of every chunk (bf16);
//   3. chunk_bwd_scan_kernel: the serial reverse pass over chunks carrying dS
//      in MFMA accumulators; writes dV (final), dZ and dS' per chunk;
//   4. chunk_bwd_grad_kernel: one workgroup per chunk, all chunks in
//      parallel: dq, dk, dg, dbeta.
#include "kda_chunk_common.h"
#include "kda_internal.h"

namespace kda {
namespace {

// ---- reverse state scan -----------------------------------------------------
// One workgroup per (head, 16 NCW value columns), eight waves: 8 - NCW loader
// waves copy the next (lower) chunk's operand block global -> LDS with 16-byte
// LDS-destination loads and write dO^T of the value slice next to it; NCW
// consumer waves each hold a 128 x 16 slice of dS in accumulators.  The
// contraction operands that are products of the previous step stay in
// registers (accumulator tiles packed in pairs as B operands); the block's
// operands are read as 16-byte A units (WSB_* in kda_chunk_common.h), and the
// zero pairs of the upper triangular Aqk^T and Tm^T are skipped.
template <int NCW> struct BScanCfg {
    static constexpr int DV = 16 * NCW;
    static constexpr int NLW = 8 - NCW;
    static constexpr int NT = 512;
    static constexpr int OFF_DOT = 0;                       // dO^T [DV][64], swizzled (dot_at)
    static constexpr int OFF_BLK = DV * C * 2;
    static constexpr int STAGE = OFF_BLK + WSB_CHUNK;
    static constexpr int TOTAL = 2 * STAGE;
    static constexpr int VG = DV / 8;                       // 16-byte units per token row
    static constexpr int VPL = (C * VG + 255) / 256;        // dO units per lane of the first four waves
    static_assert(TOTAL <= 160 * 1024, "LDS budget");
    static_assert(NLW >= 4, "the first four waves are loaders");
};
// Element (value column j, token r) of the dO^T tile: rows of 64 tokens with
// no padding, their 8-token blocks XOR-permuted by the low bits of j, so that
// the consumers' reads of 4 tokens from 16 consecutive rows hit distinct banks.
__device__ __forceinline__ int dot_at(int j, int r) { return j * C + ((((r >> 3) ^ (j & 7))) << 3) + (r & 7); }
constexpr int BS_KIB = WSB_CHUNK / 1024;

template <int NCW>
__global__ void __launch_bounds__(512)
chunk_bwd_scan_kernel(const char* wsb, const bf16_t* dO, const float* dST, bf16_t* dv, float* dS0,
                      bf16_t* svdS, bf16_t* svdZ, int T, int H)
{
    using SC = BScanCfg<NCW>;
    __shared__ __attribute__((aligned(1024))) char smem[SC::TOTAL];

    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const bool loader = wave < SC::NLW;
    const int ln = lane & 15, lg = lane >> 4;
    const int cw = wave - SC::NLW;
    constexpr int nsplit = DK / SC::DV;
    const int nchunks = (T + C - 1) / C;
    const int nwg = gridDim.x, w = blockIdx.x;
    const int lid = (nwg % 8 == 0) ? (w % 8) * (nwg / 8) + w / 8 : w;   // slices of a head on one XCD
    const int head = lid / nsplit, slice = lid % nsplit;
    const int b = head / H, h = head % H;
    const int j0 = slice * SC::DV;
    const size_t tokstride = (size_t)H * DK;
    const size_t hbase = ((size_t)b * T * H + h) * DK;
    const size_t sbase = (size_t)head * DK * DK;
    const char* wsh = wsb + (size_t)head * nchunks * WSB_CHUNK;

    // ---- loader side: lane pt moves dO unit (token ut, columns 8 ug ..)
    const int pt = t & 255;
    bf16x8 drow[SC::VPL];                     // unit i of a lane: pt + 256 i
    auto load_block = [&](int n) {
        const char* src = wsh + (size_t)n * WSB_CHUNK;
        char* dst = smem + (n & 1) * SC::STAGE + SC::OFF_BLK;
        for (int u = wave; u < BS_KIB; u += SC::NLW)
            __builtin_amdgcn_global_load_lds(src + (size_t)u * 1024 + lane * 16,
                                             (__attribute__((address_space(3))) void*)(dst + u * 1024), 16, 0, 0);
    };
    auto load_do = [&](int n) {
        if (t >= 256) return;
#pragma unroll
        for (int i = 0; i < SC::VPL; ++i) {
            const int u = pt + 256 * i, ut = u / SC::VG, ug = u % SC::VG;
            if (ut >= C) continue;
            const int tok = min(n * C + ut, T - 1);
            drow[i] = *reinterpret_cast<const bf16x8*>(dO + hbase + (size_t)tok * tokstride + j0 + 8 * ug);
        }
    };
    auto write_dot = [&](int n) {             // dO^T of chunk n into stage n % 2 (zero past T)
        bf16_t* dt = reinterpret_cast<bf16_t*>(smem + (n & 1) * SC::STAGE + SC::OFF_DOT);
        if (t >= 256) return;
#pragma unroll
        for (int i = 0; i < SC::VPL; ++i) {
            const int u = pt + 256 * i, ut = u / SC::VG, ug = u % SC::VG;
            if (ut >= C) continue;
            const bool ok = n * C + ut < T;
#pragma unroll
            for (int c = 0; c < 8; ++c) dt[dot_at(8 * ug + c, ut)] = ok ? drow[i][c] : bf16_t{};
        }
    };

    // ---- consumer side: dS[16cb + 4lg + e][j0 + jc] in acc_s[cb][e]
    const int jc = 16 * cw + ln;
    f32x4 acc_s[8];
    if (!loader) {
#pragma unroll
        for (int cb = 0; cb < 8; ++cb)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                acc_s[cb][e] = dST ? dST[sbase + (size_t)(16 * cb + 4 * lg + e) * DK + j0 + jc] : 0.f;
    } else {
        load_block(nchunks - 1);
        load_do(nchunks - 1);
        __builtin_amdgcn_s_waitcnt(0);
        write_dot(nchunks - 1);
    }
    lds_barrier();

    for (int n = nchunks - 1; n >= 0; --n) {
        if (loader) {
            if (n > 0) { load_block(n - 1); load_do(n - 1); }
            __builtin_amdgcn_s_waitcnt(0);    // the stage must be complete at the barrier
            if (n > 0) write_dot(n - 1);
        } else {
            const char* st = smem + (n & 1) * SC::STAGE;
            const char* blk = st + SC::OFF_BLK;
            const bf16_t* sdOT = reinterpret_cast<const bf16_t*>(st + SC::OFF_DOT);
            // A operands from the block (layout WSB_* in kda_chunk_common.h):
            // pair p of row block Rb of the upper triangular Aqk^T, Tm^T, and
            // unit 4p + lg of a row of Qt^T, Kh^T, Kt
            auto tri_up = [&](int mat, int Rb, int p) {
                const char* q = blk + mat + wsb_pair_off(Rb, p);
                if (wsb_pair_full(Rb, p)) return *reinterpret_cast<const bf16x8*>(q + 16 * (4 * ln + lg));
                return cat8(bf16x4{}, *reinterpret_cast<const bf16x4*>(q + 8 * (4 * ln + lg)));
            };
            const bf16_t* sQtT = reinterpret_cast<const bf16_t*>(blk + WSB_QTT);
            const bf16_t* sKhT = reinterpret_cast<const bf16_t*>(blk + WSB_KHT);
            const bf16_t* sKt = reinterpret_cast<const bf16_t*>(blk + WSB_KT);
            const float* sGam = reinterpret_cast<const float*>(blk + WSB_GAM);
            const float* sBeta = reinterpret_cast<const float*>(blk + WSB_BETA);
            const size_t cidx = (size_t)head * nchunks + n;

            // Outputs of this step: dS' (the gradient of the state the chunk
            // hands on, i.e. acc_s before the update), dZ and dV.  Neighbouring
            // lanes pair up so that each store is a 4-byte column pair (see
            // pair_rows_bf16).  The stores are issued at the end of the step:
            // issued at its start they queue behind the loader waves' block
            // copy and hold up the dependent MFMA chain.
            const int prow = 4 * lg + 2 * (ln & 1), pcol = j0 + 16 * cw + (ln & ~1);

            bf16x8 sb[4], dob[2];
#pragma unroll
            for (int p = 0; p < 4; ++p) sb[p] = cat8(to_bf16x4(acc_s[2 * p]), to_bf16x4(acc_s[2 * p + 1]));
#pragma unroll
            for (int p = 0; p < 2; ++p)
                dob[p] = cat8(ld4(sdOT + dot_at(jc, 32 * p + 4 * lg)),
                              ld4(sdOT + dot_at(jc, 32 * p + 16 + 4 * lg)));

            // dVn = Aqk^T dO + Kt dS'
            f32x4 dvn[4];
#pragma unroll
            for (int Rb = 0; Rb < 4; ++Rb) {
                f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int p = 0; p < 2; ++p)
                    if (!wsb_pair_zero(Rb, p))
                        a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tri_up(WSB_AQKT, Rb, p), dob[p], a, 0, 0, 0);
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const bf16x8 k8 = *reinterpret_cast<const bf16x8*>(sKt + wsk_tok_unit(16 * Rb + ln, 4 * p + lg));
                    a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k8, sb[p], a, 0, 0, 0);
                }
                dvn[Rb] = a;
            }

            // dZ = Tm^T dVn, dV = Diag(beta) dZ
            bf16x8 vb[2];
#pragma unroll
            for (int p = 0; p < 2; ++p) vb[p] = cat8(to_bf16x4(dvn[2 * p]), to_bf16x4(dvn[2 * p + 1]));
            f32x4 dvv[4];
            bf16x2 zp[4][2], dp[4][2];
#pragma unroll
            for (int Rb = 0; Rb < 4; ++Rb) {
                f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int p = 0; p < 2; ++p)
                    if (!wsb_pair_zero(Rb, p))
                        a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tri_up(WSB_TMT, Rb, p), vb[p], a, 0, 0, 0);
#pragma unroll
                for (int e = 0; e < 4; ++e) dvv[Rb][e] = sBeta[16 * Rb + 4 * lg + e] * a[e];
                pair_rows_bf16(a, lane, zp[Rb][0], zp[Rb][1]);
                pair_rows_bf16(dvv[Rb], lane, dp[Rb][0], dp[Rb][1]);
            }

            bf16x2 sp[8][2];                     // dS', stored after the update
#pragma unroll
            for (int cb = 0; cb < 8; ++cb) pair_rows_bf16(acc_s[cb], lane, sp[cb][0], sp[cb][1]);
            // dS <- Diag(gamma) dS' + Qt^T dO - Kh^T dV
            bf16x8 nb[2];
#pragma unroll
            for (int p = 0; p < 2; ++p) nb[p] = cat8(to_bf16x4(-dvv[2 * p]), to_bf16x4(-dvv[2 * p + 1]));
#pragma unroll
            for (int cb = 0; cb < 8; ++cb) {
                const f32x4 gv = *reinterpret_cast<const f32x4*>(sGam + 16 * cb + 4 * lg);
                f32x4 a = acc_s[cb] * gv;
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    const int u = wsk_kbt_unit(16 * cb + ln, 4 * p + lg);
                    a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8*>(sQtT + u), dob[p], a, 0, 0, 0);
                    a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8*>(sKhT + u), nb[p], a, 0, 0, 0);
                }
                acc_s[cb] = a;
            }
#pragma unroll
            for (int cb = 0; cb < 8; ++cb) {
                *reinterpret_cast<bf16x2*>(svdS + sv_at(cidx, DK, 16 * cb + prow, pcol)) = sp[cb][0];
                *reinterpret_cast<bf16x2*>(svdS + sv_at(cidx, DK, 16 * cb + prow + 1, pcol)) = sp[cb][1];
            }
#pragma unroll
            for (int Rb = 0; Rb < 4; ++Rb) {
                const int r0 = 16 * Rb + prow, tok = n * C + r0;
                *reinterpret_cast<bf16x2*>(svdZ + sv_at(cidx, C, r0, pcol)) = zp[Rb][0];
                *reinterpret_cast<bf16x2*>(svdZ + sv_at(cidx, C, r0 + 1, pcol)) = zp[Rb][1];
                if (tok < T) *reinterpret_cast<bf16x2*>(dv + hbase + (size_t)tok * tokstride + pcol) = dp[Rb][0];
                if (tok + 1 < T) *reinterpret_cast<bf16x2*>(dv + hbase + (size_t)(tok + 1) * tokstride + pcol) = dp[Rb][1];
            }
        }
        lds_barrier();
    }

    if (!loader && dS0) {
#pragma unroll
        for (int cb = 0; cb < 8; ++cb)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                dS0[sbase + (size_t)(16 * cb + 4 * lg + e) * DK + j0 + jc] = acc_s[cb][e];
    }
}

// ---- per-chunk gradients -------------------------------------------------------
// One workgroup (eight waves) per (head, chunk).  Wave w owns key channels
// 16w .. 16w+15 for all 64 tokens, lane (lg, ln) the channel 16w + ln and rows
// 16m + 4lg + e (m, e = 0..3): the layout of a 16 x 16 MFMA output tile, so the
// decay computed first and the gradient tiles accumulated last line up in
// registers.
//
// Every global read is issued at the start: q, k and g go global -> LDS with
// 16-byte LDS-destination loads, the rest into registers (the dO and Vn tiles
// that are then parked in LDS, the dZ rows of the wave's C x C tiles as A
// fragments, the Y and dZ values of the first dbeta term, the S and dS' rows
// of its channel block as B fragments), in the order the phases consume them;
// -dV = -Diag(beta) dZ is formed from the dZ values.  LDS regions are reused
// phase by phase:
//   A  : g staging (fp32) -> Kh, Kb -> dV -> dq, dk staging
//   B  : Qt^T, Kh^T, Kb^T -> dg staging (fp32)
//   CR : q, k staging -> dAqk, dAqk^T, dA', dA'^T
//   DO, VN: dO and Vn tiles for both product phases.
struct GradLds {
    static constexpr int P64 = C + 8, P128 = DK + 8;
    static constexpr int T128 = C * P128 * 2;                 // one [64][136] bf16 tile
    static constexpr int T64 = C * P64 * 2;                   // one [64][72] bf16 tile
    static constexpr int OFF_A = 0;
    static constexpr int OFF_KB = OFF_A + T128;
    static constexpr int OFF_B = OFF_A + 2 * T128;
    static constexpr int OFF_KHT = OFF_B + DK * P64 * 2;
    static constexpr int OFF_KBT = OFF_KHT + DK * P64 * 2;
    static constexpr int OFF_CR = OFF_KBT + DK * P64 * 2;
    static constexpr int OFF_DAQKT = OFF_CR + T64;
    static constexpr int OFF_DAP = OFF_DAQKT + T64;
    static constexpr int OFF_DAPT = OFF_DAP + T64;
    static constexpr int OFF_DO = OFF_DAPT + T64;
    static constexpr int OFF_VN = OFF_DO + T128;
    static constexpr int OFF_BETA = OFF_VN + T128;            // beta [64] fp32
    static constexpr int OFF_DB = OFF_BETA + C * 4;           // dbeta [64] fp32
    static constexpr int OFF_F = OFF_DB + C * 4;              // F [6 block pairs][128] bf16
    static constexpr int TOTAL = OFF_F + 6 * DK * 2;
    static_assert(TOTAL <= 160 * 1024, "LDS budget");
    static_assert(2 * T128 >= C * DK * 4, "g staging fits in region A");
    static_assert(4 * T64 >= 2 * C * DK * 2, "q, k staging fits in region CR");
    static_assert(OFF_CR - OFF_B >= C * DK * 4, "dg staging fits in region B");
};

__device__ __forceinline__ bf16x8 ld8(const bf16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ void dma16(const void* g, char* lds) {
    __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}

// GATE: GATE_CHANNEL (g and dg [B, T, H, 128]), GATE_HEAD (g and dg [B, T, H]:
// the per-channel gradient summed over the head's channels, since the one decay
// enters every channel) or GATE_NONE (g = 0, dg not written).
template <int GATE>
__global__ void __launch_bounds__(512)
chunk_bwd_grad_kernel(const bf16_t* q, const bf16_t* k, const float* g, const bf16_t* beta,
                      const bf16_t* dO, const bf16_t* svS, const bf16_t* svdS,
                      const bf16_t* svY, const bf16_t* svVn, const bf16_t* svdZ,
                      bf16_t* dq, bf16_t* dk, float* dg, bf16_t* dbeta, int T, int H)
{
    using L = GradLds;
    __shared__ __attribute__((aligned(1024))) char smem[L::TOTAL];
    bf16_t* sKh = reinterpret_cast<bf16_t*>(smem + L::OFF_A);
    bf16_t* sKb = reinterpret_cast<bf16_t*>(smem + L::OFF_KB);
    bf16_t* sDV = reinterpret_cast<bf16_t*>(smem + L::OFF_A);
    bf16_t* sQtT = reinterpret_cast<bf16_t*>(smem + L::OFF_B);
    bf16_t* sKhT = reinterpret_cast<bf16_t*>(smem + L::OFF_KHT);
    bf16_t* sKbT = reinterpret_cast<bf16_t*>(smem + L::OFF_KBT);
    bf16_t* sdAqk = reinterpret_cast<bf16_t*>(smem + L::OFF_CR);
    bf16_t* sdAqkT = reinterpret_cast<bf16_t*>(smem + L::OFF_DAQKT);
    bf16_t* sdAp = reinterpret_cast<bf16_t*>(smem + L::OFF_DAP);
    bf16_t* sdApT = reinterpret_cast<bf16_t*>(smem + L::OFF_DAPT);
    bf16_t* sDO = reinterpret_cast<bf16_t*>(smem + L::OFF_DO);
    bf16_t* sVN = reinterpret_cast<bf16_t*>(smem + L::OFF_VN);
    float* sbeta = reinterpret_cast<float*>(smem + L::OFF_BETA);
    float* sdb = reinterpret_cast<float*>(smem + L::OFF_DB);
    bf16_t* sF = reinterpret_cast<bf16_t*>(smem + L::OFF_F);
    // staging, unpadded row-major [64][128]
    const float* stG = reinterpret_cast<const float*>(smem + L::OFF_A);
    const bf16_t* stQ = reinterpret_cast<const bf16_t*>(smem + L::OFF_CR);
    const bf16_t* stK = stQ + C * DK;

    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int ln = lane & 15, lg = lane >> 4;
    const int nchunks = (T + C - 1) / C;
    const int head = blockIdx.x / nchunks, n = blockIdx.x % nchunks;
    const int b = head / H, h = head % H;
    const size_t tokstride = (size_t)H * DK;
    const size_t hbase = ((size_t)b * T * H + h) * DK;
    const size_t cidx = (size_t)head * nchunks + n;
    const int tok0 = n * C;
    const int c = 16 * wave + ln;                 // this lane's key channel
    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};

    // ===== issue every global read =====
    for (int u = wave; u < 32; u += 8) {          // q, k: 16 rows of 1 KiB each = 4 tokens
        const bf16_t* src = u < 16 ? q : k;
        const int row = 4 * (u & 15) + (lane >> 4);
        dma16(src + hbase + (size_t)min(tok0 + row, T - 1) * tokstride + 8 * (lane & 15),
              smem + L::OFF_CR + u * 1024);
    }
    if constexpr (GATE == GATE_CHANNEL) {
        for (int u = wave; u < 32; u += 8) {      // g: 1 KiB = 2 tokens
            const int row = 2 * u + (lane >> 5);
            dma16(g + hbase + (size_t)min(tok0 + row, T - 1) * tokstride + 4 * (lane & 31),
                  smem + L::OFF_A + u * 1024);
        }
    }
    float gh[4][4];                                // GATE_HEAD: this lane's rows' decays
    if constexpr (GATE == GATE_HEAD) {
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                gh[m][e] = g[((size_t)b * T + min(tok0 + 16 * m + 4 * lg + e, T - 1)) * H + h];
    }
    // row r = t / 8, columns 16 (t % 8) .. +15 of the 64 x 128 value-side tiles
    const int vr = t >> 3, vc = 16 * (t & 7);
    const bool vok = tok0 + vr < T;
    const size_t vat = hbase + (size_t)min(tok0 + vr, T - 1) * tokstride + vc;
    // Register loads in the order they are consumed (dO and Vn are parked in
    // LDS after the decay phase, dZ and Y feed the C x C products, S and dS'
    // the C x d_k products); dV is not read: it is Diag(beta) dZ.
    __builtin_amdgcn_sched_barrier(0);            // keep them behind the LDS-destination loads
    bf16x8 yv[2], zv[2], dov[2], vnv[2];
    const bf16_t betr = beta[((size_t)b * T + min(tok0 + (t & 63), T - 1)) * H + h];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        dov[i] = ld8(dO + vat + 8 * i);
        vnv[i] = ld8(svVn + sv_at(cidx, C, vr, vc + 8 * i));
    }
    // C x C tiles (mb, nb) = (wave / 2, 2 (wave % 2) + j), j = 0, 1: both of a
    // wave's tiles in one row block, so its dZ rows are loaded once (the tiles
    // above the diagonal are zero and skipped; their wave still loads the rows,
    // so the count is fixed)
    const int mbw = wave >> 1;
    bf16x8 dzf[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) dzf[s] = ld8(svdZ + sv_at(cidx, C, 16 * mbw + ln, 32 * s + 8 * lg));
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const size_t wat = sv_at(cidx, C, vr, vc + 8 * i);
        yv[i] = ld8(svY + wat);
        zv[i] = ld8(svdZ + wat);
    }
    bf16x8 sf[4], dsf[4];                          // S, dS' rows c as B fragments
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        sf[s] = ld8(svS + sv_at(cidx, DK, c, 32 * s + 8 * lg));
        dsf[s] = ld8(svdS + sv_at(cidx, DK, c, 32 * s + 8 * lg));
    }
    if (!vok) { dov[0] = bf16x8{}; dov[1] = bf16x8{}; }
    // The loads return in issue order: once at most the 16 register loads
    // issued after beta, dO and Vn are outstanding, the LDS-destination loads
    // are complete (vmcnt 16, no wait on the other counters).  The rest
    // arrive while the decay phase and the C x C products run.
    wait_vmcnt<16>();
    lds_barrier();

    // ===== decay and the decay-scaled keys / queries =====
    float G[4][4], qv[4][4], kv[4][4];
    float carry = 0.f;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        float s4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 16 * m + 4 * lg + e;
            const bool ok = tok0 + r < T;
            // (the staged rows past T hold the clamped last token: read, then mask)
            float gl = 0.f;
            if constexpr (GATE == GATE_CHANNEL) gl = stG[r * DK + c] * LOG2E;
            else if constexpr (GATE == GATE_HEAD) gl = gh[m][e] * LOG2E;
            const float qr = (float)stQ[r * DK + c], kr = (float)stK[r * DK + c];
            gl = ok ? gl : 0.f;
            qv[m][e] = ok ? qr : 0.f;
            kv[m][e] = ok ? kr : 0.f;
            s4[e] = (e ? s4[e - 1] : 0.f) + gl;
        }
        float bs[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) bs[j] = __shfl(s4[3], ln + 16 * j);
        const float excl = (lg > 0 ? bs[0] : 0.f) + (lg > 1 ? bs[1] : 0.f) + (lg > 2 ? bs[2] : 0.f);
#pragma unroll
        for (int e = 0; e < 4; ++e) G[m][e] = carry + excl + s4[e];   // log2 units
        carry += bs[0] + bs[1] + bs[2] + bs[3];
    }
    const float Gc = carry;
    // Sub-chunk boundaries of this lane's channel: Bv[j] = G at the end of
    // sub-chunk j - 1 (16-token blocks; Bv[0] = 0, Bv[4] = G_64).  Every
    // decay factor below is referenced to one of them, so that none grows
    // with the chunk's total decay (only with one sub-chunk's).
    float Bv[5];
    Bv[0] = 0.f;
#pragma unroll
    for (int m = 0; m < 4; ++m) Bv[m + 1] = __shfl(G[m][3], ln + 48);
    // A wave whose 16 channels all keep their chunk decay within 2^-96 takes
    // every reference at the chunk start instead (Bv = 0: the factors below
    // reduce to 2^{G}, 2^{-G} and 1), which skips the per-block rescaling of
    // the token contractions; the choice is per wave, the formulas the same.
    const bool fastw = __builtin_amdgcn_ballot_w64(Gc < -96.f) == 0;
    if (fastw) {
#pragma unroll
        for (int j = 0; j < 5; ++j) Bv[j] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        *reinterpret_cast<bf16x8*>(sDO + vr * L::P128 + vc + 8 * i) = dov[i];
        *reinterpret_cast<bf16x8*>(sVN + vr * L::P128 + vc + 8 * i) = vnv[i];
    }
    lds_barrier();                                 // staging reads done before A and CR are reused
    // row r of block m:  Ke = 2^{G_r - B_{m+1}} k (>= 1), Kend = 2^{B_{m+1} - G_r} k (<= 1)
    // token-major for K K^T; Qs = 2^{G_r - B_m} q, Ks = 2^{G_r - B_m} k (<= 1) and
    // Kend transposed for the token contractions
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        f32x4 qs, ks, kend;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float ea = __builtin_amdgcn_exp2f(G[m][e] - Bv[m + 1]);
            const float eai = __builtin_amdgcn_exp2f(Bv[m + 1] - G[m][e]);
            const float esi = __builtin_amdgcn_exp2f(G[m][e] - Bv[m]);
            qs[e] = esi * qv[m][e]; ks[e] = esi * kv[m][e]; kend[e] = eai * kv[m][e];
            const int r = 16 * m + 4 * lg + e;
            sKh[r * L::P128 + c] = (bf16_t)(ea * kv[m][e]);
            sKb[r * L::P128 + c] = (bf16_t)kend[e];
        }
        store_vec4<bf16_t>(sQtT + c * L::P64 + 16 * m + 4 * lg, qs);
        store_vec4<bf16_t>(sKhT + c * L::P64 + 16 * m + 4 * lg, ks);
        store_vec4<bf16_t>(sKbT + c * L::P64 + 16 * m + 4 * lg, kend);
    }
    if (lg == 0) {
        // F[R, I] = 2^{B_{R+1} - B_{I+1}} (<= 1) for block pairs R > I, index R (R - 1) / 2 + I
#pragma unroll
        for (int R = 1; R < 4; ++R)
#pragma unroll
            for (int I = 0; I < R; ++I)
                sF[(R * (R - 1) / 2 + I) * DK + c] = (bf16_t)__builtin_amdgcn_exp2f(Bv[R + 1] - Bv[I + 1]);
    }
    if (t < C) {
        const int tok = tok0 + t;
        sbeta[t] = tok < T ? (float)betr : 0.f;
        sdb[t] = 0.f;
    }
    lds_barrier();

    // ===== C x C products: KK = Kh Kb^T, M1 = dZ Vn^T, M2 = dO Vn^T =====
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int mb = mbw, nb = 2 * (wave & 1) + j;
        const int r0 = 16 * mb + 4 * lg, i = 16 * nb + ln;
        if (nb > mb) {
#pragma unroll
            for (int e = 0; e < 4; ++e) { sdAqk[(r0 + e) * L::P64 + i] = bf16_t{}; sdAp[(r0 + e) * L::P64 + i] = bf16_t{}; }
            store_vec4<bf16_t>(sdAqkT + i * L::P64 + r0, z4);
            store_vec4<bf16_t>(sdApT + i * L::P64 + r0, z4);
            continue;
        }
        const int ra = 16 * mb + ln, rb = 16 * nb + ln;
        f32x4 kk = z4, m1 = z4, m2 = z4;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int ko = 32 * s + 8 * lg;
            const bf16x8 vnf = ld8(sVN + rb * L::P128 + ko);
            // (K K^T)[r, i] = sum_c Ke_r Kend_i F[mb, nb] over the channels c
            bf16x8 kbf = ld8(sKb + rb * L::P128 + ko);
            if (nb < mb) {
                const bf16x8 f = ld8(sF + (mb * (mb - 1) / 2 + nb) * DK + ko);
#pragma unroll
                for (int x = 0; x < 8; ++x) kbf[x] = (bf16_t)((float)kbf[x] * (float)f[x]);
            }
            kk = mma(ld8(sKh + ra * L::P128 + ko), kbf, kk);
            m1 = mma(dzf[s], vnf, m1);
            m2 = mma(ld8(sDO + ra * L::P128 + ko), vnf, m2);
        }
        f32x4 aq, ap;
        float part[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = r0 + e;
            aq[e] = (i <= r) ? m2[e] : 0.f;
            const float dakk = (i < r) ? -m1[e] : 0.f;
            ap[e] = sbeta[r] * dakk;
            part[e] = dakk * kk[e];
            sdAqk[r * L::P64 + i] = (bf16_t)aq[e];
            sdAp[r * L::P64 + i] = (bf16_t)ap[e];
        }
        store_vec4<bf16_t>(sdAqkT + i * L::P64 + r0, aq);
        store_vec4<bf16_t>(sdApT + i * L::P64 + r0, ap);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
#pragma unroll
            for (int off = 1; off < 16; off <<= 1) part[e] += __shfl_xor(part[e], off);
        }
        if (ln == 0) {
#pragma unroll
            for (int e = 0; e < 4; ++e) atomicAdd(&sdb[r0 + e], part[e]);
        }
    }
    {   // dbeta, first term: sum over value columns of (V - Kh S) * dZ
        float d = 0.f;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int x = 0; x < 8; ++x) d += (float)yv[i][x] * (float)zv[i][x];
        d += __shfl_xor(d, 1);
        d += __shfl_xor(d, 2);
        d += __shfl_xor(d, 4);
        if ((t & 7) == 0) atomicAdd(&sdb[vr], d);
    }
    lds_barrier();                                 // Kh, Kb dead; dA tiles and dbeta complete
    if (t < C && tok0 + t < T) dbeta[((size_t)b * T + tok0 + t) * H + h] = (bf16_t)sdb[t];
#pragma unroll
    for (int i = 0; i < 2; ++i) {                  // -dV = -Diag(beta) dZ
        bf16x8 dvn;
        const float nb = -sbeta[vr];
#pragma unroll
        for (int x = 0; x < 8; ++x) dvn[x] = (bf16_t)(nb * (float)zv[i][x]);
        *reinterpret_cast<bf16x8*>(sDV + vr * L::P128 + vc + 8 * i) = dvn;
    }
    lds_barrier();

    // ===== C x d_k products: wave w -> channel block w, token blocks m = 0..3 =====
    f32x4 aQ[4], aH[4], aB[4], aT[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) { aQ[m] = z4; aH[m] = z4; aB[m] = z4; aT[m] = z4; }
    float sds = 0.f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {                  // contraction over value columns
        const int ko = 32 * s + 8 * lg;
#pragma unroll
        for (int i = 0; i < 8; ++i) sds += (float)sf[s][i] * (float)dsf[s][i];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int ar = (16 * m + ln) * L::P128 + ko;
            aQ[m] = mma(ld8(sDO + ar), sf[s], aQ[m]);
            aH[m] = mma(ld8(sDV + ar), sf[s], aH[m]);     // sDV holds -dV
            aT[m] = mma(ld8(sVN + ar), dsf[s], aT[m]);
        }
    }
    // dQt and dKh of rows in block m are carried relative to B_{m+1}: the
    // state terms (dO S^T, -dV S^T, whose own factor is 2^{G_r}) times
    // 2^{B_{m+1}} (<= 1) here, the in-chunk terms below against keys
    // referenced to B_{m+1}
    if (!fastw) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const float f = __builtin_amdgcn_exp2f(Bv[m + 1]);
#pragma unroll
            for (int e = 0; e < 4; ++e) { aQ[m][e] *= f; aH[m][e] *= f; }
        }
    }
    auto scale8 = [](bf16x8 x, float f) {
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = (bf16_t)((float)x[i] * f);
        return x;
    };
#pragma unroll
    for (int s = 0; s < 2; ++s) {                  // contraction over tokens
        const int ko = 32 * s + 8 * lg;
        const int tb = 2 * s + (lg >> 1);          // 16-token block of this lane's 8 tokens
        const bf16x8 kbt = ld8(sKbT + c * L::P64 + ko);
        const bf16x8 qtt = ld8(sQtT + c * L::P64 + ko);
        const bf16x8 kht = ld8(sKhT + c * L::P64 + ko);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int ar = (16 * m + ln) * L::P64 + ko;
            // rows of block m against keys of block tb <= m: Kend (ref B_{tb+1})
            // times 2^{B_{m+1} - B_{tb+1}}; blocks tb > m are zero in dAqk, dA'
            // (on a fast wave every factor is 1 and nothing is rescaled)
            bf16x8 kq = kbt;
            if (!fastw && tb != m) kq = scale8(kbt, tb < m ? __builtin_amdgcn_exp2f(Bv[m + 1] - Bv[tb + 1]) : 0.f);
            aQ[m] = mma(ld8(sdAqk + ar), kq, aQ[m]);
            aH[m] = mma(ld8(sdAp + ar), kq, aH[m]);
            // keys of block m against rows of block tb >= m: Qs, Ks (ref B_tb)
            // times 2^{B_tb - B_m}; blocks tb < m are zero in dAqk^T, dA'^T
            bf16x8 qq = qtt, kk2 = kht;
            if (!fastw && tb != m) {
                const float fb = tb > m ? __builtin_amdgcn_exp2f(Bv[tb] - Bv[m]) : 0.f;
                qq = scale8(qtt, fb);
                kk2 = scale8(kht, fb);
            }
            aB[m] = mma(ld8(sdAqkT + ar), qq, aB[m]);
            aB[m] = mma(ld8(sdApT + ar), kk2, aB[m]);
        }
    }

    // ===== chain rule to q, k, g; results staged in LDS, stored 16 bytes at a time =====
    sds += __shfl_xor(sds, 16);
    sds += __shfl_xor(sds, 32);
    float dG[4][4], ktp = 0.f;
    f32x4 oq[4], ok_[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            // dQt, dKh relative to B_{m+1}; dKb relative to B_m (keys of block m)
            const float ea = __builtin_amdgcn_exp2f(G[m][e] - Bv[m + 1]);
            const float es = __builtin_amdgcn_exp2f(Bv[m] - G[m][e]);
            const float et = __builtin_amdgcn_exp2f(Gc - G[m][e]);
            const float dqt = aQ[m][e], dkh = aH[m][e], dkb = aB[m][e], dkt = aT[m][e];
            dG[m][e] = qv[m][e] * ea * dqt + kv[m][e] * (ea * dkh - es * dkb - et * dkt);
            ktp += kv[m][e] * et * dkt;
            oq[m][e] = ea * dqt;
            ok_[m][e] = ea * dkh + es * dkb + et * dkt;
        }
    }
    ktp += __shfl_xor(ktp, 16);
    ktp += __shfl_xor(ktp, 32);
    // dg_r = sum over rows r' >= r of dG, plus the gradient of G_64 (which every
    // row's g enters)
    float dgo[4][4];
    float acc = __builtin_amdgcn_exp2f(Gc) * sds + ktp;
#pragma unroll
    for (int m = 3; m >= 0; --m) {
        float sfx[4];
        sfx[3] = dG[m][3];
#pragma unroll
        for (int e = 2; e >= 0; --e) sfx[e] = sfx[e + 1] + dG[m][e];
        float bs[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) bs[j] = __shfl(sfx[0], ln + 16 * j);
        const float excl = (lg < 3 ? bs[3] : 0.f) + (lg < 2 ? bs[2] : 0.f) + (lg < 1 ? bs[1] : 0.f);
#pragma unroll
        for (int e = 0; e < 4; ++e) dgo[m][e] = acc + excl + sfx[e];
        acc += bs[0] + bs[1] + bs[2] + bs[3];
    }
    lds_barrier();                                 // regions A and B no longer read
    bf16_t* stDQ = reinterpret_cast<bf16_t*>(smem + L::OFF_A);
    bf16_t* stDK = stDQ + C * DK;
    float* stDG = reinterpret_cast<float*>(smem + L::OFF_B);
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 16 * m + 4 * lg + e;
            stDQ[r * DK + c] = (bf16_t)oq[m][e];
            stDK[r * DK + c] = (bf16_t)ok_[m][e];
            if constexpr (GATE != GATE_NONE) stDG[r * DK + c] = dgo[m][e];
        }
    lds_barrier();
    if (vok) {
        const size_t at = hbase + (size_t)(tok0 + vr) * tokstride + vc;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            *reinterpret_cast<bf16x8*>(dq + at + 8 * i) = ld8(stDQ + vr * DK + vc + 8 * i);
            *reinterpret_cast<bf16x8*>(dk + at + 8 * i) = ld8(stDK + vr * DK + vc + 8 * i);
        }
        if constexpr (GATE == GATE_CHANNEL) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *reinterpret_cast<f32x4*>(dg + at + 4 * i) = *reinterpret_cast<const f32x4*>(stDG + vr * DK + vc + 4 * i);
        }
    }
    if constexpr (GATE == GATE_HEAD) {
        // row vr's 128 channels: 16 per lane, then over the 8 lanes t % 8
        // (every lane takes part in the shuffles, valid row or not)
        float d = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) d += stDG[vr * DK + vc + i];
        d += __shfl_xor(d, 1);
        d += __shfl_xor(d, 2);
        d += __shfl_xor(d, 4);
        if (vok && (t & 7) == 0) dg[((size_t)b * T + tok0 + vr) * H + h] = d;
    }
}

}  // namespace

size_t chunk_bwd_ws_layout(long long B, long long T, long long H, size_t* off)
{
    const size_t units = (size_t)B * (size_t)H * (size_t)((T + C - 1) / C);   // (head, chunk) pairs
    size_t o[KDA_BWD_WS_REGIONS + 1];
    o[KDA_BWD_WS_FWD] = 0;
    o[KDA_BWD_WS_BWD] = chunk_ws_bytes(B, T, H);
    o[KDA_BWD_WS_S] = o[KDA_BWD_WS_BWD] + units * WSB_CHUNK;
    o[KDA_BWD_WS_DS] = o[KDA_BWD_WS_S] + units * DK * DK * 2;
    o[KDA_BWD_WS_Y] = o[KDA_BWD_WS_DS] + units * DK * DK * 2;
    o[KDA_BWD_WS_VN] = o[KDA_BWD_WS_Y] + units * C * DK * 2;
    o[KDA_BWD_WS_DZ] = o[KDA_BWD_WS_VN] + units * C * DK * 2;
    o[KDA_BWD_WS_REGIONS] = o[KDA_BWD_WS_DZ] + units * C * DK * 2;
    if (off)
        for (int i = 0; i < KDA_BWD_WS_REGIONS; ++i) off[i] = o[i];
    return o[KDA_BWD_WS_REGIONS];
}

hipError_t launch_chunk_bwd(const void* q, const void* k, const void* v, const float* g,
                            const void* beta, const float* S0, const void* dO, const float* dST,
                            void* dq, void* dk, void* dv, float* dg, void* dbeta, float* dS0,
                            int B, int T, int H, char* ws, hipStream_t stream, int gate)
{
    const long long heads = (long long)B * H;
    const int nchunks = (T + C - 1) / C;
    size_t off[KDA_BWD_WS_REGIONS];
    chunk_bwd_ws_layout(B, T, H, off);
    bf16_t* svS = reinterpret_cast<bf16_t*>(ws + off[KDA_BWD_WS_S]);
    bf16_t* svdS = reinterpret_cast<bf16_t*>(ws + off[KDA_BWD_WS_DS]);
    bf16_t* svY = reinterpret_cast<bf16_t*>(ws + off[KDA_BWD_WS_Y]);
    bf16_t* svVn = reinterpret_cast<bf16_t*>(ws + off[KDA_BWD_WS_VN]);
    bf16_t* svdZ = reinterpret_cast<bf16_t*>(ws + off[KDA_BWD_WS_DZ]);
    char* wsb = ws + off[KDA_BWD_WS_BWD];

    hipError_t err = launch_bwd_forward_part(q, k, v, g, beta, S0, B, T, H, ws + off[KDA_BWD_WS_FWD],
                                             wsb, svS, svY, svVn, stream, gate);
    if (err != hipSuccess) return err;

    const int ncw = heads * 2 >= 256 ? 4 : heads * 4 >= 256 ? 2 : 1;   // one round of workgroups when possible
#define KDA_BSCAN(NCW) hipLaunchKernelGGL(chunk_bwd_scan_kernel<NCW>, dim3((unsigned)(heads * (DK / BScanCfg<NCW>::DV))), \
                                          dim3(512), 0, stream, (const char*)wsb, (const bf16_t*)dO, dST, (bf16_t*)dv, \
                                          dS0, svdS, svdZ, T, H)
    if (ncw == 4) KDA_BSCAN(4);
    else if (ncw == 2) KDA_BSCAN(2);
    else KDA_BSCAN(1);
#undef KDA_BSCAN

#define KDA_GRAD(GT) hipLaunchKernelGGL(chunk_bwd_grad_kernel<GT>, dim3((unsigned)(heads * nchunks)), dim3(512), 0, \
                                      stream, (const bf16_t*)q, (const bf16_t*)k, g, (const bf16_t*)beta,       \
                                      (const bf16_t*)dO, svS, svdS, svY, svVn, svdZ,                             \
                                      (bf16_t*)dq, (bf16_t*)dk, dg, (bf16_t*)dbeta, T, H)
    if (gate == GATE_HEAD) KDA_GRAD(GATE_HEAD);
    else if (gate == GATE_NONE) KDA_GRAD(GATE_NONE);
    else KDA_GRAD(GATE_CHANNEL);
#undef KDA_GRAD
    return hipGetLastError();
}

}  // namespace kda
