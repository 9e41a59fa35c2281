// kda_gemm.hip -- dense projections of the KDA token-mixing layer on gfx950.
//
// C[M, N] = A[M, K] * B[N, K]^T with both operands stored K-contiguous
// (activations [tokens, features], weights [out_features, in_features]),
// bf16 MFMA (v_mfma_f32_16x16x32_bf16) with fp32 accumulation.  These are the
// projections W_q, W_k, W_v, W_g, W_down, W_beta, W_up and W_o of the layer
// on page "Kimi K3论文：Kimi Linear", section 3.
//
// Tiling (general kernel): a 256-thread workgroup computes a 128 x 128 tile
// of C, each of its 4 waves a 64 x 64 sub-tile (4 x 4 MFMA tiles), over K in
// steps of 64.  Large bf16 products use the 256 x 256-tile kernel below.
// Operand tiles are staged through LDS (rows padded by 16 B against bank
// conflicts), double-buffered for bf16 A; the next K-step's global loads are
// in flight while the current step's MFMAs run.  The MFMA computes
// C^T tiles (weights as the first operand) so that each lane ends up holding
// 4 consecutive columns of one row of C, which it stores as one vector.
//
// Variants: A may be fp32 (AF32): each element is split into bf16 hi + lo
// parts (x = hi + lo to about 16 bits) and two MFMAs are issued, which keeps
// the low-rank gate path of the layer close to fp32 accuracy.  The epilogue
// may apply g = -softplus(c) (the decay gate log alpha = -softplus(.)).
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int GT = 256;                  // threads
constexpr int LDT = BK + 8;              // LDS row pitch (bf16 elements)

__device__ __forceinline__ void block_sync() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;

template <typename T> __device__ __forceinline__ void store_out4(T* p, f32x4 v, int nvalid);
template <> __device__ __forceinline__ void store_out4<float>(float* p, f32x4 v, int nvalid) {
    if (nvalid >= 4) { *reinterpret_cast<f32x4*>(p) = v; return; }
    for (int e = 0; e < nvalid; ++e) p[e] = v[e];
}
template <> __device__ __forceinline__ void store_out4<bf16_t>(bf16_t* p, f32x4 v, int nvalid) {
    if (nvalid >= 4) {
        bf16x4 b; b[0] = (bf16_t)v[0]; b[1] = (bf16_t)v[1]; b[2] = (bf16_t)v[2]; b[3] = (bf16_t)v[3];
        *reinterpret_cast<bf16x4*>(p) = b;
        return;
    }
    for (int e = 0; e < nvalid; ++e) p[e] = (bf16_t)v[e];
}

// -softplus(x) = -(max(x, 0) + log(1 + e^-|x|)), with hardware exp2/log2.
__device__ __forceinline__ float neg_softplus(float x) {
    const float e = __builtin_amdgcn_exp2f(-fabsf(x) * 1.4426950408889634f);
    return -(fmaxf(x, 0.f) + __builtin_amdgcn_logf(1.f + e) * 0.6931471805599453f);
}

template <bool AF32, typename OutT, int EPI>
__global__ void __launch_bounds__(GT)
gemm_nt_kernel(const void* A_, const bf16_t* B, OutT* C, int M, int N, int K,
               int lda, int ldb, int ldc, const bf16_t* B2, int n_split)
{
    constexpr int NA = AF32 ? 2 : 1;     // A planes in LDS (hi, lo)
    // LDS stages: two for bf16 A; one for fp32 A (its K is the small gate
    // rank), which halves the footprint to 55 KiB so two workgroups share a CU
    constexpr int NBUF = AF32 ? 1 : 2;
    __shared__ __attribute__((aligned(16))) bf16_t sA[NBUF][NA][BM * LDT];
    __shared__ __attribute__((aligned(16))) bf16_t sB[NBUF][BN * LDT];

    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int ln = lane & 15, lg = lane >> 4;
    const int wm = wave >> 1, wn = wave & 1;      // 64 x 64 sub-tile of the wave

    // tile order: consecutive workgroups walk down M for a fixed N strip.
    // With several N strips and tile rows that split evenly over the 8 XCDs
    // (workgroups are dealt to them round-robin), XCD x instead takes an
    // eighth of the tile rows with all their N tiles, so that the A tile of a
    // row is fetched into that XCD's L2 once rather than once per N strip.
    const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    int tm = blockIdx.x % tiles_m, tn = blockIdx.x / tiles_m;
    if (tiles_n > 1 && tiles_m % 8 == 0) {
        const int x = blockIdx.x % 8, j = blockIdx.x / 8;
        tm = x * (tiles_m / 8) + j / tiles_n;
        tn = j % tiles_n;
    }
    const int m0 = tm * BM, n0 = tn * BN;

    // global -> register staging: 16-byte units, rows clamped into range (rows
    // past M or N compute values that are never stored)
    constexpr int UA = AF32 ? 8 : 4;             // 16-byte units of A per thread
    i32x4 ra[UA], rb[4];
    auto gload = [&](int k0) {
        if constexpr (AF32) {
            const float* A = static_cast<const float*>(A_);
#pragma unroll
            for (int i = 0; i < UA; ++i) {       // 128 rows x 16 units of 4 floats
                const int u = t + GT * i, row = u >> 4, cu = u & 15;
                const int gr = min(m0 + row, M - 1);
                ra[i] = *reinterpret_cast<const i32x4*>(A + (size_t)gr * lda + k0 + 4 * cu);
            }
        } else {
            const bf16_t* A = static_cast<const bf16_t*>(A_);
#pragma unroll
            for (int i = 0; i < UA; ++i) {       // 128 rows x 8 units of 8 bf16
                const int u = t + GT * i, row = u >> 3, cu = u & 7;
                const int gr = min(m0 + row, M - 1);
                ra[i] = *reinterpret_cast<const i32x4*>(A + (size_t)gr * lda + k0 + 8 * cu);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int u = t + GT * i, row = u >> 3, cu = u & 7;
            const int gr = min(n0 + row, N - 1);
            const bf16_t* brow = gr < n_split ? B + (size_t)gr * ldb : B2 + (size_t)(gr - n_split) * ldb;
            rb[i] = *reinterpret_cast<const i32x4*>(brow + k0 + 8 * cu);
        }
    };
    auto lstore = [&](int buf) {
        if constexpr (AF32) {
#pragma unroll
            for (int i = 0; i < UA; ++i) {
                const int u = t + GT * i, row = u >> 4, cu = u & 15;
                const f32x4 x = *reinterpret_cast<const f32x4*>(&ra[i]);
                bf16x4 hi, lo;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    hi[e] = (bf16_t)x[e];
                    lo[e] = (bf16_t)(x[e] - (float)hi[e]);
                }
                *reinterpret_cast<bf16x4*>(&sA[buf][0][row * LDT + 4 * cu]) = hi;
                *reinterpret_cast<bf16x4*>(&sA[buf][1][row * LDT + 4 * cu]) = lo;
            }
        } else {
#pragma unroll
            for (int i = 0; i < UA; ++i) {
                const int u = t + GT * i, row = u >> 3, cu = u & 7;
                *reinterpret_cast<i32x4*>(&sA[buf][0][row * LDT + 8 * cu]) = ra[i];
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int u = t + GT * i, row = u >> 3, cu = u & 7;
            *reinterpret_cast<i32x4*>(&sB[buf][row * LDT + 8 * cu]) = rb[i];
        }
    };

    // acc[nb][mb]: C^T tile rows n = 64 wn + 16 nb + .., columns m = 64 wm + 16 mb + ..
    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int KT = K / BK;
    gload(0);
    lstore(0);
    block_sync();
    for (int kt = 0; kt < KT; ++kt) {
        const int buf = NBUF == 2 ? kt & 1 : 0;
        if (kt + 1 < KT) gload((kt + 1) * BK);
#pragma unroll
        for (int kk = 0; kk < BK; kk += 32) {
            bf16x8 fb[4];
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
                fb[nb] = *reinterpret_cast<const bf16x8*>(&sB[buf][(64 * wn + 16 * nb + ln) * LDT + kk + 8 * lg]);
#pragma unroll
            for (int p = 0; p < NA; ++p) {
#pragma unroll
                for (int mb = 0; mb < 4; ++mb) {
                    const bf16x8 fa = *reinterpret_cast<const bf16x8*>(&sA[buf][p][(64 * wm + 16 * mb + ln) * LDT + kk + 8 * lg]);
#pragma unroll
                    for (int nb = 0; nb < 4; ++nb)
                        acc[nb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[nb], fa, acc[nb][mb], 0, 0, 0);
                }
            }
        }
        if (kt + 1 < KT) {
            if (NBUF == 1) block_sync();      // every wave is done reading the stage
            lstore(NBUF == 2 ? buf ^ 1 : 0);
        }
        block_sync();
    }

    // epilogue: lane holds C[m][n .. n+3] for m = .. + ln, n = .. + 4 lg
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            const int m = m0 + 64 * wm + 16 * mb + ln;
            const int n = n0 + 64 * wn + 16 * nb + 4 * lg;
            if (m < M && n < N) {
                f32x4 v = acc[nb][mb];
                if constexpr (EPI == 1) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = neg_softplus(v[e]);
                }
                store_out4<OutT>(C + (size_t)m * ldc + n, v, N - n);
            }
        }
}

// ---- large tiles: bf16 A, bf16 C -------------------------------------------
// A 512-thread workgroup computes a 256 x 256 tile of C; wave w owns rows
// 128 (w / 4) .. +127 and columns 64 (w % 4) .. +63 (8 x 4 MFMA tiles).  Each
// K-step of 64 stages the A and B tiles (256 rows x 128 bytes each) in LDS
// with 16-byte global-to-LDS loads: one load instruction fills 1 KiB = 8
// rows, and lane l fetches the 16-byte chunk (l % 8) ^ (row % 8) of its row,
// so LDS rows hold their chunks XOR-swizzled and the MFMA fetches (16 rows,
// one chunk column) touch distinct banks.  Two stages, one barrier per
// K-step, software-pipelined: the barrier sits between the step's two 32-wide
// halves.  Before it, the first half's MFMAs run while the second half's
// operands are read; after it, the next step's loads go out into the stage
// just released, and the second half's MFMAs hide the reads of the next
// step's first-half operands.  Each step's loads have a whole step to land,
// and no wave waits on LDS right after the barrier.  K must be a multiple of
// 64 (the layer's feature sizes are).
//
// B may be up to four weight matrices stacked along N (rows n of the product
// come from matrix n / n_split, n_split a multiple of 256, so each tile reads
// one of them): the layer's q, k, v and gate projections then run as one
// product over x, whose 16 rounds of tiles amortise the pipeline's fill and
// drain better than four products of 4 rounds.
constexpr int LBM = 256, LBN = 256, LBK = 64;
constexpr int LGT = 512;
constexpr int LSTAGE = (LBM + LBN) * LBK * 2;      // 64 KiB

struct StackedB {
    const bf16_t* p[4];
};

template <int NB>    // weight matrices stacked along N (1: one matrix)
__global__ void __launch_bounds__(LGT)
gemm_nt_large_kernel(const bf16_t* A, StackedB Bs, bf16_t* C, int M, int N, int K,
                     int lda, int ldb, int ldc, int n_split)
{
    __shared__ __attribute__((aligned(1024))) char smem[2 * LSTAGE];
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int ln = lane & 15, lg = lane >> 4;
    const int wm = wave >> 2, wn = wave & 3;

    // Workgroups are dealt to the 8 XCDs round-robin.  When the tile rows split
    // evenly, XCD x takes an eighth of the row blocks with all their column
    // tiles, so that the workgroups running together on an XCD share A tiles
    // in its L2 (A, the long operand, is then read about once, and the small B
    // comes from the shared last-level cache); otherwise N strips go fastest.
    const int tiles_n = (N + LBN - 1) / LBN, tiles_m = (M + LBM - 1) / LBM;
    int tn = blockIdx.x % tiles_n, tm = blockIdx.x / tiles_n;
    if (tiles_m % 8 == 0) {
        const int x = blockIdx.x % 8, j = blockIdx.x / 8;
        tm = x * (tiles_m / 8) + j / tiles_n;
        tn = j % tiles_n;
    }
    const int m0 = tm * LBM, n0 = tn * LBN;
    // this tile's weight matrix and its rows n0 - seg n_split ..
    const int seg = NB == 1 ? 0 : n0 / n_split;
    const bf16_t* B = Bs.p[seg];
    const int nb0 = n0 - seg * n_split, nseg = min(n_split, N - seg * n_split);

    // loads of one K-step: 32 segments of A, 32 of B, 8 per wave
    const int lrow = lane >> 3, lchunk = (lane & 7) ^ lrow;    // row within segment, chunk fetched
    auto issue = [&](int k0, int stage) {
        char* st = smem + stage * LSTAGE;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int seg = wave + 8 * i;                  // 0..63, uniform per wave
            const bool isA = seg < 32;
            const int row = 8 * (seg & 31) + lrow;
            const bf16_t* src = isA ? A + (size_t)min(m0 + row, M - 1) * lda
                                    : B + (size_t)min(nb0 + row, nseg - 1) * ldb;
            __builtin_amdgcn_global_load_lds(src + k0 + 8 * lchunk,
                                             (__attribute__((address_space(3))) void*)(st + seg * 1024), 16, 0, 0);
        }
    };
    // 16-byte fragment of row r, logical chunk lc, from a swizzled tile
    auto frag = [&](const char* tile, int r, int lc) {
        return *reinterpret_cast<const bf16x8*>(tile + r * 128 + ((lc ^ (r & 7)) << 4));
    };

    f32x4 acc[4][8];      // [nb][mb]: C^T tile rows n = 64 wn + 16 nb, columns m = 128 wm + 16 mb
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // operands of one 32-wide half step kk: 4 B and 8 A fragments
    bf16x8 f0b[4], f0a[8], f1b[4], f1a[8];
    auto rd = [&](int stage, int kk, bf16x8 (&fb)[4], bf16x8 (&fa)[8]) {
        const char* sA = smem + stage * LSTAGE;
        const char* sB = sA + LBM * LBK * 2;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) fb[nb] = frag(sB, 64 * wn + 16 * nb + ln, 4 * kk + lg);
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) fa[mb] = frag(sA, 128 * wm + 16 * mb + ln, 4 * kk + lg);
    };
    auto mm = [&](bf16x8 (&fb)[4], bf16x8 (&fa)[8]) {
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int mb = 0; mb < 8; ++mb)
                acc[nb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[nb], fa[mb], acc[nb][mb], 0, 0, 0);
    };

    const int KT = K / LBK;
    issue(0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    block_sync();
    issue(min(1, KT - 1) * LBK, 1);
    rd(0, 0, f0b, f0a);
    for (int kt = 0; kt < KT; ++kt) {
        const int stage = kt & 1;
        // first half: its MFMAs, with one second-half operand read per two
        rd(stage, 1, f1b, f1a);
        mm(f0b, f0a);
#pragma unroll
        for (int i = 0; i < 12; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);     // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);     // LDS read
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(0);        // step kt+1 landed; this step's reads done
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        // step kt+2 into the stage just released (clamped: at the end the last
        // tile is reloaded into a stage that is not read again), the next
        // step's first-half operands (after the last step: unused reads of the
        // idle stage), then the second half's MFMAs
        issue(min(kt + 2, KT - 1) * LBK, stage);
        rd(stage ^ 1, 0, f0b, f0a);
        __builtin_amdgcn_sched_barrier(0);
        mm(f1b, f1a);
        __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_waitcnt(0);

    // epilogue: lane holds C[m][n .. n+3] for m = .. + ln, n = .. + 4 lg
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) {
            const int m = m0 + 128 * wm + 16 * mb + ln;
            const int n = n0 + 64 * wn + 16 * nb + 4 * lg;
            if (m < M && n < N) store_out4<bf16_t>(C + (size_t)m * ldc + n, acc[nb][mb], N - n);
        }
}

}  // namespace

bool gemm_stacked_ok(int M, int n_split, int nmat)
{
    return M >= LBM && n_split > 0 && n_split % LBN == 0 && nmat >= 1 && nmat <= 4;
}

hipError_t launch_gemm_nt_stacked(const bf16_t* A, const bf16_t* const* B, int nmat, bf16_t* C, int M,
                                  int n_split, int K, int lda, int ldb, int ldc, hipStream_t stream)
{
    if (!gemm_stacked_ok(M, n_split, nmat)) return hipErrorInvalidValue;
    StackedB bs;
    for (int i = 0; i < 4; ++i) bs.p[i] = B[i < nmat ? i : nmat - 1];
    const int N = nmat * n_split;
    const unsigned tiles = (unsigned)(((M + LBM - 1) / LBM) * (N / LBN));
#define KDA_LARGE(NB) hipLaunchKernelGGL(gemm_nt_large_kernel<NB>, dim3(tiles), dim3(LGT), 0, stream, A, bs, C, M, N, \
                                         K, lda, ldb, ldc, n_split)
    if (nmat == 4) KDA_LARGE(4);
    else if (nmat == 3) KDA_LARGE(3);
    else if (nmat == 2) KDA_LARGE(2);
    else KDA_LARGE(1);
#undef KDA_LARGE
    return hipGetLastError();
}

hipError_t launch_gemm_nt(const void* A, bool a_f32, const bf16_t* B, void* C, bool c_f32,
                          int epilogue, int M, int N, int K, int lda, int ldb, int ldc,
                          hipStream_t stream, const bf16_t* B2, int n_split)
{
    if (M <= 0 || N <= 0) return hipSuccess;
    if (!B2 && !a_f32 && !c_f32 && epilogue == 0 && M >= LBM && N >= LBN) {
        const unsigned tiles = (unsigned)(((M + LBM - 1) / LBM) * ((N + LBN - 1) / LBN));
        const StackedB bs = {{B, B, B, B}};
        hipLaunchKernelGGL(gemm_nt_large_kernel<1>, dim3(tiles), dim3(LGT), 0, stream,
                           (const bf16_t*)A, bs, (bf16_t*)C, M, N, K, lda, ldb, ldc, N);
        return hipGetLastError();
    }
    const dim3 grid((unsigned)(((M + BM - 1) / BM) * ((N + BN - 1) / BN))), block(GT);
#define KDA_GEMM(AF, OT, EP) \
    hipLaunchKernelGGL((gemm_nt_kernel<AF, OT, EP>), grid, block, 0, stream, A, B, (OT*)C, M, N, K, lda, ldb, ldc, \
                       B2 ? B2 : B, B2 ? n_split : N)
    if (a_f32) {
        if (c_f32 && epilogue == 1) KDA_GEMM(true, float, 1);
        else if (c_f32) KDA_GEMM(true, float, 0);
        else KDA_GEMM(true, bf16_t, 0);
    } else {
        if (c_f32 && epilogue == 1) KDA_GEMM(false, float, 1);
        else if (c_f32) KDA_GEMM(false, float, 0);
        else KDA_GEMM(false, bf16_t, 0);
    }
#undef KDA_GEMM
    return hipGetLastError();
}

}  // namespace kda
