// kda_chunk_common.h -- device helpers and workspace layouts shared by the
// chunked KDA kernels (the forward schedules in kda_prefill.hip and the
// backward pass in kda_backward.hip).  Internal to libkda.
#pragma once
#include "kda_device.h"

namespace kda {
namespace {

constexpr int C = 64;     // chunk length
constexpr int DK = 128;   // key / value head dimension
constexpr float LOG2E = 1.4426950408889634f;

// Forget-gate layouts (the kda_gate_t values of the C ABI).
constexpr int GATE_CHANNEL = 0, GATE_HEAD = 1, GATE_NONE = 2;

// Barrier that orders LDS traffic only: global loads stay in flight.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// s_waitcnt on the vector-memory counter only: at most N vector memory
// operations of this wave outstanding (vmcnt is bits 3:0 and 15:14 of the
// immediate; expcnt and lgkmcnt at their maxima, i.e. not waited on).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
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
    constexpr int UNR = (K / Mma<E>::KS) < 2 ? (K / Mma<E>::KS) : 2;
#pragma unroll UNR
    for (int k = 0; k < K; k += Mma<E>::KS) {
        const auto a = Mma<E>::frag_kc(A, lda, arow0, k, lane);
#pragma unroll
        for (int t = 0; t < NB; ++t) acc[t] = Mma<E>::mma(a, Mma<E>::frag_kc(B, ldb, brow[t], k, lane), acc[t]);
    }
}

// ---- lane exchange between 16-lane rows -----------------------------------
// Value held by lane l ^ 16 (rows 0<->1, 2<->3) and by lane l ^ 32 (rows
// 0,1 <-> 2,3), with the gfx950 row-swap instructions (plain VALU, unlike a
// general shuffle, which goes through the LDS crossbar).  Inactive source
// lanes are read too (fetch-inactive set), so a call under a partial exec
// mask still sees the partner's value; callers nevertheless call these with
// the whole wave active.
__device__ __forceinline__ float lane_xor16(float x, int lane) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), true, false);
    return __uint_as_float((lane & 16) ? r[0] : r[1]);
}
__device__ __forceinline__ float lane_xor32(float x, int lane) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), true, false);
    return __uint_as_float((lane & 32) ? r[0] : r[1]);
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

// When TmT is not null, X_RI is also written unscaled and transposed there
// (TmT[i][r] = X[r][i], row pitch PT), for the backward pass.
template <int I, int PA, int PT>
__device__ __forceinline__ void ut_offdiag_column(const float* RA, bf16_t* RT, const float* s_beta, int lane,
                                                  bf16_t* TmT = nullptr) {
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
        if (TmT) *reinterpret_cast<bf16x4*>(TmT + (16 * I + ln) * PT + 16 * R + 4 * lg) = to_bf16x4(X[R]);
    }
}

// ---- MFMA operands split over two 16-column blocks ---------------------------
__device__ __forceinline__ bf16x8 cat8(const bf16x4& a, const bf16x4& b) {
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) { r[i] = a[i]; r[i + 4] = b[i]; }
    return r;
}
__device__ __forceinline__ bf16x4 ld4(const bf16_t* p) { return *reinterpret_cast<const bf16x4*>(p); }

// Two adjacent 16-column blocks (2p, 2p+1) of one row as an A-operand: lane
// (row ln, group lg) takes columns 32p + 4lg .. +3 and 32p + 16 + 4lg .. +3;
// with `hi` false the second half is zero.  The matching B operand is two
// accumulator tiles (rows 32p + 4lg + e and 32p + 16 + 4lg + e of a product's
// output) packed side by side, so a product's output feeds the next product
// without leaving registers.
__device__ __forceinline__ bf16x8 a_pair(const bf16_t* row, int p, int lg, bool hi) {
    const bf16x4 a = ld4(row + 32 * p + 4 * lg);
    const bf16x4 b = hi ? ld4(row + 32 * p + 16 + 4 * lg) : bf16x4{};
    return cat8(a, b);
}

// ---- forward state scan: per-chunk operand block -------------------------------
// Workspace block of one chunk, written by a prep kernel and read by
// chunk_scan_kernel (bf16 only).  It is the image of the scan's LDS stage:
// rows keep their 16-byte padding and Kt^T its swizzle (kbt_swz), so the scan
// copies it linearly in 1 KiB pieces.  The general DPLR block (WS_*, 72,704
// bytes) keeps padded rows as below.  The KDA block (WSK_*, 60,416 bytes)
// drops the padding: its rows are XOR-swizzled in 16-byte units instead, and
// it keeps only the ten lower 16 x 16 tiles of the triangular Tm Diag(beta)
// and Aqk.  Byte offsets of the DPLR block:
constexpr int WS_P128 = DK + 8, WS_P64 = C + 8;    // padded row pitches (elements)
constexpr int WS_QT = 0;                            // Qt   [64][136] bf16, token-major
constexpr int WS_KH = WS_QT + C * WS_P128 * 2;      // Kh   [64][136] bf16, token-major
constexpr int WS_KBT = WS_KH + C * WS_P128 * 2;     // Kt^T [128][72] bf16, channel-major, swizzled
                                                    //   (Kt = e^{G_64 - G} k; DPLR: (e^{-G} a)^T)
constexpr int WS_TM = WS_KBT + DK * WS_P64 * 2;     // Tm Diag(beta) [64][72] bf16
constexpr int WS_QK = WS_TM + C * WS_P64 * 2;       // Aqk  [64][72] bf16
constexpr int WS_GAM = WS_QK + C * WS_P64 * 2;      // e^{G_64} [128] fp32
constexpr int WS_USED = WS_GAM + DK * 4;            // 72,192 bytes written
constexpr int WS_CHUNK = (WS_USED + 1023) / 1024 * 1024;   // 72,704: whole KiB per block
// KDA block.  Every MFMA A-operand the scan reads is one contiguous 16-byte
// unit: for a row (token of Qt / Kh, channel of Kt^T) and a pair p of
// 16-column blocks, lane group lg (lane / 16) takes columns 32p + 4lg .. +3
// and 32p + 16 + 4lg .. +3 (see a_pair), stored together as unit 4p + lg.
//   Qt, Kh  [64 tokens][16 units] bf16, rows of 256 B; unit u of row r at
//           u ^ (r % 16), so the 16 lanes of a lane group read 16 distinct
//           units (every bank once);
//   Kt^T    [128 channels][8 units], rows of 128 B; unit u of row c at
//           u ^ ((c / 2) % 8) (rows two apart share banks);
//   Tm Diag(beta), Aqk: the lower part only, as the six operand pairs
//           (Rb, p), 2p <= Rb, in the order (0,0) (1,0) (2,0) (2,1) (3,0)
//           (3,1) (wsk_pair_off): a pair whose second block lies above the
//           diagonal holds 8-byte units (the first block's four columns),
//           the others 16-byte units, each [16 rows][4 lane groups];
//   e^{G_64} [128] fp32.
constexpr int WS_TRI = 5 * 1024;                            // bytes of one triangular matrix
constexpr int WSK_QT = 0;
constexpr int WSK_KH = WSK_QT + C * DK * 2;                 // 16 KiB
constexpr int WSK_KBT = WSK_KH + C * DK * 2;
constexpr int WSK_TM = WSK_KBT + DK * C * 2;                // Tm Diag(beta) pairs
constexpr int WSK_QK = WSK_TM + WS_TRI;                     // Aqk pairs
constexpr int WSK_GAM = WSK_QK + WS_TRI;                    // e^{G_64} [128] fp32
constexpr int WSK_USED = WSK_GAM + DK * 4;                  // 59,904 bytes written
constexpr int WSK_CHUNK = (WSK_USED + 1023) / 1024 * 1024;  // 60,416
// element offset of unit (row r, logical unit u) of Qt / Kh, and of Kt^T
__device__ __forceinline__ constexpr int wsk_tok_unit(int r, int u) { return r * DK + ((u ^ (r & 15)) << 3); }
__device__ __forceinline__ constexpr int wsk_kbt_unit(int c, int u) { return c * C + ((u ^ ((c >> 1) & 7)) << 3); }
// byte offset of operand pair (Rb, p) of a triangular matrix, and whether it
// holds both blocks
__device__ __forceinline__ constexpr int wsk_pair_off(int Rb, int p) {
    return Rb == 0 ? 0 : Rb == 1 ? 512 : Rb == 2 ? (p == 0 ? 1536 : 2560) : (p == 0 ? 3072 : 4096);
}
__device__ __forceinline__ constexpr bool wsk_pair_full(int Rb, int p) { return 2 * p + 1 <= Rb; }

// Element (channel c, token i) of the swizzled Kb^T: the 8-token blocks of a
// row are XOR-permuted by bits 3..5 of the channel.
__device__ __forceinline__ constexpr int kbt_swz(int c, int i) {
    return c * WS_P64 + ((((i >> 3) ^ ((c >> 3) & 7)) << 3) | (i & 7));
}

// ---- backward pass: saved per-chunk tensors -----------------------------------
// S_n and dS' ([128 channels][128 value columns] per chunk) and Y, Vn, dZ
// ([64 tokens][128 columns]) are written by the scans' consumer waves, whose
// lane (ln, lg) holds rows 4 lg + e (e < 4) of column ln of a 16 x 16 tile,
// and read by the gradient kernel as 8 consecutive columns of one row.  They
// are stored as 16 x 16 tiles, [chunk][16-column slice][16-row block][256],
// the rows of a tile in the order 4 e + lg and each row's 16 columns
// contiguous: a consumer store of one e covers 128 contiguous bytes (a whole
// line, instead of four 32-byte pieces), and a row's 8 columns stay 16
// contiguous bytes for the reader.  Element offset of (row r, column c) of a
// chunk with `rows` rows:
__device__ __forceinline__ size_t sv_at(size_t cidx, int rows, int r, int c) {
    return ((cidx * (DK / 16) + (c >> 4)) * (rows >> 4) + (r >> 4)) * 256 + (((r & 3) << 2) | ((r >> 2) & 3)) * 16 +
           (c & 15);
}

// Pair exchange for stores of an accumulator tile (lane (ln, lg) holds rows
// 4 lg + e of column ln): neighbouring lanes swap halves (DPP quad_perm
// [1,0,3,2]) so that an even lane holds rows 4 lg, 4 lg + 1 and an odd lane
// rows 4 lg + 2, 4 lg + 3, each at the column pair (ln & ~1, ln | 1).
// Returns the two 4-byte pieces of the lane: piece i is row
// 4 lg + 2 (ln & 1) + i, columns (ln & ~1, ln | 1).
__device__ __forceinline__ void pair_rows_bf16(const f32x4& x, int lane, bf16x2& p0, bf16x2& p1) {
    const bool odd = lane & 1;
    const float s0 = odd ? x[0] : x[2], s1 = odd ? x[1] : x[3];
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, s0), 0xB1, 0xF, 0xF, false));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, s1), 0xB1, 0xF, 0xF, false));
    if (odd) {
        p0[0] = (bf16_t)r0; p0[1] = (bf16_t)x[2];
        p1[0] = (bf16_t)r1; p1[1] = (bf16_t)x[3];
    } else {
        p0[0] = (bf16_t)x[0]; p0[1] = (bf16_t)r0;
        p1[0] = (bf16_t)x[1]; p1[1] = (bf16_t)r1;
    }
}

// ---- backward pass: per-chunk operand block of the reverse state scan --------
// Written by the prep kernel next to the forward block, read by
// chunk_bwd_scan_kernel (copied linearly into LDS and read there as MFMA A
// operands).  bf16 except the two vectors, no row padding:
//   Aqk^T, Tm^T (no beta): upper triangular, as the operand pairs (Rb, p) of
//           their nonzero blocks (wsb_pair_off): row block Rb, pair p of
//           columns 32p + 4lg .. +3 and 32p + 16 + 4lg .. +3 for lane group
//           lg; a pair whose first block lies below the diagonal holds 8-byte
//           units (the second block's four columns), the others 16-byte
//           units, each [16 rows][4 lane groups];
//   Qt^T, Kh^T [128][64]: the unit layout of the forward block's Kt^T
//           (wsk_kbt_unit);
//   Kt = e^{G_64 - G} k [64][128]: the unit layout of its Qt (wsk_tok_unit);
//   e^{G_64} [128] and beta [64] (0 past T), fp32.
constexpr int WSB_AQKT = 0;
constexpr int WSB_TMT = WSB_AQKT + WS_TRI;
constexpr int WSB_QTT = WSB_TMT + WS_TRI;                // 16 KiB each
constexpr int WSB_KHT = WSB_QTT + DK * C * 2;
constexpr int WSB_KT = WSB_KHT + DK * C * 2;
constexpr int WSB_GAM = WSB_KT + C * DK * 2;
constexpr int WSB_BETA = WSB_GAM + DK * 4;
constexpr int WSB_USED = WSB_BETA + C * 4;               // 60,160 bytes
constexpr int WSB_CHUNK = (WSB_USED + 1023) / 1024 * 1024;   // 60,416
// byte offset of operand pair (Rb, p) of an upper triangular matrix (pairs
// with 2p + 1 < Rb are zero and not stored), and whether it holds both blocks
__device__ __forceinline__ constexpr int wsb_pair_off(int Rb, int p) {
    return Rb == 0 ? 1024 * p : Rb == 1 ? (p == 0 ? 2048 : 2560) : Rb == 2 ? 3584 : 4608;
}
__device__ __forceinline__ constexpr bool wsb_pair_full(int Rb, int p) { return 2 * p >= Rb; }
__device__ __forceinline__ constexpr bool wsb_pair_zero(int Rb, int p) { return 2 * p + 1 < Rb; }
// row pitch (elements) of the prep's Tm^T staging tile in LDS
constexpr int TMT_P = C + 8;

// Eight consecutive elements (one 16-byte load for bf16, two for fp32).
template <typename E> struct Raw8;
template <> struct Raw8<bf16_t> {
    bf16x8 x;
    __device__ __forceinline__ void load(const bf16_t* p) { x = *reinterpret_cast<const bf16x8*>(p); }
    __device__ __forceinline__ float operator[](int i) const { return (float)x[i]; }
};
template <> struct Raw8<float> {
    f32x4 a, b;
    __device__ __forceinline__ void load(const float* p) {
        a = reinterpret_cast<const f32x4*>(p)[0];
        b = reinterpret_cast<const f32x4*>(p)[1];
    }
    __device__ __forceinline__ float operator[](int i) const { return i < 4 ? a[i] : b[i - 4]; }
};
struct Raw8f {   // eight fp32 values (the log-decay)
    f32x4 a, b;
    __device__ __forceinline__ void load(const float* p) {
        a = reinterpret_cast<const f32x4*>(p)[0];
        b = reinterpret_cast<const f32x4*>(p)[1];
    }
    __device__ __forceinline__ float operator[](int i) const { return i < 4 ? a[i] : b[i - 4]; }
};
template <typename E> __device__ __forceinline__ void store8(E* p, const float* x);
template <> __device__ __forceinline__ void store8<bf16_t>(bf16_t* p, const float* x) {
    bf16x8 v;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (bf16_t)x[i];
    *reinterpret_cast<bf16x8*>(p) = v;
}
template <> __device__ __forceinline__ void store8<float>(float* p, const float* x) {
    reinterpret_cast<f32x4*>(p)[0] = f32x4{x[0], x[1], x[2], x[3]};
    reinterpret_cast<f32x4*>(p)[1] = f32x4{x[4], x[5], x[6], x[7]};
}

}  // namespace
}  // namespace kda
