// kda_layer.hip -- the KDA token-mixing layer around the KDA operator, gfx950.
//
// Page "Kimi K3论文：Kimi Linear", section 3 parameterises the inputs of each
// head as q, k = L2Norm(Swish(ShortConv(W_{q/k} x))), v = Swish(ShortConv(W_v
// x)), alpha = f(W_up W_down x), beta = Sigmoid(W_beta x), and closes the
// layer with a head-wise RMSNorm and a sigmoid output gate.  Readings used
// here: f(u) = exp(-softplus(u)) (so log alpha = -softplus(u)); ShortConv is a
// causal depthwise convolution with 4 taps, zero left padding, no bias;
// Swish(x) = x sigmoid(x); L2Norm and RMSNorm put 1e-6 inside the square root
// and RMSNorm has no gain; the gate is sigmoid(W_g x).
//
// Kernels (all elementwise / per-head reductions, HBM-bound):
//   conv_act_kernel  : pre-activations of q, k, v -> conv -> Swish -> L2Norm
//                      (q, k), bf16 outputs in [tokens, H, 128]; also beta.
//   out_gate_kernel  : RMSNorm(o per head) * sigmoid(gate) -> bf16.
// Each lane handles 8 consecutive channels (16-byte accesses); a head's 128
// channels are 16 lanes, reduced with lane shuffles.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int HD = 128;          // head dimension
constexpr int TAPS = 4;          // ShortConv taps

__device__ __forceinline__ float sigmoid_f(float x) {
    return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-x * 1.4426950408889634f));
}

__device__ __forceinline__ void load8(const bf16_t* p, float* x) {
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = (float)v[i];
}
__device__ __forceinline__ void store8b(bf16_t* p, const float* x) {
    bf16x8 v;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (bf16_t)x[i];
    *reinterpret_cast<bf16x8*>(p) = v;
}

// Sum over the 16 lanes of a head (lanes 16 apart hold other heads).
__device__ __forceinline__ float head_sum(float s) {
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) s += __shfl_xor(s, off);
    return s;
}

// grid (token tiles of CONV_TT tokens per sequence, B, 3): blockIdx.z selects
// q (0), k (1) or v (2).  Each thread covers 8 consecutive channels (a 16-lane
// group covers one head) and walks the tile's tokens in order, keeping the
// last three inputs in registers, so every pre-activation row is read once
// (plus a three-row halo per tile) and the taps are loaded once per tile.
constexpr int CONV_TT = 64;      // tokens per tile
constexpr int CONV_G = 8;        // tokens whose loads are issued together

__global__ void __launch_bounds__(256)
conv_act_kernel(const bf16_t* pre, int ld_pre, const bf16_t* conv_q, const bf16_t* conv_k,
                const bf16_t* conv_v, bf16_t* q, bf16_t* k, bf16_t* v, const float* beta_pre,
                int ld_bp, bf16_t* beta, int T, int H)
{
    const int which = blockIdx.z;
    const int t0 = blockIdx.x * CONV_TT;
    const size_t row0 = (size_t)blockIdx.y * T;          // first row of the sequence
    const int C = H * HD;
    const int t1 = min(t0 + CONV_TT, T);
    bf16_t* out = which == 0 ? q : (which == 1 ? k : v);
    const bf16_t* cw = which == 0 ? conv_q : (which == 1 ? conv_k : conv_v);
    for (int c0 = 8 * threadIdx.x; c0 < C; c0 += 8 * blockDim.x) {
        const int col = which * C + c0;                  // column in the pre-activations
        float w[8][TAPS];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const bf16x4 wt = *reinterpret_cast<const bf16x4*>(cw + (size_t)(c0 + i) * TAPS);
#pragma unroll
            for (int j = 0; j < TAPS; ++j) w[i][j] = (float)wt[j];
        }
        // window: x[t-3], x[t-2], x[t-1] (zero before the sequence starts)
        float x3[8], x2[8], x1[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) { x3[i] = 0.f; x2[i] = 0.f; x1[i] = 0.f; }
        if (t0 >= 3) load8(pre + (row0 + t0 - 3) * ld_pre + col, x3);
        if (t0 >= 2) load8(pre + (row0 + t0 - 2) * ld_pre + col, x2);
        if (t0 >= 1) load8(pre + (row0 + t0 - 1) * ld_pre + col, x1);
        for (int tg = t0; tg < t1; tg += CONV_G) {
            bf16x8 raw[CONV_G];
#pragma unroll
            for (int u = 0; u < CONV_G; ++u)                 // clamped: rows past t1 are not used
                raw[u] = *reinterpret_cast<const bf16x8*>(pre + (row0 + min(tg + u, t1 - 1)) * ld_pre + col);
#pragma unroll
            for (int u = 0; u < CONV_G; ++u) {
                if (tg + u < t1) {
                    float x0[8], y[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        x0[i] = (float)raw[u][i];
                        y[i] = w[i][0] * x3[i] + w[i][1] * x2[i] + w[i][2] * x1[i] + w[i][3] * x0[i];
                        y[i] = y[i] * sigmoid_f(y[i]);            // Swish
                    }
                    if (which < 2) {                             // L2Norm over the head
                        float ss = 0.f;
#pragma unroll
                        for (int i = 0; i < 8; ++i) ss += y[i] * y[i];
                        ss = head_sum(ss);
                        const float inv = __builtin_amdgcn_rsqf(ss + 1e-6f);
#pragma unroll
                        for (int i = 0; i < 8; ++i) y[i] *= inv;
                    }
                    store8b(out + (row0 + tg + u) * C + c0, y);
#pragma unroll
                    for (int i = 0; i < 8; ++i) { x3[i] = x2[i]; x2[i] = x1[i]; x1[i] = x0[i]; }
                }
            }
        }
    }
    if (which == 2) {
        for (int e = threadIdx.x; e < (t1 - t0) * H; e += blockDim.x) {
            const size_t row = row0 + t0 + e / H;
            const int hh = e % H;
            beta[row * H + hh] = (bf16_t)sigmoid_f(beta_pre[row * ld_bp + hh]);
        }
    }
}

// grid rows = B*T; o [rows, H*128] bf16, gate [rows, ld_gate] bf16 (pre-sigmoid)
__global__ void __launch_bounds__(256)
out_gate_kernel(const bf16_t* o, const bf16_t* gate, int ld_gate, bf16_t* z, int H)
{
    const int row = blockIdx.x;
    const int C = H * HD;
    for (int c0 = 8 * threadIdx.x; c0 < C; c0 += 8 * blockDim.x) {
        float x[8], gt[8];
        load8(o + (size_t)row * C + c0, x);
        load8(gate + (size_t)row * ld_gate + c0, gt);
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) ss += x[i] * x[i];
        ss = head_sum(ss);
        const float inv = __builtin_amdgcn_rsqf(ss * (1.f / HD) + 1e-6f);
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = x[i] * inv * sigmoid_f(gt[i]);
        store8b(z + (size_t)row * C + c0, x);
    }
}

// threads per row: enough 8-channel groups for the row, whole heads per wave
int row_threads(int H) {
    int n = H * HD / 8;
    return n >= 256 ? 256 : n;
}

}  // namespace

hipError_t launch_conv_act(const bf16_t* pre, int ld_pre, const bf16_t* conv_q,
                           const bf16_t* conv_k, const bf16_t* conv_v, bf16_t* q, bf16_t* k,
                           bf16_t* v, const float* beta_pre, int ld_bp, bf16_t* beta, int B, int T,
                           int H, hipStream_t stream)
{
    if ((long long)B * T <= 0) return hipSuccess;
    const dim3 grid((unsigned)((T + CONV_TT - 1) / CONV_TT), (unsigned)B, 3);
    hipLaunchKernelGGL(conv_act_kernel, grid, dim3(row_threads(H)), 0, stream,
                       pre, ld_pre, conv_q, conv_k, conv_v, q, k, v, beta_pre, ld_bp, beta, T, H);
    return hipGetLastError();
}

hipError_t launch_out_gate(const bf16_t* o, const bf16_t* gate, int ld_gate, bf16_t* z,
                           long long rows, int H, hipStream_t stream)
{
    if (rows <= 0) return hipSuccess;
    hipLaunchKernelGGL(out_gate_kernel, dim3((unsigned)rows), dim3(row_threads(H)), 0, stream,
                       o, gate, ld_gate, z, H);
    return hipGetLastError();
}

// ---- the whole layer --------------------------------------------------------
// Workspace regions (each 256-byte aligned), R = B*T rows, HDm = H*128:
//   PRE   [R, 4*HDm] bf16  pre-activations x W^T of q | k | v | output gate
//   LOW   [R, ldz]   fp32  W_down x (rank columns) | W_beta x (H columns)
//   Q,K,V [R, HDm]   bf16  KDA inputs (= [B, T, H, 128])
//   G     [R, HDm]   fp32  log alpha = -softplus(W_up (W_down x))
//   BETA  [R, H]     bf16
//   O     [R, HDm]   bf16  KDA output
//   ZG    [R, HDm]   bf16  RMSNorm(o) * sigmoid(gate), the input of W_o
//   CHUNK             key-side chunk operands of the two-kernel KDA schedule
size_t layer_ws_layout(long long B, long long T, long long H, long long rank, size_t* off)
{
    const size_t R = (size_t)(B * T), HDm = (size_t)(H * HD);
    const size_t ldz = (size_t)((rank + H + 3) / 4 * 4);
    const bool two = chunk_prefers_two_kernel(B, T, H, 1);
    const size_t sizes[KDA_LAYER_WS_REGIONS] = {
        R * 4 * HDm * 2, R * ldz * 4, R * HDm * 2, R * HDm * 2, R * HDm * 2,
        R * HDm * 4,     R * (size_t)H * 2, R * HDm * 2, R * HDm * 2,
        two ? chunk_fwd_ws_bytes(B, T, H) : 0};
    size_t p = 0;
    for (int i = 0; i < KDA_LAYER_WS_REGIONS; ++i) {
        if (off) off[i] = p;
        p += (sizes[i] + 255) / 256 * 256;
    }
    return p;
}

hipError_t launch_layer_fwd(const LayerWeights& W, const bf16_t* x, bf16_t* y, int B, int T,
                            int d_model, int H, int rank, char* ws, hipStream_t stream)
{
    size_t off[KDA_LAYER_WS_REGIONS];
    layer_ws_layout(B, T, H, rank, off);
    const bool two = chunk_prefers_two_kernel(B, T, H, 1);
    const int R = B * T, HDm = H * HD, NY = 4 * HDm, ldz = (rank + H + 3) / 4 * 4;
    bf16_t* pre = (bf16_t*)(ws + off[KDA_LAYER_WS_PRE]);
    float* low = (float*)(ws + off[KDA_LAYER_WS_LOW]);
    bf16_t* q = (bf16_t*)(ws + off[KDA_LAYER_WS_Q]);
    bf16_t* k = (bf16_t*)(ws + off[KDA_LAYER_WS_K]);
    bf16_t* v = (bf16_t*)(ws + off[KDA_LAYER_WS_V]);
    float* g = (float*)(ws + off[KDA_LAYER_WS_G]);
    bf16_t* beta = (bf16_t*)(ws + off[KDA_LAYER_WS_BETA]);
    bf16_t* o = (bf16_t*)(ws + off[KDA_LAYER_WS_O]);
    bf16_t* zg = (bf16_t*)(ws + off[KDA_LAYER_WS_ZG]);
    char* kws = two ? ws + off[KDA_LAYER_WS_CHUNK] : nullptr;
    hipError_t e;
    // 1. projections: q, k, v and gate pre-activations in bf16; the low-rank
    //    gate input W_down x and the beta logits in fp32
    //    (as one product over the four stacked weights when the tiles allow)
    const bf16_t* Win[4] = {W.W_q, W.W_k, W.W_v, W.W_g};
    if (gemm_stacked_ok(R, HDm, 4)) {
        if ((e = launch_gemm_nt_stacked(x, Win, 4, pre, R, HDm, d_model, d_model, d_model, NY, stream)))
            return e;
    } else {
        for (int i = 0; i < 4; ++i)
            if ((e = launch_gemm_nt(x, false, Win[i], pre + (size_t)i * HDm, false, 0, R, HDm, d_model,
                                    d_model, d_model, NY, stream)))
                return e;
    }
    //    ([W_down; W_beta] stacked: one pass over x writes both)
    if ((e = launch_gemm_nt(x, false, W.W_down, low, true, 0, R, rank + H, d_model, d_model, d_model,
                            ldz, stream, W.W_beta, rank)))
        return e;
    // 2. log alpha = -softplus(W_up (W_down x)); fp32 A operand (hi/lo split)
    if ((e = launch_gemm_nt(low, true, W.W_up, g, true, 1, R, HDm, rank, ldz, rank, HDm, stream)))
        return e;
    // 3. ShortConv + Swish (+ L2Norm for q, k); beta = sigmoid(W_beta x)
    if ((e = launch_conv_act(pre, NY, W.conv_q, W.conv_k, W.conv_v, q, k, v, low + rank, ldz, beta,
                             B, T, H, stream)))
        return e;
    // 4. the KDA operator, zero initial state
    if ((e = launch_chunk_fwd(q, k, v, g, beta, nullptr, o, nullptr, B, T, H, 1, kws, stream,
                              KDA_GATE_CHANNEL, nullptr, true)))
        return e;
    // 5. RMSNorm(o) * sigmoid(W_g x), then W_o
    if ((e = launch_out_gate(o, pre + 3 * (size_t)HDm, NY, zg, R, H, stream))) return e;
    return launch_gemm_nt(zg, false, W.W_o, y, false, 0, R, d_model, HDm, HDm, HDm, d_model, stream);
}

}  // namespace kda
