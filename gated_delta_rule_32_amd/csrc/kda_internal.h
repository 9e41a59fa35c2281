// kda_internal.h -- launchers behind the C ABI (internal to libkda).
// Every launcher assumes the arguments were validated by the C ABI layer.
#pragma once
#include <hip/hip_runtime.h>

namespace kda {

// Decode step over `heads` = N*H independent heads; dtype 0 = fp32, 1 = bf16.
hipError_t launch_decode_step(const void* q, const void* k, const void* v,
                              const float* g, const void* beta, float* S, void* o,
                              long long heads, int dtype, hipStream_t stream);

// Chunked prefill over B*H heads of T >= 1 tokens (d_k = d_v = 128).  With
// `ws` non-null (bf16 only, at least chunk_ws_bytes(B, T, H) bytes) the
// two-kernel schedule runs; otherwise the fused single kernel.
hipError_t launch_chunk_fwd(const void* q, const void* k, const void* v,
                            const float* g, const void* beta, const float* S0,
                            void* o, float* S_T, int B, int T, int H, int dtype,
                            void* ws, hipStream_t stream);

// Bytes of workspace the two-kernel schedule needs: one 66,048-byte block of
// key-side operands per (batch, head, 64-token chunk).
size_t chunk_ws_bytes(long long B, long long T, long long H);

// Whether the two-kernel schedule is expected to be faster for this shape.
bool chunk_prefers_two_kernel(long long B, long long T, long long H, int dtype);

// S_T = S0 (or zeros when S0 is NULL) for `heads` states; used when T = 0.
hipError_t launch_state_copy(const float* S0, float* S_T, long long heads,
                             hipStream_t stream);

}  // namespace kda
