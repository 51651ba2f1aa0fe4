// Weighted combine ("Mixture of experts" page, Code: moe_infer's weighted sum of
// each token's K expert outputs, and forward's addition of the shared expert), optionally
// with the block's residual addition ("Input features" page, evidence "block"):
//   out[n] = bf16( sum_{k<K} w[n][k] * y_sorted[slot_pos[n*K+k]] + shared[n] + residual[n] )
// float32, ascending k, then the shared term, then the residual, one nearest-even rounding.
// Each workgroup owns whole tokens and writes every output element exactly once, so no
// atomics are needed and the result is deterministic. out may be the residual itself: a lane
// reads each chunk of it before writing that chunk.
//
// Memory-bound: a lane moves 8 bf16 (16 B) per source row per chunk; the K source rows
// of a token are 14 KB contiguous runs at K2 shapes.
#include "moe_internal.h"

namespace moe {

__device__ __forceinline__ void unpack8(const uint4 r, float (&f)[8]) {
    f[0] = bf16_to_f32(r.x & 0xffffu); f[1] = bf16_to_f32(r.x >> 16);
    f[2] = bf16_to_f32(r.y & 0xffffu); f[3] = bf16_to_f32(r.y >> 16);
    f[4] = bf16_to_f32(r.z & 0xffffu); f[5] = bf16_to_f32(r.z >> 16);
    f[6] = bf16_to_f32(r.w & 0xffffu); f[7] = bf16_to_f32(r.w >> 16);
}

// Expert outputs are read exactly once: their loads carry the nontemporal hint, which
// measured 12% faster at prefill (940 MB of y_sorted) than plain loads.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_once(const uint4* p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// One wave per (token, 1024-column slice); lane L owns 16-B chunks L and L + 64 of the
// slice. The token's K source rows and weights are read once (lanes < K) and broadcast by
// lane reads; for each batch of up to 8 choices every load of both chunks is issued before
// any is accumulated, so a lane keeps up to 16 loads in flight.
constexpr int kSliceChunks = 128;  // 16-B chunks (8 bf16) per wave slice

__global__ __launch_bounds__(256) void k_combine(const uint16_t* __restrict__ y, const int32_t* __restrict__ slot_pos,
                                                 const float* __restrict__ w, const uint16_t* __restrict__ shared,
                                                 const uint16_t* residual, int64_t N, int K, int d, uint16_t* out) {
    const int lane = threadIdx.x & 63;
    const int chunks = d / 8;
    const int slices = (chunks + kSliceChunks - 1) / kSliceChunks;
    const int64_t wv = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t n = wv / slices;
    if (n >= N) return;  // uniform over the wave
    const int c0 = (int)(wv % slices) * kSliceChunks + lane;
    const int64_t NK = N * K;
    int32_t my_p = -1;
    float my_w = 0.0f;
    if (lane < K) {
        const int32_t p = slot_pos[n * K + lane];
        my_p = (p >= 0 && p < NK) ? p : -1;
        my_w = w[n * K + lane];
    }
    const bool v0 = c0 < chunks, v1 = c0 + 64 < chunks;
    float acc[2][8];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[j][i] = 0.0f;
    for (int k0 = 0; k0 < K; k0 += 8) {
        uint4 r[8][2];
        int32_t pk[8];
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            const int k = k0 + kk < K ? k0 + kk : K - 1;
            pk[kk] = __shfl(my_p, k);
            const bool ok = k0 + kk < K && pk[kk] >= 0;
            const uint4* src = reinterpret_cast<const uint4*>(y + (int64_t)(ok ? pk[kk] : 0) * d) + c0;
            r[kk][0] = (ok && v0) ? load_once(src) : make_uint4(0, 0, 0, 0);
            r[kk][1] = (ok && v1) ? load_once(src + 64) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            const int k = k0 + kk < K ? k0 + kk : K - 1;
            const float wk = __shfl(my_w, k);
            if (k0 + kk < K && pk[kk] >= 0) {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    float f[8];
                    unpack8(r[kk][j], f);
#pragma unroll
                    for (int i = 0; i < 8; ++i) acc[j][i] += wk * f[i];
                }
            }
        }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int c = c0 + 64 * j;
        if (c >= chunks) continue;
        if (shared) {
            float f[8];
            unpack8(*(reinterpret_cast<const uint4*>(shared + n * d) + c), f);
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[j][i] += f[i];
        }
        if (residual) {
            float f[8];
            unpack8(*(reinterpret_cast<const uint4*>(residual + n * d) + c), f);
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[j][i] += f[i];
        }
        uint4 o;
        o.x = f32_to_bf16(acc[j][0]) | (f32_to_bf16(acc[j][1]) << 16);
        o.y = f32_to_bf16(acc[j][2]) | (f32_to_bf16(acc[j][3]) << 16);
        o.z = f32_to_bf16(acc[j][4]) | (f32_to_bf16(acc[j][5]) << 16);
        o.w = f32_to_bf16(acc[j][6]) | (f32_to_bf16(acc[j][7]) << 16);
        *(reinterpret_cast<uint4*>(out + n * d) + c) = o;
    }
}

hipError_t launch_combine(const uint16_t* y, const int32_t* slot_pos, const float* w, const uint16_t* shared,
                          const uint16_t* residual, int64_t N, int K, int d, uint16_t* out, hipStream_t stream) {
    if (N == 0) return hipSuccess;
    const int64_t slices = (d / 8 + kSliceChunks - 1) / kSliceChunks;
    const int64_t blocks = (N * slices + 3) / 4;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_combine, dim3((unsigned)blocks), dim3(256), 0, stream, y, slot_pos, w, shared, residual, N,
                       K, d, out);
    return hipGetLastError();
}

}  // namespace moe
