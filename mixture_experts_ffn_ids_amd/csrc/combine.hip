// Weighted combine ("Mixture of experts" page, Code: moe_infer's weighted sum of
// each token's K expert outputs, and forward's addition of the shared expert):
//   out[n] = bf16( sum_{k<K} w[n][k] * y_sorted[slot_pos[n*K+k]] + shared[n] )
// float32, ascending k, shared term last, one nearest-even rounding. Each
// workgroup owns whole tokens and writes every output element exactly once, so
// no atomics are needed and the result is deterministic.
//
// Memory-bound: a lane moves 8 bf16 (16 B) per row per step; the K source rows of
// a token are 14 KB contiguous runs at K2 shapes.
#include "moe_internal.h"

namespace moe {

__device__ __forceinline__ void unpack8(const uint4 r, float (&f)[8]) {
    f[0] = bf16_to_f32(r.x & 0xffffu); f[1] = bf16_to_f32(r.x >> 16);
    f[2] = bf16_to_f32(r.y & 0xffffu); f[3] = bf16_to_f32(r.y >> 16);
    f[4] = bf16_to_f32(r.z & 0xffffu); f[5] = bf16_to_f32(r.z >> 16);
    f[6] = bf16_to_f32(r.w & 0xffffu); f[7] = bf16_to_f32(r.w >> 16);
}

__global__ __launch_bounds__(256) void k_combine(const uint16_t* __restrict__ y, const int32_t* __restrict__ slot_pos,
                                                 const float* __restrict__ w, const uint16_t* __restrict__ shared,
                                                 int64_t N, int K, int d, uint16_t* __restrict__ out) {
    __shared__ int64_t sPos[kMaxTopK];
    __shared__ float sW[kMaxTopK];
    const int64_t NK = N * K;
    for (int64_t n = blockIdx.x; n < N; n += gridDim.x) {
        __syncthreads();
        if (threadIdx.x < K) {
            const int32_t p = slot_pos[n * K + threadIdx.x];
            sPos[threadIdx.x] = (p >= 0 && p < NK) ? (int64_t)p : -1;
            sW[threadIdx.x] = w[n * K + threadIdx.x];
        }
        __syncthreads();
        for (int c = threadIdx.x * 8; c < d; c += blockDim.x * 8) {
            float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            for (int k = 0; k < K; ++k) {
                const int64_t p = sPos[k];
                if (p < 0) continue;
                float f[8];
                unpack8(*reinterpret_cast<const uint4*>(y + p * d + c), f);
                const float wk = sW[k];
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] += wk * f[i];
            }
            if (shared) {
                float f[8];
                unpack8(*reinterpret_cast<const uint4*>(shared + n * d + c), f);
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] += f[i];
            }
            uint4 o;
            o.x = f32_to_bf16(acc[0]) | (f32_to_bf16(acc[1]) << 16);
            o.y = f32_to_bf16(acc[2]) | (f32_to_bf16(acc[3]) << 16);
            o.z = f32_to_bf16(acc[4]) | (f32_to_bf16(acc[5]) << 16);
            o.w = f32_to_bf16(acc[6]) | (f32_to_bf16(acc[7]) << 16);
            *reinterpret_cast<uint4*>(out + n * d + c) = o;
        }
    }
}

hipError_t launch_combine(const uint16_t* y, const int32_t* slot_pos, const float* w, const uint16_t* shared,
                          int64_t N, int K, int d, uint16_t* out, hipStream_t stream) {
    if (N == 0) return hipSuccess;
    const int64_t blocks = N < 65536 ? N : 65536;
    hipLaunchKernelGGL(k_combine, dim3((unsigned)blocks), dim3(256), 0, stream, y, slot_pos, w, shared, N, K, d, out);
    return hipGetLastError();
}

}  // namespace moe
