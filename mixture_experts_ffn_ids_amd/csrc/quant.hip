// Dynamic e4m3 quantisation of bfloat16 rows, one float32 scale per 128 values.
// ("Input features" page, evidence "linear": activation_scheme dynamic, fmt e4m3.)
//
// Memory-bound: each group of 16 lanes owns one 128-value group; a lane loads 8
// bf16 (16 B), the group's largest magnitude is reduced across the 16 lanes with
// xor shuffles, then every lane divides by the scale (IEEE division) and stores
// 8 codes (8 B).
#include "moe_internal.h"

namespace moe {

__global__ __launch_bounds__(256) void k_quantize_rows(const uint16_t* __restrict__ x, int64_t groups,
                                                       int cols, uint8_t* __restrict__ q,
                                                       float* __restrict__ s) {
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int sub = threadIdx.x & 15;
    const int gpr = cols / kGroup;  // groups per row
    // every lane of a 16-lane group runs the same number of iterations (groups*16 rounded
    // to the grid stride keeps whole groups together), so the shuffles below are uniform
    for (int64_t t = tid; t < ((groups * 16 + stride - 1) / stride) * stride; t += stride) {
        const int64_t g = t >> 4;
        const bool valid = g < groups;
        const int64_t row = valid ? g / gpr : 0;
        const int64_t col = valid ? (g % gpr) * kGroup + sub * 8 : 0;
        uint4 raw = make_uint4(0, 0, 0, 0);
        if (valid) raw = *reinterpret_cast<const uint4*>(x + row * cols + col);
        float v[8];
        v[0] = bf16_to_f32(raw.x & 0xffffu); v[1] = bf16_to_f32(raw.x >> 16);
        v[2] = bf16_to_f32(raw.y & 0xffffu); v[3] = bf16_to_f32(raw.y >> 16);
        v[4] = bf16_to_f32(raw.z & 0xffffu); v[5] = bf16_to_f32(raw.z >> 16);
        v[6] = bf16_to_f32(raw.w & 0xffffu); v[7] = bf16_to_f32(raw.w >> 16);
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[i]));
#pragma unroll
        for (int m = 8; m >= 1; m >>= 1) amax = __builtin_fmaxf(amax, __shfl_xor(amax, m, 16));
        const float sc = group_scale(amax);
        uint32_t lo = f32x2_to_e4m3(v[0] / sc, v[1] / sc) | (f32x2_to_e4m3(v[2] / sc, v[3] / sc) << 16);
        uint32_t hi = f32x2_to_e4m3(v[4] / sc, v[5] / sc) | (f32x2_to_e4m3(v[6] / sc, v[7] / sc) << 16);
        if (valid) {
            *reinterpret_cast<uint2*>(q + row * cols + col) = make_uint2(lo, hi);
            if (sub == 0) s[row * gpr + col / kGroup] = sc;
        }
    }
}

hipError_t launch_quantize_rows(const uint16_t* x, int64_t rows, int cols, uint8_t* q, float* s,
                                hipStream_t stream) {
    const int64_t groups = rows * (cols / kGroup);
    if (groups == 0) return hipSuccess;
    const int64_t threads = groups * 16;
    int64_t blocks = (threads + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(k_quantize_rows, dim3((unsigned)blocks), dim3(256), 0, stream, x, groups, cols, q, s);
    return hipGetLastError();
}

}  // namespace moe
