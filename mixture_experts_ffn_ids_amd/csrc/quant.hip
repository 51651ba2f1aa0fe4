// Dynamic e4m3 quantisation of bfloat16 rows, one float32 scale per 128 values.
// ("Input features" page, evidence "linear": activation_scheme dynamic, fmt e4m3.)
//
// Memory-bound: each group of 16 lanes owns 128-value groups; a lane loads 8 bf16
// (16 B) of a group, the group's largest magnitude is reduced across the 16 lanes
// with xor shuffles, then every lane divides by the scale (IEEE division) and stores
// 8 codes (8 B).
#include "moe_internal.h"

namespace moe {

// One 128-value group: lane `sub` of its 16 holds values 8 sub .. 8 sub + 7 in raw.
__device__ __forceinline__ void quant_group(const uint4 raw, uint2& codes, float& scale) {
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
    codes.x = f32x2_to_e4m3(v[0] / sc, v[1] / sc) | (f32x2_to_e4m3(v[2] / sc, v[3] / sc) << 16);
    codes.y = f32x2_to_e4m3(v[4] / sc, v[5] / sc) | (f32x2_to_e4m3(v[6] / sc, v[7] / sc) << 16);
    scale = sc;
}

// Each 16-lane group quantises two consecutive 128-value groups per step (both loads in
// flight before either is reduced).
__global__ __launch_bounds__(256) void k_quantize_rows(const uint16_t* __restrict__ x, int64_t groups,
                                                       int cols, uint8_t* __restrict__ q,
                                                       float* __restrict__ s) {
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int sub = threadIdx.x & 15;
    const int gpr = cols / kGroup;  // groups per row
    const int64_t pairs = (groups + 1) / 2;
    // every lane of a 16-lane group runs the same number of iterations (pairs*16 rounded to
    // the grid stride keeps whole groups together), so the shuffles below are uniform
    for (int64_t t = tid; t < ((pairs * 16 + stride - 1) / stride) * stride; t += stride) {
        const int64_t g0 = (t >> 4) * 2;
        uint4 raw[2];
        bool valid[2];
        int64_t off[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int64_t g = g0 + h;
            valid[h] = g < groups;
            const int64_t row = valid[h] ? g / gpr : 0;
            off[h] = row * cols + (valid[h] ? (g % gpr) * kGroup + sub * 8 : 0);
            raw[h] = valid[h] ? *reinterpret_cast<const uint4*>(x + off[h]) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            uint2 codes;
            float sc;
            quant_group(raw[h], codes, sc);
            if (valid[h]) {
                *reinterpret_cast<uint2*>(q + off[h]) = codes;
                if (sub == 0) s[(g0 + h)] = sc;
            }
        }
    }
}

hipError_t launch_quantize_rows(const uint16_t* x, int64_t rows, int cols, uint8_t* q, float* s,
                                hipStream_t stream) {
    const int64_t groups = rows * (cols / kGroup);
    if (groups == 0) return hipSuccess;
    const int64_t threads = (groups + 1) / 2 * 16;
    int64_t blocks = (threads + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(k_quantize_rows, dim3((unsigned)blocks), dim3(256), 0, stream, x, groups, cols, q, s);
    return hipGetLastError();
}

}  // namespace moe
