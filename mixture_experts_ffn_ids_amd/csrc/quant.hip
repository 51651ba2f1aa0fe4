// Dynamic e4m3 quantisation of bfloat16 rows, one float32 scale per 128 values.
// ("Input features" page, evidence "linear": activation_scheme dynamic, fmt e4m3.)
//
// Memory-bound: each group of 16 lanes owns 128-value groups; a lane loads 8 bf16
// (16 B) of a group, the group's largest magnitude is reduced across the 16 lanes
// with xor shuffles, then every lane divides by the scale (the IEEE quotient, by a
// correction of the product with the reciprocal) and stores 8 codes (8 B).
#include "moe_internal.h"

namespace moe {

// v / s rounded to nearest even in binary32, the IEEE quotient, from r = 1/s (itself the
// IEEE quotient): q = v r is within an ulp of v / s, the fused multiply-add gives the remainder
// v - q s, and q + (v - q s) r rounded once is the correctly rounded quotient (Markstein's
// correction). Two fused multiply-adds per value instead of a full division; the caller keeps
// s finite and >= 2^-100, so that neither the remainder nor its product with r underflows. A
// zero result takes q's sign (that of v), as the division would.
__device__ __forceinline__ float div_by_scale(float v, float s, float r) {
    const float q = v * r;
    const float rem = __builtin_fmaf(-q, s, v);
    const float out = __builtin_fmaf(rem, r, q);
    return out == 0.0f ? q : out;
}

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
    float q[8];
    if (sc >= 0x1p-100f && sc <= 0x1.fffffep127f) {   // an infinite amax divides, as before
        const float r = 1.0f / sc;
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = div_by_scale(v[i], sc, r);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = v[i] / sc;
    }
    codes.x = f32x2_to_e4m3(q[0], q[1]) | (f32x2_to_e4m3(q[2], q[3]) << 16);
    codes.y = f32x2_to_e4m3(q[4], q[5]) | (f32x2_to_e4m3(q[6], q[7]) << 16);
    scale = sc;
}

// Each 16-lane group quantises two consecutive 128-value groups per step (both loads in
// flight before either is reduced). With a tile job, the last workgroup builds the GEMM tile
// list instead (it does not depend on the quantised rows), which saves a launch.
__global__ __launch_bounds__(256) void k_quantize_rows(const uint16_t* __restrict__ x, int64_t groups,
                                                       int cols, uint8_t* __restrict__ q,
                                                       float* __restrict__ s, const TileJob job,
                                                       const ZeroRowsJob zj) {
    const int qblocks = gridDim.x - (job.tiles ? 1 : 0);
    if ((int)blockIdx.x == qblocks) {   // only with a tile job
        build_tiles_block(job.offsets, job.E, job.rows, job.BM, job.cap, job.tiles, job.num_tiles);
        return;
    }
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)qblocks * blockDim.x;
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
        int32_t pos[2] = {0, 0};   // with the zero-rows job: the row's slot_pos entry
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int64_t g = g0 + h;
            valid[h] = g < groups;
            const int64_t row = valid[h] ? g / gpr : 0;
            off[h] = row * cols + (valid[h] ? (g % gpr) * kGroup + sub * 8 : 0);
            raw[h] = valid[h] ? *reinterpret_cast<const uint4*>(x + off[h]) : make_uint4(0, 0, 0, 0);
            // loaded with the row, so that its latency overlaps the row's
            if (zj.out && valid[h]) pos[h] = zj.slot_pos[row];
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            uint2 codes;
            float sc;
            quant_group(raw[h], codes, sc);
            if (valid[h]) {
                *reinterpret_cast<uint2*>(q + off[h]) = codes;
                if (sub == 0) s[(g0 + h)] = sc;
                if (zj.out) {   // a token left out by the dispatch: its output row is +0
                    if (pos[h] < 0 || pos[h] >= zj.slots)
                        *reinterpret_cast<uint4*>(zj.out + off[h]) = make_uint4(0, 0, 0, 0);
                }
            }
        }
    }
}

__global__ __launch_bounds__(256) void k_tiles_only(const TileJob job) {
    build_tiles_block(job.offsets, job.E, job.rows, job.BM, job.cap, job.tiles, job.num_tiles);
}

// RMSNorm of a bfloat16 row with a bfloat16 gain, fused with the e4m3 quantisation of the
// result ("Input features" page, evidence "rmsnorm": float32 normalisation, back to the
// input dtype, then the gain; evidence "linear": dynamic e4m3 per 128 values). One
// workgroup per row; thread t owns the 16-B chunks t, t + 256, ..., so chunk c is lane c % 16
// of 128-value group c / 16 in both passes:
//   pass 1: the sum of squares in double (a bf16 value squared is exact in double), reduced
//           over the workgroup; v = fp32(sum / cols), r = fp32(1 / sqrt(fp32(v + eps)));
//   pass 2: t = bf16(x * r), y = bf16(g * t) -- g * t is exact in float32 -- optionally
//           stored, then quantised exactly as k_quantize_rows does.
// The first KEEP chunks of each thread stay in registers between the passes (rows of up to
// 256 * 8 * KEEP values are read once); chunks beyond them are read again, from L2.
constexpr int kNormKeep = 8;

__global__ __launch_bounds__(256) void k_rmsnorm_quantize(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ gain, float eps,
                                                          int cols, uint16_t* __restrict__ y,
                                                          uint8_t* __restrict__ q, float* __restrict__ s) {
    __shared__ double red[4];
    const int64_t row = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint16_t* xr = x + row * cols;
    const int chunks = cols / 8;
    const int iters = (chunks + 255) / 256;   // the same for every thread
    uint4 keep[kNormKeep];
    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < kNormKeep; ++i) {
        const int c = threadIdx.x + 256 * i;
        keep[i] = (i < iters && c < chunks) ? *reinterpret_cast<const uint4*>(xr + c * 8) : make_uint4(0, 0, 0, 0);
    }
    for (int i = 0; i < iters; ++i) {
        const int c = threadIdx.x + 256 * i;
        uint4 raw;
        if (i < kNormKeep) {
#pragma unroll
            for (int k = 0; k < kNormKeep; ++k)
                if (k == i) raw = keep[k];
        } else {
            raw = c < chunks ? *reinterpret_cast<const uint4*>(xr + c * 8) : make_uint4(0, 0, 0, 0);
        }
        const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const double a = bf16_to_f32(w4[k] & 0xffffu), b = bf16_to_f32(w4[k] >> 16);
            ss += a * a;
            ss += b * b;
        }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m);
    if (lane == 0) red[wave] = ss;
    __syncthreads();
    const double total = (red[0] + red[1]) + (red[2] + red[3]);
    const float var = (float)(total / (double)cols);
    const float r = (float)(1.0 / sqrt((double)(var + eps)));

    // pass 2; a 16-lane group is one 128-value group, and all 16 lanes of it run every
    // iteration, so the shuffles inside quant_group stay uniform
    const int groups = cols / kGroup;
    const int sub = threadIdx.x & 15;
    for (int i = 0; i < iters; ++i) {
        const int c = threadIdx.x + 256 * i;
        const int g = c >> 4;
        const bool valid = c < chunks;
        uint4 raw;
        if (i < kNormKeep) {
#pragma unroll
            for (int k = 0; k < kNormKeep; ++k)
                if (k == i) raw = keep[k];
        } else {
            raw = valid ? *reinterpret_cast<const uint4*>(xr + c * 8) : make_uint4(0, 0, 0, 0);
        }
        const uint4 graw = valid ? *reinterpret_cast<const uint4*>(gain + c * 8) : make_uint4(0, 0, 0, 0);
        const uint32_t xv[4] = {raw.x, raw.y, raw.z, raw.w};
        const uint32_t gv[4] = {graw.x, graw.y, graw.z, graw.w};
        uint32_t yv[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float t0 = bf16_to_f32(f32_to_bf16(bf16_to_f32(xv[k] & 0xffffu) * r));
            const float t1 = bf16_to_f32(f32_to_bf16(bf16_to_f32(xv[k] >> 16) * r));
            yv[k] = f32_to_bf16(bf16_to_f32(gv[k] & 0xffffu) * t0) |
                    (f32_to_bf16(bf16_to_f32(gv[k] >> 16) * t1) << 16);
        }
        const uint4 yn = make_uint4(yv[0], yv[1], yv[2], yv[3]);
        if (valid && y) *reinterpret_cast<uint4*>(y + row * cols + c * 8) = yn;
        uint2 codes;
        float sc;
        quant_group(yn, codes, sc);
        if (valid) {
            *reinterpret_cast<uint2*>(q + row * cols + c * 8) = codes;
            if (sub == 0) s[row * groups + g] = sc;
        }
    }
}

hipError_t launch_rmsnorm_quantize(const uint16_t* x, const uint16_t* gain, float eps, int64_t rows, int cols,
                                   uint16_t* y, uint8_t* q, float* s, hipStream_t stream) {
    if (rows == 0) return hipSuccess;
    if (rows > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_rmsnorm_quantize, dim3((unsigned)rows), dim3(256), 0, stream, x, gain, eps, cols, y, q, s);
    return hipGetLastError();
}

hipError_t launch_quantize_rows(const uint16_t* x, int64_t rows, int cols, uint8_t* q, float* s,
                                hipStream_t stream, const TileJob* tile_job, const ZeroRowsJob* zero_job) {
    const int64_t groups = rows * (cols / kGroup);
    const TileJob job = tile_job ? *tile_job : TileJob{};
    const ZeroRowsJob zj = zero_job ? *zero_job : ZeroRowsJob{};
    if (groups == 0) {
        if (job.tiles)
            hipLaunchKernelGGL(k_tiles_only, dim3(1), dim3(256), 0, stream, job);
        return hipGetLastError();
    }
    const int64_t threads = (groups + 1) / 2 * 16;
    int64_t blocks = (threads + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (job.tiles) ++blocks;
    hipLaunchKernelGGL(k_quantize_rows, dim3((unsigned)blocks), dim3(256), 0, stream, x, groups, cols, q, s, job,
                       zj);
    return hipGetLastError();
}

}  // namespace moe
