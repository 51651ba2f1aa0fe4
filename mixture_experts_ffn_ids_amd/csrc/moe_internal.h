// Internal declarations shared by the HIP sources of libmoe (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <type_traits>
#include <stdint.h>

#include "moe.h"

namespace moe {

constexpr int kGroup = 128;          // quantisation block edge (weight_block_size 128 x 128)
constexpr int kMaxTopK = 64;         // MOE_MAX_TOPK
constexpr float kE4m3Max = 448.0f;   // largest finite OCP e4m3 magnitude

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- number formats
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// float -> bfloat16 bits, nearest-even: the hardware conversion (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

// Saturation to the largest finite e4m3 magnitude: |v| > 448 (infinities included) becomes
// +-448. A NaN fails the comparison and passes through unchanged, so it is encoded as a NaN
// code (the format has no infinity, and NaN is its only non-finite value).
__device__ __forceinline__ float sat_e4m3(float v) {
    return __builtin_fabsf(v) > kE4m3Max ? __builtin_copysignf(kE4m3Max, v) : v;
}

// Two floats -> two OCP e4m3 codes (nearest-even) in the low 16 bits; out-of-range values
// saturate to +-448 first, NaNs give a NaN code (exponent and mantissa bits all ones).
__device__ __forceinline__ uint32_t f32x2_to_e4m3(float a, float b) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(sat_e4m3(a), sat_e4m3(b), 0, false) & 0xffffu;
}

// silu(z) = z * sigmoid(z) with the hardware exponential and reciprocal (a few ulp; the
// product is requantised to 3 mantissa bits right after).
__device__ __forceinline__ float silu_fast(float z) {
    return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

// Per-group scale from the group's largest magnitude: amax/448, or 1 for a zero group.
__device__ __forceinline__ float group_scale(float amax) {
    return amax > 0.0f ? amax / kE4m3Max : 1.0f;
}

// The values to encode, v / s, for the requantisation of h inside the GEMM epilogues: v times
// the correctly rounded reciprocal of s (one division per group instead of one per value).
// The product can differ from the quotient by an ulp, which moves an e4m3 code only when the
// quotient lies within an ulp of a rounding midpoint. A subnormal s (reciprocal out of
// range) takes the division; the branch is skipped unless some lane needs it.
template <int NV>
__device__ __forceinline__ void scale_group(float (&v)[NV], float s) {
    if (s < 0x1p-126f) {
#pragma unroll
        for (int k = 0; k < NV; ++k) v[k] = v[k] / s;
    } else {
        const float inv = 1.0f / s;
#pragma unroll
        for (int k = 0; k < NV; ++k) v[k] = v[k] * inv;
    }
}

// 16x16x128 FP8 x FP8 -> FP32 matrix core op with unit block scales (E8M0 127 = 2^0).
// Lane l supplies row (l & 15) of A and column (l & 15) of B, 32 K-values each;
// the result holds D[4*(l>>4) + i][l & 15] in element i.
// Its sum is not exact: measured on gfx950, the FP8 ops (this one and the 16x16x32 and
// 32x32x64 forms alike) add their products in groups and align the group sums to the largest
// one, dropping the bits below about 2^-14 of it (448*448 + 127*1 gives 200824, not 200831);
// the error is up to ~7e-5 of the sum of |products|. Used where the result is not requantised
// (the down projection), so that error stays far below the output tolerance.
__device__ __forceinline__ v4f mfma_16x16x128_fp8(const v8i& a, const v8i& b) {
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 127, 0, 127);
}

// The same 128-wide block product with the sum formed exactly (to float32 rounding): every
// e4m3 value is a bfloat16 value, so the fragment is widened to bfloat16 (one conversion per
// two codes) and multiplied by four chained 16x16x32 bf16 ops, whose products and sums are
// exact up to float32 roundings (measured: 448*448 + 127*1 gives 200831; error about 3e-8 of
// the sum of |products|). Used for gate|up, whose results are requantised: an accumulation
// error there moves e4m3 codes of h across rounding midpoints, and a moved code of a large h
// element alone can exceed the output tolerance.
// Widened fragment: k[j] holds the 8 values of bytes [8j, 8j+8) of the lane's 32 K-bytes, so
// op j covers K-values 32 (l >> 4) + 8j + (0..7) for A and B alike, and the four ops together
// the whole block.
// The widening is v_cvt_scalef32_pk_bf16_fp8 with a unit scale held in a register: op_sel 0
// converts bytes 0 and 1 of the source, op_sel 1 bytes 2 and 3, one instruction per two codes.
// Measured on gfx950 over all 256 codes, written this way it reproduces every value (and gives
// NaN for the NaN codes). The compiler builtin of the same instruction, which encodes the scale
// as an inline constant, was measured to repeat the first value of each pair instead.
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
struct Frag16 {
    v8bf k[4];
};
__device__ __forceinline__ uint32_t widen2(uint32_t w, float one, std::false_type) {
    uint32_t r;
    asm("v_cvt_scalef32_pk_bf16_fp8 %0, %1, %2" : "=v"(r) : "v"(w), "v"(one));
    return r;
}
__device__ __forceinline__ uint32_t widen2(uint32_t w, float one, std::true_type) {
    uint32_t r;
    asm("v_cvt_scalef32_pk_bf16_fp8 %0, %1, %2 op_sel:[1,0,0]" : "=v"(r) : "v"(w), "v"(one));
    return r;
}
__device__ __forceinline__ v8bf widen8(uint32_t lo, uint32_t hi) {
    const float one = 1.0f;
    typedef uint32_t v4u __attribute__((ext_vector_type(4)));
    const v4u r = {widen2(lo, one, std::false_type{}), widen2(lo, one, std::true_type{}),
                   widen2(hi, one, std::false_type{}), widen2(hi, one, std::true_type{})};
    return __builtin_bit_cast(v8bf, r);
}
__device__ __forceinline__ Frag16 widen(const v8i& f) {
    Frag16 w;
#pragma unroll
    for (int j = 0; j < 4; ++j) w.k[j] = widen8((uint32_t)f[2 * j], (uint32_t)f[2 * j + 1]);
    return w;
}
__device__ __forceinline__ v4f mfma_block_exact(const Frag16& a, const Frag16& b) {
    v4f c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.k[j], b.k[j], c, 0, 0, 0);
    return c;
}
// Four such block products sharing the second operand, r[n] = a[n] . b, with their chains
// interleaved (quarter q of every product before quarter q + 1 of any), so that no matrix op
// waits for the one just issued. Each r[n] is summed in the same order as mfma_block_exact.
__device__ __forceinline__ void mfma_block_exact4(const Frag16 (&a)[4], const Frag16& b, v4f (&r)[4]) {
#pragma unroll
    for (int n = 0; n < 4; ++n) r[n] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int n = 0; n < 4; ++n) r[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[n].k[q], b.k[q], r[n], 0, 0, 0);
}

// ---------------------------------------------------------------- launchers

// Keeps e as the value moe_last_hip_error() reports on this thread; returns MOE_ERR_HIP.
moe_status record_hip_error(hipError_t e);

hipError_t launch_rmsnorm_quantize(const uint16_t* x, const uint16_t* gain, float eps, int64_t rows, int cols,
                                   uint16_t* y, uint8_t* q, float* s, hipStream_t stream);

constexpr int kDispatchChunk = 256;
constexpr int kSmallDispatch = 8192;         // slots up to which one workgroup does the whole dispatch
constexpr int kSmallDispatchExperts = 4096;  // and experts (its two LDS tables stay within 32 KB)
hipError_t launch_dispatch(const int32_t* ids, int64_t N, int K, int E, int32_t* counts,
                           int32_t* offsets, int32_t* sorted_slot, int32_t* slot_pos,
                           int32_t* chunk_counts, int32_t* err_flag, bool checked,
                           hipStream_t stream);

// Tile list: one entry per (expert, block of up to BM sorted rows), experts in order.
// first/count: index of the expert's first tile and its number of tiles.
struct Tile {
    int32_t expert;
    int32_t row_begin;
    int32_t row_end;
    int32_t first;
    int32_t count;
    int32_t pad[3];
};

int64_t max_tiles(int64_t rows, int E, int BM);

// Block-wide exclusive scan of one value per thread (up to 1024 threads = 16 waves).
template <typename T>
__device__ T block_exclusive_scan(T v, T* total) {
    __shared__ T wsum[16];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    T incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        T t = __shfl_up(incl, off, 64);
        if (lane >= off) incl += t;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    T base = 0, all = 0;
    const int nw = blockDim.x >> 6;
    for (int w = 0; w < nw; ++w) {
        if (w < wave) base += wsum[w];
        all += wsum[w];
    }
    __syncthreads();
    *total = all;
    return base + incl - v;
}

// num_tiles[0]: tiles written; num_tiles[1]: 1 when every expert with rows got one tile
// Run by one whole workgroup (any size up to 1024 threads, a multiple of 64).
__device__ inline void build_tiles_block(const int32_t* __restrict__ offsets, int E, int64_t rows, int BM,
                                         int64_t cap, Tile* __restrict__ tiles, int32_t* __restrict__ num_tiles) {
    // each thread owns a contiguous range of experts; offsets are clamped to [0, rows]
    // so that any offsets array yields in-bounds tiles
    const int per = (E + blockDim.x - 1) / blockDim.x;
    const int e0 = threadIdx.x * per;
    int64_t local = 0, local_busy = 0;
    for (int e = e0; e < e0 + per && e < E; ++e) {
        int64_t b = offsets[e], en = offsets[e + 1];
        b = b < 0 ? 0 : (b > rows ? rows : b);
        en = en < b ? b : (en > rows ? rows : en);
        local += (en - b + BM - 1) / BM;
        local_busy += en > b ? 1 : 0;
    }
    int64_t total, busy;
    block_exclusive_scan<int64_t>(local_busy, &busy);
    int64_t t = block_exclusive_scan<int64_t>(local, &total);
    for (int e = e0; e < e0 + per && e < E; ++e) {
        int64_t b = offsets[e], en = offsets[e + 1];
        b = b < 0 ? 0 : (b > rows ? rows : b);
        en = en < b ? b : (en > rows ? rows : en);
        const int64_t first = t;
        const int64_t count = (en - b + BM - 1) / BM;
        // stops at the cap, so arbitrary offsets cannot make this loop long
        for (int64_t r = b; r < en && t < cap; r += BM, ++t) {
            Tile tl;
            tl.expert = e;
            tl.row_begin = (int32_t)r;
            tl.row_end = (int32_t)(r + BM < en ? r + BM : en);
            tl.first = (int32_t)first;
            tl.count = (int32_t)count;
            tl.pad[0] = tl.pad[1] = tl.pad[2] = 0;
            tiles[t] = tl;
        }
    }
    if (threadIdx.x == 0) {
        num_tiles[0] = (int32_t)(total < cap ? total : cap);
        // every expert with rows fits one tile: each weight block is then read by one
        // workgroup only
        num_tiles[1] = total == busy && total <= cap ? 1 : 0;
    }
}


// A tile list to build (build_tiles_block's arguments); tiles == NULL: none.
struct TileJob {
    const int32_t* offsets; int E; int64_t rows; int BM; int64_t cap; Tile* tiles; int32_t* num_tiles;
};

// Rows of out[rows][cols] (bf16, the shape of the quantised x) to set to +0: those whose
// slot_pos entry lies outside [0, slots), i.e. the tokens a top-1 dispatch left out, which
// no GEMM epilogue writes. out == NULL: none.
struct ZeroRowsJob {
    const int32_t* slot_pos; int64_t slots; uint16_t* out;
};

// Dynamic e4m3 quantisation of rows; with tile_job, the same launch also builds that tile list;
// with zero_job, it also zeroes those rows of zero_job->out.
hipError_t launch_quantize_rows(const uint16_t* x, int64_t rows, int cols, uint8_t* q, float* s,
                                hipStream_t stream, const TileJob* tile_job = nullptr,
                                const ZeroRowsJob* zero_job = nullptr);

// num_tiles[2]: the number of tiles, and 1 if every expert with rows got exactly one tile
hipError_t launch_build_tiles(const int32_t* offsets, int E, int64_t rows, int BM, int64_t max_tiles,
                              Tile* tiles, int32_t* num_tiles, hipStream_t stream);

enum class TileShape { Rows16 = 0, Rows128 = 1, Rows192 = 2, Rows224 = 3, Rows256 = 4 };
int tile_rows(TileShape shape);   // BM of the gate|up and down kernels for this shape

struct GateUpArgs {
    const uint8_t* xq;      // [N][d] e4m3
    const float* xs;        // [N][d/128]
    const int32_t* sorted_slot;
    int64_t N;
    int K;
    int64_t rows;           // N*K
    int d, d_ff;
    const uint8_t* wg; const float* sg;
    const uint8_t* wu; const float* su;
    const Tile* tiles; const int32_t* num_tiles; int64_t max_tiles;
    uint8_t* hq;            // [rows][d_ff]
    float* hs;              // [rows][d_ff/128]
};

struct DownArgs {
    const uint8_t* hq; const float* hs;
    int64_t rows;
    int d, d_ff;
    const uint8_t* wd; const float* sd;
    const Tile* tiles; const int32_t* num_tiles; int64_t max_tiles;
    uint16_t* y;            // [rows][d] bf16 in sorted order, or [out_rows][d] with scatter
    // top-1 combine in the epilogue (NULL: none): sorted row p goes to row scatter[p] of y,
    // times scatter_w[scatter[p]]; rows whose target lies outside [0, out_rows) are dropped
    const int32_t* scatter; const float* scatter_w; int64_t out_rows;
};

hipError_t launch_gate_up(const GateUpArgs& a, TileShape shape, hipStream_t stream);
hipError_t launch_down(const DownArgs& a, TileShape shape, hipStream_t stream);

// LDS-staged kernels for tiles of 128, 192, 224 or 256 rows (gemm_lds.hip)
hipError_t launch_gate_up_lds(const GateUpArgs& a, int rows, hipStream_t stream);
hipError_t launch_down_lds(const DownArgs& a, int rows, hipStream_t stream);


hipError_t launch_combine(const uint16_t* y, const int32_t* slot_pos, const float* w,
                          const uint16_t* shared, const uint16_t* residual, int64_t N, int K, int d,
                          uint16_t* out, hipStream_t stream);

}  // namespace moe
