// Grouped FP8 GEMMs of the routed experts on CDNA4 matrix cores.
//
//   gate|up:  G, U [rows of expert e][d_ff] = Xq[rows] . W_gate[e]^T, . W_up[e]^T
//             then h = silu(G) * U requantised to e4m3 per 128 features
//             ("SwiGLU output" page, evidence "mlp"; "Element-wise product" page,
//             h = a (.) u with a = silu(gate x));
//   down:     Y [rows][d] = Hq[rows] . W_down[e]^T, stored as bfloat16.
// Weights are e4m3 with one float32 scale per 128 x 128 block, activations e4m3
// with one float32 scale per row per 128 features ("Input features" page,
// evidence "linear").
//
// One workgroup computes one (tile, n-block): a tile is up to BM consecutive
// sorted rows of one expert (built on the device from the dispatch offsets), an
// n-block is BN output columns (per weight tensor). The K loop walks 128-wide
// blocks: one v_mfma_scale_f32_16x16x128_f8f6f4 covers exactly one quantisation
// block, so each 16x16 partial product is scaled by (row scale x weight block
// scale) and added to the float32 accumulator -- the block-scale dequantisation
// happens in the accumulator, never on the operands.
//
// Operands: the activation tile (BM x 128 bytes per K block) is staged through
// LDS (double-buffered, rows padded to 144 bytes so 16 rows read at one column
// fall in distinct banks) because every wave of the workgroup reads it; each
// weight byte is needed by one wave only, so weights go straight from HBM into
// the MFMA operand registers, one K block ahead of use.
//
// Any 16x16x128 operand layout works as long as A and B use the same one: lane l
// supplies row (l & 15) and the 32 K-values [32*(l>>4), 32*(l>>4)+32) of its
// 128-wide block for both operands, so the hardware's K order cancels out.
#include "moe_internal.h"

namespace moe {

constexpr int kAPitch = 144;  // LDS bytes per activation row (128 + 16 pad)

struct GemmParams {
    const uint8_t* a;          // activation codes, row stride Kdim
    const float* as;           // activation scales, row stride Kdim/128
    const int32_t* gather;     // gate|up: sorted_slot (row p -> token sorted_slot[p]/K); down: NULL
    int K_top;
    int64_t src_rows;          // rows of `a` (tokens for gate|up, sorted rows for down)
    int Kdim, Ndim;
    const uint8_t* w0; const float* s0;   // gate (or down)
    const uint8_t* w1; const float* s1;   // up (gate|up only)
    const Tile* tiles; const int32_t* num_tiles;
    uint8_t* hq; float* hs;    // gate|up outputs [rows][d_ff], [rows][d_ff/128]
    uint16_t* y;               // down output [rows][d] bf16 (or [out_rows][d] with scatter)
    const int32_t* scatter; const float* scatter_w; int64_t out_rows;   // top-1 combine
};

__device__ __forceinline__ v8i load_frag_global(const uint8_t* p) {
    const uint4* q = reinterpret_cast<const uint4*>(p);
    const uint4 lo = q[0], hi = q[1];
    v8i r;
    r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
    r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
    return r;
}

__device__ __forceinline__ v8i load_frag_lds(const uint8_t* p) {
    const uint4* q = reinterpret_cast<const uint4*>(p);
    const uint4 lo = q[0], hi = q[1];
    v8i r;
    r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
    r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
    return r;
}


// MODE 0: gate|up with the silu*up requant epilogue; MODE 1: down with bf16 output.
template <int MODE, int WM, int WN, int MT, int NT>
__global__ __launch_bounds__(WM* WN * 64) void k_grouped_gemm(const GemmParams P) {
    constexpr int NTEN = MODE == 0 ? 2 : 1;
    constexpr int BM = WM * MT * 16;
    constexpr int BN = WN * NT * 16;
    constexpr int THREADS = WM * WN * 64;
    constexpr int A_CHUNKS = BM * 8;  // 16-byte chunks per activation K block
    constexpr int A_PER_THREAD = (A_CHUNKS + THREADS - 1) / THREADS;
    static_assert(128 % (NT * 16) == 0, "a wave's columns must sit in one 128-wide scale block");
    static_assert(MODE == 1 || BN == 128, "gate|up requantises whole 128-column groups");

    __shared__ __attribute__((aligned(16))) uint8_t sA[2][BM * kAPitch];
    __shared__ float sAs[2][BM];
    __shared__ int32_t sRow[BM];
    __shared__ float sRed[MODE == 0 ? WN : 1][BM];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int n_blocks = (P.Ndim + BN - 1) / BN;
    const int64_t t = blockIdx.x / n_blocks;
    const int nb = blockIdx.x % n_blocks;
    if (t >= *P.num_tiles) return;  // uniform over the workgroup
    const Tile tile = P.tiles[t];
    const int e = tile.expert;
    const int64_t p0 = tile.row_begin;
    const int nrows = tile.row_end - tile.row_begin;
    const int n0 = nb * BN;
    const int KB = P.Kdim / 128;
    const int NB128 = P.Ndim / 128;

    for (int r = tid; r < BM; r += THREADS) {
        int32_t src = -1;
        if (r < nrows) {
            const int64_t p = p0 + r;
            if (MODE == 0) {
                int64_t tok = P.gather[p] / P.K_top;
                tok = tok < 0 ? 0 : (tok >= P.src_rows ? P.src_rows - 1 : tok);
                src = (int32_t)tok;
            } else {
                src = (int32_t)p;
            }
        }
        sRow[r] = src;
    }
    __syncthreads();

    // ---- activation tile staging
    uint4 aReg[A_PER_THREAD];
    float asReg[(BM + THREADS - 1) / THREADS];
    auto loadA = [&](int kb) {
#pragma unroll
        for (int i = 0; i < A_PER_THREAD; ++i) {
            const int c = tid + i * THREADS;
            aReg[i] = make_uint4(0, 0, 0, 0);
            if (c < A_CHUNKS) {
                const int src = sRow[c >> 3];
                if (src >= 0)
                    aReg[i] = *reinterpret_cast<const uint4*>(P.a + (int64_t)src * P.Kdim + kb * 128 + (c & 7) * 16);
            }
        }
#pragma unroll
        for (int i = 0; i < (BM + THREADS - 1) / THREADS; ++i) {
            const int r = tid + i * THREADS;
            asReg[i] = 0.0f;
            if (r < BM) {
                const int src = sRow[r];
                if (src >= 0) asReg[i] = P.as[(int64_t)src * KB + kb];
            }
        }
    };
    auto storeA = [&](int buf) {
#pragma unroll
        for (int i = 0; i < A_PER_THREAD; ++i) {
            const int c = tid + i * THREADS;
            if (c < A_CHUNKS) *reinterpret_cast<uint4*>(&sA[buf][(c >> 3) * kAPitch + (c & 7) * 16]) = aReg[i];
        }
#pragma unroll
        for (int i = 0; i < (BM + THREADS - 1) / THREADS; ++i) {
            const int r = tid + i * THREADS;
            if (r < BM) sAs[buf][r] = asReg[i];
        }
    };

    // ---- weight fragments, straight to registers
    const int wcol0 = n0 + wn * NT * 16;        // first column of this wave (per tensor)
    const int cblk = wcol0 / 128;                // its 128-row weight scale block
    const bool wave_live = wcol0 < P.Ndim;
    const uint8_t* W[2] = {P.w0, P.w1};
    const float* S[2] = {P.s0, P.s1};
    auto loadB = [&](int kb, v8i (&dst)[NTEN][NT]) {
#pragma unroll
        for (int ten = 0; ten < NTEN; ++ten)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const int col = wcol0 + nt * 16 + (lane & 15);
                if (col < P.Ndim) {
                    const uint8_t* ptr = W[ten] + ((int64_t)e * P.Ndim + col) * P.Kdim + kb * 128 + (lane >> 4) * 32;
                    dst[ten][nt] = load_frag_global(ptr);
                } else {
                    dst[ten][nt] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
                }
            }
    };

    v4f acc[NTEN][MT][NT];
#pragma unroll
    for (int ten = 0; ten < NTEN; ++ten)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) acc[ten][mt][nt] = v4f{0.f, 0.f, 0.f, 0.f};

    v8i bCur[NTEN][NT], bNext[NTEN][NT];
    loadA(0);
    loadB(0, bCur);
    storeA(0);
    __syncthreads();

    for (int kb = 0; kb < KB; ++kb) {
        const int buf = kb & 1;
        const bool more = kb + 1 < KB;
        if (more) {
            loadA(kb + 1);
            loadB(kb + 1, bNext);
        }
        float sw[NTEN];
#pragma unroll
        for (int ten = 0; ten < NTEN; ++ten)
            sw[ten] = wave_live ? S[ten][((int64_t)e * NB128 + cblk) * KB + kb] : 0.0f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int rbase = wm * MT * 16 + mt * 16;
            const v8i a = load_frag_lds(&sA[buf][(rbase + (lane & 15)) * kAPitch + (lane >> 4) * 32]);
            float sa[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) sa[i] = sAs[buf][rbase + 4 * (lane >> 4) + i];
#pragma unroll
            for (int ten = 0; ten < NTEN; ++ten) {
                float f[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) f[i] = sa[i] * sw[ten];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    const v4f r = mfma_16x16x128_fp8(a, bCur[ten][nt]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[ten][mt][nt][i] += f[i] * r[i];
                }
            }
        }
        if (more) storeA(buf ^ 1);
        __syncthreads();
        if (more) {
#pragma unroll
            for (int ten = 0; ten < NTEN; ++ten)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) bCur[ten][nt] = bNext[ten][nt];
        }
    }

    if constexpr (MODE == 0) {
        // h = silu(g) * u; per-row amax over the 128 columns of this workgroup
        float h[MT][NT][4];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float m = 0.0f;
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    const float v = silu_fast(acc[0][mt][nt][i]) * acc[1][mt][nt][i];
                    h[mt][nt][i] = v;
                    m = __builtin_fmaxf(m, __builtin_fabsf(v));
                }
#pragma unroll
                for (int msk = 8; msk >= 1; msk >>= 1) m = __builtin_fmaxf(m, __shfl_xor(m, msk, 16));
                if ((lane & 15) == 0) sRed[wn][wm * MT * 16 + mt * 16 + 4 * (lane >> 4) + i] = m;
            }
        __syncthreads();
        const int dff = P.Ndim;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = wm * MT * 16 + mt * 16 + 4 * (lane >> 4) + i;
                float amax = 0.0f;
#pragma unroll
                for (int w = 0; w < WN; ++w) amax = __builtin_fmaxf(amax, sRed[w][row]);
                const float sc = group_scale(amax);
                float q[NT];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) q[nt] = h[mt][nt][i];
                scale_group(q, sc);
                if (row < nrows) {
                    const int64_t p = p0 + row;
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) {
                        const int col = wcol0 + nt * 16 + (lane & 15);
                        P.hq[p * dff + col] = (uint8_t)f32x2_to_e4m3(q[nt], 0.0f);
                    }
                    if (wn == 0 && (lane & 15) == 0) P.hs[p * (dff / 128) + n0 / 128] = sc;
                }
            }
    } else {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = wm * MT * 16 + mt * 16 + 4 * (lane >> 4) + i;
                if (row < nrows) {
                    const int64_t p = p0 + row;
                    int64_t dst = p;
                    float wgt = 1.0f;
                    if (P.scatter) {   // top-1 combine: bf16(0 + w * bf16(y)), the combine's arithmetic
                        dst = P.scatter[p];
                        if (dst < 0 || dst >= P.out_rows) continue;
                        wgt = P.scatter_w[dst];
                    }
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) {
                        const int col = wcol0 + nt * 16 + (lane & 15);
                        if (col < P.Ndim) {
                            uint32_t v = f32_to_bf16(acc[0][mt][nt][i]);
                            if (P.scatter) {
                                float c = 0.0f;
                                c += wgt * bf16_to_f32(v);
                                v = f32_to_bf16(c);
                            }
                            P.y[dst * P.Ndim + col] = (uint16_t)v;
                        }
                    }
                }
            }
    }
}

// ---------------------------------------------------------------- tile shapes
// BM (rows per tile) of each shape; the gate|up and down kernels of a shape share it
// so that one tile list serves both.
int tile_rows(TileShape shape) {
    switch (shape) {
        case TileShape::Rows16: return 16;
        case TileShape::Rows128: return 128;
        case TileShape::Rows192: return 192;
        case TileShape::Rows224: return 224;
        default: return 256;
    }
}

template <int MODE, int WM, int WN, int MT, int NT>
static hipError_t launch(const GemmParams& P, int64_t max_tiles, hipStream_t stream) {
    constexpr int BN = WN * NT * 16;
    const int64_t n_blocks = (P.Ndim + BN - 1) / BN;
    const int64_t grid = max_tiles * n_blocks;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_grouped_gemm<MODE, WM, WN, MT, NT>), dim3((unsigned)grid), dim3(WM * WN * 64), 0, stream,
                       P);
    return hipGetLastError();
}

hipError_t launch_gate_up(const GateUpArgs& a, TileShape shape, hipStream_t stream) {
    GemmParams P{};
    P.a = a.xq; P.as = a.xs; P.gather = a.sorted_slot; P.K_top = a.K; P.src_rows = a.N;
    P.Kdim = a.d; P.Ndim = a.d_ff;
    P.w0 = a.wg; P.s0 = a.sg; P.w1 = a.wu; P.s1 = a.su;
    P.tiles = a.tiles; P.num_tiles = a.num_tiles;
    P.hq = a.hq; P.hs = a.hs;
    switch (shape) {
        case TileShape::Rows16: return launch<0, 1, 4, 1, 2>(P, a.max_tiles, stream);
        default: return launch_gate_up_lds(a, tile_rows(shape), stream);
    }
}

hipError_t launch_down(const DownArgs& a, TileShape shape, hipStream_t stream) {
    GemmParams P{};
    P.a = a.hq; P.as = a.hs; P.gather = nullptr; P.K_top = 1; P.src_rows = a.rows;
    P.Kdim = a.d_ff; P.Ndim = a.d;
    P.w0 = a.wd; P.s0 = a.sd; P.w1 = nullptr; P.s1 = nullptr;
    P.tiles = a.tiles; P.num_tiles = a.num_tiles;
    P.y = a.y; P.scatter = a.scatter; P.scatter_w = a.scatter_w; P.out_rows = a.out_rows;
    switch (shape) {
        // 128 output columns per workgroup (two 16-column subtiles per wave): 96 registers,
        // so 5 waves per SIMD instead of 3 with four subtiles, and 3% faster at decode
        case TileShape::Rows16: return launch<1, 1, 4, 1, 2>(P, a.max_tiles, stream);
        default: return launch_down_lds(a, tile_rows(shape), stream);
    }
}

}  // namespace moe
