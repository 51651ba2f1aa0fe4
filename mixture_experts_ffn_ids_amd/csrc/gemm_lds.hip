// Grouped GEMMs (e4m3 operands) for tiles of many rows (prefill): both operands staged in
// LDS by direct global->LDS copies, with a deeper ring for the weights than for the
// activations.
//
// Same mathematics as gemm.hip ("SwiGLU output" page, evidence "mlp"; "Element-wise
// product" page; FP8 block format from "Input features" page, evidence "linear"):
//   gate|up: G, U = Xq[rows] . W_gate[e]^T, . W_up[e]^T -> h = silu(G) * U, e4m3 per 128
//   down:    Y = Hq[rows] . W_down[e]^T -> bf16
// Per 128-wide quantisation block: gate|up sums it exactly, its fragments widened to bf16
// in registers and multiplied by four 16x16x32 bf16 matrix ops (mfma_block_exact4); down
// uses one 16x16x128 FP8 matrix op. Each 16x16 block product is multiplied by (row
// activation scale x weight block scale) and added to the fp32 accumulator.
//
// Workgroup: 8 waves (2 along the rows x 4 along the weight rows), 512 threads. It owns
// one tile (<= BM = 32 MT sorted rows of one expert, MT = 4, 6, 7 or 8) and 256 weight rows:
// for gate|up the 128 gate and 128 up rows of one 128-wide d_ff block (so the
// requantisation group is complete), for down 256 output columns. Each wave computes
// 16 MT rows x 4 weight-row subtiles of 16 (64 columns): MT x 4 MFMA tiles.
//
// The weights are the MFMA's first operand and the token rows its second, so a lane's
// four results belong to one token row (lane & 15) and four consecutive weight rows. The
// activation scale is then one number per lane and row subtile, and the weight block scale
// one number per wave: the per-block factor costs a broadcast read and a multiply instead
// of a table lookup per result.
//
// Data movement per 128-wide K block, all by global_load_lds (lane L of a wave writes its
// 16 bytes at LDS base + 16 L; no registers involved). Waves 0-3 copy activations, waves
// 4-7 weights: a wave's copies complete in issue order, so a wave that copied both would
// wait for older weight copies (from HBM) before its newer activation copies (from L2)
// counted as landed.
//   * weights (256 x 128 B) into a ring of 3 stages (2 for 256-row tiles, where LDS runs
//     out), so that two weight blocks are in flight from HBM while one is multiplied. The
//     kernel waits on these copies' latency: a ring of 2 instead of 3 costs 30%;
//   * activations (BM x 128 B, gathered token rows for gate|up) and their row scales into
//     a ring of 2 stages (they come mostly from L2: the n-blocks of a tile run together on
//     one XCD; a third stage measured 3-5% slower at 128 rows).
// Rows are 128 B with 16-B chunks XOR-swizzled so that fragment reads are free of bank
// conflicts. Row scales are stored so that the MT scales one lane needs are adjacent.
// Rows past the end of the tile copy a valid row (the tile's first row, or the last weight
// row) and are never stored; a wave skips the matrix work of its row subtiles that hold no
// row of the tile. The copies are written as inline assembly so
// that the compiler does not wait for them at every LDS read; completion is awaited
// explicitly (s_waitcnt vmcnt) before the barrier that publishes a block.
//
// Scheduling: workgroups are dispatched round-robin over the 8 XCDs. The workgroup id is
// remapped so that each XCD gets a contiguous range of items ordered (expert, group of up to
// 8 row tiles, n-block, row tile): the row tiles that share a weight block, and the n-blocks
// that share a tile's rows, run on the same XCD at about the same time and share its L2.
//
// Epilogue: down results are staged through the (then idle) stage buffers and written with
// coalesced 16-byte stores; gate|up codes go from registers straight to global memory.
#include <atomic>
#include <type_traits>

#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kXcds = 8;
constexpr int kMaxDevices = 64;     // devices per process the launcher keeps state for
constexpr int kOutPitch = 256 + 8;  // bf16 elements per row of the staged down-GEMM output
// Row tiles of one expert that sweep its n-blocks together. An XCD runs about 32 consecutive
// items at once (one workgroup per CU); 8 row tiles x 4 n-blocks is the window that fetches the
// fewest activation and weight bytes per K block (8 x 16 KB + 4 x 32 KB at 128 rows, against
// 30 x 16 KB + 32 KB when 30 row tiles of one n-block run together). Measured on the dense MLP
// (43 row tiles of 192 rows): 3.7% faster step than sweeping all row tiles per n-block, 3% with
// groups of 4; level on workloads whose experts have at most 8 row tiles, where the order is
// unchanged.
constexpr int kRowGroup = 8;

typedef __attribute__((address_space(3))) void* lds_ptr_t;

template <int MODE, int MT>
struct Cfg {
    static constexpr int NW = 8;                  // waves: 2 along the rows x 4 along the weights
    static constexpr int THREADS = NW * 64;
    static constexpr int BM = 32 * MT;            // rows per tile
    static constexpr int BR = 256;                // weight rows per workgroup
    static constexpr int A_BYTES = BM * 128;      // one activation stage
    static constexpr int B_BYTES = BR * 128;      // one weight stage
    static constexpr int NA = 2;                  // activation stages
    static constexpr int NBS = BM <= 224 ? 3 : 2; // weight stages
    // waves 0..3 copy the activations and their row scales, waves 4..7 the weights, so that
    // each wave's in-order copy counter tracks one ring only
    static constexpr int ROLE_W = NW / 2;
    static constexpr int A_Q = BM * 8 / (ROLE_W * 64);  // 1-KB copies of A per A-wave per block
    static constexpr int B_Q = BR * 8 / (ROLE_W * 64);  // same for B per B-wave
    static constexpr int S_L = BM / ROLE_W;       // row scales copied by each A-wave (one copy)
    static constexpr int S_STAGE = ROLE_W * 64;   // floats per row-scale stage (64 per A-wave)
    static constexpr int STAGES = NA * A_BYTES + NBS * B_BYTES;
    static constexpr int OUT_BYTES = MODE == 1 ? BM * kOutPitch * 2 : 4 * BM * 4;
    static constexpr int MAIN = STAGES > OUT_BYTES ? STAGES : OUT_BYTES;
    static constexpr int MAX_KB = 65536 / 128;    // K blocks at the largest supported K
    // LDS: A stages | B stages (or the output tile) | row scales [NA][S_STAGE] | source rows
    //      [BM] | weight block scales [2][MAX_KB]
    static constexpr int LDS = MAIN + NA * S_STAGE * 4 + BM * 4 + 2 * MAX_KB * 4;
    static_assert(A_Q * ROLE_W * 64 == BM * 8 && B_Q * ROLE_W * 64 == BR * 8, "copy split");
    static_assert(S_L <= 64 && BM % ROLE_W == 0, "scale copies");
    static_assert(LDS <= 160 * 1024, "LDS budget");
    static_assert(2 * BM <= 2 * MAX_KB && BM <= THREADS, "the top-1 epilogue's row table");
    static_assert(NA >= 2 && NA <= 4 && NBS >= 2 && NBS <= 4, "ring depths");
    static_assert((NA - 2) * (A_Q + 1) <= 63 && (NBS - 2) * B_Q <= 63, "pending copies fit the wait counter");
};

struct LdsGemmParams {
    const uint8_t* a;          // activation codes, row stride Kdim
    const float* as;           // activation scales, row stride Kdim/128
    const int32_t* gather;     // gate|up: sorted_slot; down: NULL
    int K_top;
    int64_t src_rows;
    int Kdim, Ndim;            // Ndim: d_ff (gate|up) or d (down)
    const uint8_t* w0; const float* s0;
    const uint8_t* w1; const float* s1;
    const Tile* tiles; const int32_t* num_tiles;
    int row_group;             // row tiles of one expert that sweep the n-blocks together
    uint8_t* hq; float* hs;
    uint16_t* y;
    const int32_t* scatter; const float* scatter_w; int64_t out_rows;   // top-1 combine (down)
};

// Byte offset of 16-B chunk c of row r in a swizzled [rows][128 B] LDS tile. A fragment read
// has 16 lanes fetch one logical chunk of 16 consecutive rows; the chunk is placed at
// c ^ (r & 7) ^ ((r >> 3) & 1), which gives those 16 rows distinct 16-B slots modulo 256 B
// and each aligned group of 8 rows distinct slots modulo 128 B: no bank conflicts whether
// the LDS serves 16 lanes over 64 banks or 8 lanes over 32 banks per cycle.
__device__ __forceinline__ int swz_pos(int r, int c) { return c ^ (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int swz(int r, int c) { return r * 128 + (swz_pos(r, c) << 4); }

__device__ __forceinline__ v8i lds_frag(const uint8_t* tile, int r, int kg) {
    // 32 K-bytes [32*kg, 32*kg+32) of row r: logical chunks 2kg and 2kg+1
    const uint4 lo = *reinterpret_cast<const uint4*>(tile + swz(r, 2 * kg));
    const uint4 hi = *reinterpret_cast<const uint4*>(tile + swz(r, 2 * kg + 1));
    v8i v;
    v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
    v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
    return v;
}

// Global -> LDS copies (global_load_lds): lane L reads 16 (or 4) bytes at g + off (g the
// same for the whole wave, off the lane's 32-bit byte offset) and writes them at LDS byte
// address l + 16 L (or 4 L); l must be the same for the whole wave.
__device__ __forceinline__ uint32_t lds_addr(const void* l) {
    return (uint32_t)(size_t)(lds_ptr_t)(l);
}
// a wave-uniform pointer, made visibly uniform (scalar registers) for the copy's base operand
__device__ __forceinline__ const void* uniform_ptr(const void* g) {
    const uint64_t v = (uint64_t)g;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (const void*)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ void copy16(const void* g, uint32_t off, uint32_t l) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(
                     __builtin_amdgcn_readfirstlane(l)), "v"(off), "s"(uniform_ptr(g))
                 : "memory", "m0");
}
// the same with the nontemporal hint, for weight blocks that no other workgroup reads
__device__ __forceinline__ void copy16_nt(const void* g, uint32_t off, uint32_t l) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt" ::"s"(
                     __builtin_amdgcn_readfirstlane(l)), "v"(off), "s"(uniform_ptr(g))
                 : "memory", "m0");
}
__device__ __forceinline__ void copy4(const void* g, uint32_t off, uint32_t l) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2" ::"s"(
                     __builtin_amdgcn_readfirstlane(l)), "v"(off), "s"(uniform_ptr(g))
                 : "memory", "m0");
}
// wait until at most N of this wave's copies are still in flight (they complete in order)
template <int N>
__device__ __forceinline__ void wait_copies() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Row of the tile whose activation scale sits in slot `slot` of a row-scale stage: the MT
// scales of row subtiles 0..MT-1 that lane t of row-wave wm needs are adjacent, at
// wm * 16 MT + t * MT.
template <int MT>
__device__ __forceinline__ int scale_slot_row(int slot) {
    const int wm = slot / (MT * 16), rem = slot % (MT * 16);
    return wm * MT * 16 + (rem % MT) * 16 + rem / MT;
}

template <int MODE, int MT>
__global__ __launch_bounds__(512) void k_gemm_lds(const LdsGemmParams P) {
    using C = Cfg<MODE, MT>;
    constexpr int BM = C::BM, NA = C::NA, NBS = C::NBS;

    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    uint8_t* const sA = smem;                                   // [NA][BM][128]
    uint8_t* const sB = smem + NA * C::A_BYTES;                 // [NBS][256][128]
    float* const sSA = reinterpret_cast<float*>(smem + C::MAIN); // [NA][S_STAGE] row scales
    int32_t* const sRow = reinterpret_cast<int32_t*>(sSA + NA * C::S_STAGE);  // [BM]
    float* const sSw = reinterpret_cast<float*>(sRow + BM);     // [2][MAX_KB]

    const int tid = threadIdx.x, lane = tid & 63;
    // the wave index is uniform within a wave: keep what derives from it in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 2, wn = wave & 3;
    const int n_blocks = MODE == 0 ? P.Ndim / 128 : (P.Ndim + 255) / 256;

    // ---- XCD-aware work item (expert, row-tile group, n-block, row tile)
    const int32_t ntile = *P.num_tiles;
    const int64_t work = (int64_t)ntile * n_blocks;
    const int64_t per_xcd = (work + kXcds - 1) / kXcds;
    const int64_t item = (int64_t)(blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
    if (blockIdx.x / kXcds >= per_xcd || item >= work) return;
    const Tile head = P.tiles[item / n_blocks];   // a tile of the item's expert
    // within the expert: groups of up to P.row_group row tiles, each group's (n-block, row
    // tile) items in that order, row tile fastest
    const int64_t local = item - (int64_t)n_blocks * head.first;
    const int64_t gspan = (int64_t)P.row_group * n_blocks;
    const int g = (int)(local / gspan);
    const int r = (int)(local - g * gspan);
    const int grem = head.count - g * P.row_group;
    const int gsize = grem < P.row_group ? grem : P.row_group;
    const int nb = r / gsize;
    const int t = head.first + g * P.row_group + r % gsize;
    if (t >= ntile) return;
    const Tile tile = P.tiles[t];
    const int e = tile.expert;
    const int64_t p0 = tile.row_begin;
    const int nrows = tile.row_end - tile.row_begin;
    const int KB = P.Kdim / 128;
    const int NB128 = P.Ndim / 128;
    const int n0 = MODE == 0 ? nb * 128 : nb * 256;

    // ---- per-lane copy plan. Wave copy q fills rows 8q .. 8q+7 of a stage; lane L lands in
    // row 8q + (L >> 3), slot L & 7, which holds logical chunk (L & 7) ^ (L >> 3) ^ (q & 1).
    // A-wave w (0..3) makes copies q = w + 4i of the activations, B-wave w (4..7) copies
    // q = w - 4 + 4i of the weights: all q of a wave have the parity of the wave.
    const bool b_wave = wave >= C::ROLE_W;
    const int rw = b_wave ? wave - C::ROLE_W : wave;
    const int lrow = lane >> 3;
    const int lchunk = (lane & 7) ^ lrow ^ (wave & 1);
    // weight tensors of expert e; gate|up copies 0..3 are gate rows, 4..7 up rows
    const uint8_t* const wBase0 = P.w0 + (int64_t)e * P.Ndim * P.Kdim;
    const uint8_t* const wBase1 = (MODE == 0 ? P.w1 : P.w0) + (int64_t)e * P.Ndim * P.Kdim;
    // row scales: lane L < S_L of A-wave rw copies the scale of slot rw * S_L + L into position
    // rw * 64 + L of a stage; the other lanes copy a valid value into the padding (so the copy
    // needs no branch). Set once the source rows are in LDS.
    uint32_t sOff = 0;
    const uint32_t ldsA = lds_addr(sA) + rw * 1024, ldsB = lds_addr(sB) + rw * 1024;
    const uint32_t ldsS = lds_addr(sSA) + rw * 256;

    // weight-row base (within the B tile) of this wave's 4 subtiles
    int bbase[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        bbase[j] = MODE == 0 ? (j >> 1) * 128 + wn * 32 + (j & 1) * 16 : wn * 64 + j * 16;

    v4f acc[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[mt][j] = v4f{0.f, 0.f, 0.f, 0.f};

    const int rlane = lane & 15, kg = lane >> 4;
    // row subtiles of this wave that hold rows of the tile (uniform per wave): the matrix
    // work of the others is skipped, their copies still run (they keep the waits exact)
    int live_mt = (nrows - wm * MT * 16 + 15) / 16;
    live_mt = __builtin_amdgcn_readfirstlane(live_mt < 0 ? 0 : (live_mt > MT ? MT : live_mt));
    // weight block scale table of the wave's columns: gate|up subtiles 0,1 gate (table 0),
    // 2,3 up (table 1); down: the wave's 64 columns lie in 128-column block wn >> 1
    const int wtab0 = MODE == 0 ? 0 : (wn >> 1);
    const float* const sSw0 = sSw + wtab0 * C::MAX_KB;
    const float* const sSw1 = sSw + (MODE == 0 ? 1 : wtab0) * C::MAX_KB;
    // this lane's MT row scales: slots wm 16 MT + rlane MT + (0..MT-1), at padded positions
    const int sa_slot = wm * MT * 16 + rlane * MT;
    const int sa_pos = (sa_slot / C::S_L) * 64 + sa_slot % C::S_L;

    // The K loop, instantiated per copy role (BW: this wave copies weights) so that the
    // copies it issues between the matrix ops are straight-line code.
    // FULL: every row subtile of the wave is live, and the matrix work has no branches.
    // STREAM (gate|up weight waves): every expert has one tile, so each weight block is read
    // by this workgroup only and is copied with the nontemporal hint (measured 6% faster
    // gate|up at 2048 tokens, 2% at prefill; where several row tiles share an expert's
    // weights through L2 the hint cost 2-5%, so it is off there).
    auto run = [&](auto role, auto full, auto stream) {
        constexpr bool BW = decltype(role)::value;
        constexpr bool FULL = decltype(full)::value;
        constexpr bool STREAM = decltype(stream)::value;
        constexpr int NQ = BW ? C::B_Q : C::A_Q + 1;  // copies per block (A: rows + scales)
        constexpr int NR = BW ? NBS : NA;             // ring depth
        // byte offset of copy i in block 0: in the activations (A) or the weight tensor (B);
        // the host keeps both below 2^32. Computed once per item and held in registers.
        auto off = [&](int i) -> uint32_t {
            const int r = 8 * (rw + i * C::ROLE_W) + lrow;
            if constexpr (!BW) {
                return (uint32_t)sRow[r] * (uint32_t)P.Kdim + lchunk * 16;
            } else {
                int wrow = MODE == 0 ? n0 + (r & 127) : n0 + r;
                wrow = wrow < P.Ndim ? wrow : P.Ndim - 1;
                return (uint32_t)wrow * (uint32_t)P.Kdim + lchunk * 16;
            }
        };
        uint32_t cIdx[NQ];
        auto plan = [&]() {
#pragma unroll
            for (int i = 0; i < NQ; ++i) cIdx[i] = (!BW && i == C::A_Q) ? 0u : off(i);
            if constexpr (!BW)
                sOff = lane < C::S_L ? (uint32_t)sRow[scale_slot_row<MT>(rw * C::S_L + lane)] * (uint32_t)KB * 4u
                                     : 0u;
        };
        // issue copies [lo, hi) of block kb
        auto issue = [&](int kb, int lo, int hi) {
            const int ko = kb * 128;
#pragma unroll
            for (int i = 0; i < NQ; ++i) {
                if (i < lo || i >= hi) continue;
                if constexpr (!BW) {
                    if (i < C::A_Q)
                        copy16(P.a + ko, cIdx[i], ldsA + (kb % NA) * C::A_BYTES + i * C::ROLE_W * 1024);
                    else
                        copy4(P.as + kb, sOff, ldsS + (kb % NA) * C::S_STAGE * 4);
                } else {
                    const void* src = (MODE == 0 && i >= C::B_Q / 2 ? wBase1 : wBase0) + ko;
                    const uint32_t dst = ldsB + (kb % NBS) * C::B_BYTES + i * C::ROLE_W * 1024;
                    if constexpr (STREAM)
                        copy16_nt(src, cIdx[i], dst);
                    else
                        copy16(src, cIdx[i], dst);
                }
            }
        };

        // multiply K block kb (landed and published) into the accumulators; with ISSUE, also
        // issue the copies of block `next`, spread over the row subtiles: a copy can stall its
        // wave until the memory pipeline takes it, and spread out those stalls overlap the
        // matrix work instead of preceding it
        // Exception: with a 2-stage activation ring an A-wave issues its whole block first,
        // for the most lead time (its copies must land by the end of this iteration).
        constexpr int SLOTS = (BW || NA > 2) ? MT : 1;
        auto compute = [&](int kb, auto issue_tag, int next) {
            constexpr bool ISSUE = decltype(issue_tag)::value;
            const uint8_t* A = sA + (kb % NA) * C::A_BYTES;
            const uint8_t* B = sB + (kb % NBS) * C::B_BYTES;
            const float* SA = sSA + (kb % NA) * C::S_STAGE + sa_pos;
            v8i bf[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) bf[j] = lds_frag(B, bbase[j] + rlane, kg);
            // one row subtile at a time (a scheduling barrier after each keeps the compiler
            // from gathering all of them, which would hold every fragment at once); the next
            // subtile's activation fragment is read ahead.
            auto scale_add = [&](int mt, const v4f (&r)[4], float f0, float f1) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float f = (MODE == 0 && j >= 2) ? f1 : f0;
                    acc[mt][j][0] += f * r[j][0];
                    acc[mt][j][1] += f * r[j][1];
                    acc[mt][j][2] += f * r[j][2];
                    acc[mt][j][3] += f * r[j][3];
                }
            };
            v8i af = lds_frag(A, wm * MT * 16 + rlane, kg);
            if constexpr (MODE == 0) {
                // gate|up, exact block sums (mfma_block_exact4): the weight fragments are widened
                // to bf16 once per block, each activation fragment just before its subtile's
                // matrix ops.
                // DEFER (up to 192 rows, where the 16 registers fit): a subtile's products are
                // scaled into the accumulators after the next subtile's matrix ops are issued,
                // so the wave does not wait for its own products.
                constexpr bool DEFER = MT <= 6;
                const float w0 = sSw0[kb], w1 = sSw1[kb];
                Frag16 bw[4];
                v4f rp[DEFER ? 4 : 1];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    v8i af_next;
                    if (mt + 1 < MT) af_next = lds_frag(A, wm * MT * 16 + (mt + 1) * 16 + rlane, kg);
                    if constexpr (ISSUE) {
                        if (mt % (MT / SLOTS) == 0) {
                            const int slot = mt / (MT / SLOTS);
                            issue(next, slot * NQ / SLOTS, (slot + 1) * NQ / SLOTS);
                        }
                    }
                    v4f r[4];
                    if (FULL || mt < live_mt) {
                        if (mt == 0) {
#pragma unroll
                            for (int j = 0; j < 4; ++j) bw[j] = widen(bf[j]);
                        }
                        mfma_block_exact4(bw, widen(af), r);
                        if constexpr (!DEFER) {
                            const float sam = SA[mt];   // this subtile's row scale, read when needed
                            scale_add(mt, r, sam * w0, sam * w1);
                        }
                    }
                    if constexpr (DEFER) {
                        if (mt > 0 && (FULL || mt - 1 < live_mt)) {
                            const float sam = SA[mt - 1];
                            scale_add(mt - 1, rp, sam * w0, sam * w1);
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    if constexpr (DEFER) {
#pragma unroll
                        for (int j = 0; j < 4; ++j) rp[j] = r[j];
                    }
                    if (mt + 1 < MT) af = af_next;
                }
                if constexpr (DEFER) {
                    if (FULL || MT - 1 < live_mt) {
                        const float sam = SA[MT - 1];
                        scale_add(MT - 1, rp, sam * w0, sam * w1);
                    }
                }
                return;
            }
            // down: one FP8 op per 128-wide block (its result is not requantised)
            const float w0 = sSw0[kb];
            float sa[MT];
            if constexpr (MT % 2 == 0) {   // pairs are 8-byte aligned when MT is even
#pragma unroll
                for (int mt = 0; mt < MT; mt += 2) {
                    const float2 v = *reinterpret_cast<const float2*>(SA + mt);
                    sa[mt] = v.x;
                    sa[mt + 1] = v.y;
                }
            } else {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) sa[mt] = SA[mt];
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                v8i af_next;
                if (mt + 1 < MT) af_next = lds_frag(A, wm * MT * 16 + (mt + 1) * 16 + rlane, kg);
                if constexpr (ISSUE) {
                    if (mt % (MT / SLOTS) == 0) {
                        const int slot = mt / (MT / SLOTS);
                        issue(next, slot * NQ / SLOTS, (slot + 1) * NQ / SLOTS);
                    }
                }
                if (FULL || mt < live_mt) {
                    const float f = sa[mt] * w0;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const v4f p = mfma_16x16x128_fp8(bf[j], af);
                        acc[mt][j][0] += f * p[0];
                        acc[mt][j][1] += f * p[1];
                        acc[mt][j][2] += f * p[2];
                        acc[mt][j][3] += f * p[3];
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
                if (mt + 1 < MT) af = af_next;
            }
        };

        // ---- pipeline. Block kb's activations (with their row scales) are copied NA-1
        // iterations ahead by the A-waves, its weights NBS-1 ahead by the B-waves. At the end
        // of iteration kb, block kb+1 must have landed; what a wave may leave in flight then
        // is the copies it issued last, so an in-order count of pending copies is an exact
        // wait. Both roles pass the same number of barriers.
        // Prologue. The weights' first blocks depend only on the tile, so B-waves issue them
        // at once; meanwhile the A-waves (no copies in flight yet, so their loads cost no
        // extra waits) fill the tables of source rows and weight block scales, and after the
        // barrier that publishes them they issue the activations' first blocks.
        // the first NR - 1 blocks of a role's ring (fewer when K is shorter)
        auto prologue = [&]() {
#pragma unroll
            for (int b = 0; b < NR - 1; ++b)
                if (b < KB) issue(b, 0, NQ);
        };
        if constexpr (BW) {
            plan();
            prologue();
        } else {
            // source row of every tile row; rows past the end repeat the tile's first row
            for (int r = tid; r < BM; r += C::ROLE_W * 64) {
                const int64_t p = p0 + (r < nrows ? r : 0);
                int32_t src;
                if (MODE == 0) {
                    int64_t tok = P.gather[p] / P.K_top;
                    tok = tok < 0 ? 0 : (tok >= P.src_rows ? P.src_rows - 1 : tok);
                    src = (int32_t)tok;
                } else {
                    src = (int32_t)p;
                }
                sRow[r] = src;
            }
            // weight block scales of the workgroup's columns for every K block: gate|up ->
            // gate and up scales of d_ff block nb; down -> the two 128-column blocks of n-block
            // nb
            for (int i = tid; i < 2 * KB; i += C::ROLE_W * 64) {
                const int which = i / KB, kb = i % KB;
                float v;
                if (MODE == 0) {
                    v = (which == 0 ? P.s0 : P.s1)[((int64_t)e * NB128 + nb) * KB + kb];
                } else {
                    const int cb = n0 / 128 + which;
                    v = cb < NB128 ? P.s0[((int64_t)e * NB128 + cb) * KB + kb] : 0.0f;
                }
                sSw[which * C::MAX_KB + kb] = v;
            }
        }
        __syncthreads();
        if constexpr (!BW) {
            plan();
            prologue();
        }
        // block 0 landed; the later prologue blocks may still be in flight
        if (KB >= NR - 1)
            wait_copies<(NR - 2) * NQ>();
        else
            wait_copies<0>();
        __syncthreads();

        // steady state: every ring is refilled in every iteration and the wait count is a
        // constant, with no branch between the matrix work and the wait
        constexpr int AHEAD = (NA > NBS ? NA : NBS) - 1;
        static_assert(AHEAD >= 1 && AHEAD <= 3, "ring depths of 2 to 4");
        for (int kb = 0; kb < KB - AHEAD; ++kb) {
            // refill the stage read in iteration kb - 1 (the barrier below separates them)
            compute(kb, std::true_type{}, kb + NR - 1);
            __builtin_amdgcn_sched_barrier(0);
            wait_copies<(NR - 2) * NQ>();
            __syncthreads();
        }
        // the last AHEAD blocks (t = 0 .. AHEAD-1 is block KB - AHEAD + t, skipped when K is
        // shorter): whether a role still has a block to copy is known at compile time
        auto drain = [&](auto t_tag) {
            constexpr int T = decltype(t_tag)::value;
            const int kbt = KB - AHEAD + T;
            if (kbt < 0) return;
            compute(kbt, std::integral_constant<bool, (T + NR - 1 < AHEAD)>{}, kbt + NR - 1);
            __builtin_amdgcn_sched_barrier(0);
            wait_copies<0>();
            __syncthreads();
        };
        drain(std::integral_constant<int, 0>{});
        if constexpr (AHEAD > 1) drain(std::integral_constant<int, 1>{});
        if constexpr (AHEAD > 2) drain(std::integral_constant<int, 2>{});
    };
    // every variant passes the same barriers, so the waves of one workgroup may differ.
    // Only gate|up has the streaming variant: down gained nothing from it, and its extra
    // copy of the K loop cost the down kernel 4% where it was not taken.
    const bool one_tile_per_expert = MODE == 0 && P.num_tiles[1] != 0;   // uniform over the launch
    if (live_mt == MT) {
        if (b_wave) {
            if constexpr (MODE == 0) {
                if (one_tile_per_expert) {
                    run(std::true_type{}, std::true_type{}, std::true_type{});
                } else {
                    run(std::true_type{}, std::true_type{}, std::false_type{});
                }
            } else {
                run(std::true_type{}, std::true_type{}, std::false_type{});
            }
        } else {
            run(std::false_type{}, std::true_type{}, std::false_type{});
        }
    } else {
        if (b_wave) {
            if constexpr (MODE == 0) {
                if (one_tile_per_expert) {
                    run(std::true_type{}, std::false_type{}, std::true_type{});
                } else {
                    run(std::true_type{}, std::false_type{}, std::false_type{});
                }
            } else {
                run(std::true_type{}, std::false_type{}, std::false_type{});
            }
        } else {
            run(std::false_type{}, std::false_type{}, std::false_type{});
        }
    }

    // acc[mt][j][i]: row rb + rlane of the tile (rb = wm MT 16 + 16 mt), weight row
    // bbase[j] + 4 kg + i of the workgroup's 256
    if constexpr (MODE == 0) {
        // ---- h = silu(g) * u, per-row amax over the 128 columns, e4m3 requantisation; each
        // lane stores its 4 consecutive codes per subtile straight from registers (measured
        // faster here than staging the 24-KB code tile through LDS)
        float* sRed = reinterpret_cast<float*>(smem);                 // [4][BM] row maxima
        float h[MT][2][4];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            float m = 0.0f;
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float v = silu_fast(acc[mt][jj][i]) * acc[mt][jj + 2][i];
                    h[mt][jj][i] = v;
                    m = __builtin_fmaxf(m, __builtin_fabsf(v));
                }
            m = __builtin_fmaxf(m, __shfl_xor(m, 16));
            m = __builtin_fmaxf(m, __shfl_xor(m, 32));
            if (kg == 0) sRed[wn * BM + wm * MT * 16 + mt * 16 + rlane] = m;
        }
        __syncthreads();
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int row = wm * MT * 16 + mt * 16 + rlane;
            const float amax = __builtin_fmaxf(__builtin_fmaxf(sRed[row], sRed[BM + row]),
                                               __builtin_fmaxf(sRed[2 * BM + row], sRed[3 * BM + row]));
            const float sc = group_scale(amax);
            float q[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) q[k] = h[mt][k >> 2][k & 3];
            scale_group(q, sc);
            if (row < nrows) {
                const int64_t p = p0 + row;
#pragma unroll
                for (int jj = 0; jj < 2; ++jj) {
                    const uint32_t lo = f32x2_to_e4m3(q[4 * jj], q[4 * jj + 1]);
                    const uint32_t hi = f32x2_to_e4m3(q[4 * jj + 2], q[4 * jj + 3]);
                    *reinterpret_cast<uint32_t*>(P.hq + p * P.Ndim + n0 + wn * 32 + jj * 16 + 4 * kg) = lo | (hi << 16);
                }
                if (wn == 0 && kg == 0) P.hs[p * NB128 + nb] = sc;
            }
        }
    } else {
        // ---- bf16 Y tile [BM][256] through LDS, coalesced 16-B stores of valid rows/columns.
        // With the top-1 combine, each tile row's destination row and weight are read once
        // (their loads overlap the staging) into the weight-scale table, unused from here on.
        int32_t* const sDst = reinterpret_cast<int32_t*>(sSw);
        float* const sWt = sSw + BM;
        int32_t my_dst = -1;
        float my_w = 0.0f;
        if (P.scatter) {
            for (int r = tid; r < BM; r += C::THREADS) {   // BM <= THREADS: one row per thread
                if (r < nrows) {
                    const int64_t d = P.scatter[p0 + r];
                    if (d >= 0 && d < P.out_rows) {
                        my_dst = (int32_t)d;
                        my_w = P.scatter_w[d];
                    }
                }
            }
        }
        uint16_t* out = reinterpret_cast<uint16_t*>(smem);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int row = wm * MT * 16 + mt * 16 + rlane;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                uint2 v;
                v.x = f32_to_bf16(acc[mt][j][0]) | (f32_to_bf16(acc[mt][j][1]) << 16);
                v.y = f32_to_bf16(acc[mt][j][2]) | (f32_to_bf16(acc[mt][j][3]) << 16);
                *reinterpret_cast<uint2*>(out + row * kOutPitch + wn * 64 + j * 16 + 4 * kg) = v;
            }
        }
        if (P.scatter && tid < BM) {
            sDst[tid] = my_dst;
            sWt[tid] = my_w;
        }
        __syncthreads();
        const int ncols = P.Ndim - n0 < 256 ? P.Ndim - n0 : 256;
        if (P.scatter) {
            // top-1 combine: row p of the tile goes to row scatter[p] of y as
            // bf16(0 + w * bf16(y)), the combine's arithmetic for one choice
            for (int c = tid; c < BM * 32; c += C::THREADS) {
                const int row = c >> 5, cc = (c & 31) * 8;
                if (row >= nrows || cc >= ncols) continue;
                const int64_t dst = sDst[row];
                if (dst < 0) continue;
                const float wgt = sWt[row];
                const uint4 v = *reinterpret_cast<const uint4*>(out + row * kOutPitch + cc);
                const uint32_t in[4] = {v.x, v.y, v.z, v.w};
                uint32_t o[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    float lo = 0.0f, hi = 0.0f;
                    lo += wgt * bf16_to_f32(in[k] & 0xffffu);
                    hi += wgt * bf16_to_f32(in[k] >> 16);
                    o[k] = f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
                }
                *reinterpret_cast<uint4*>(P.y + dst * P.Ndim + n0 + cc) = make_uint4(o[0], o[1], o[2], o[3]);
            }
        } else {
            for (int c = tid; c < BM * 32; c += C::THREADS) {
                const int row = c >> 5, cc = (c & 31) * 8;
                if (row < nrows && cc < ncols)
                    *reinterpret_cast<uint4*>(P.y + (p0 + row) * P.Ndim + n0 + cc) =
                        *reinterpret_cast<const uint4*>(out + row * kOutPitch + cc);
            }
        }
    }
}

template <int MODE, int MT>
hipError_t launch_lds(LdsGemmParams P, int64_t max_tiles, hipStream_t stream) {
    using C = Cfg<MODE, MT>;
    P.row_group = kRowGroup;
    const int64_t n_blocks = MODE == 0 ? P.Ndim / 128 : (P.Ndim + 255) / 256;
    int64_t grid = max_tiles * n_blocks;
    grid = (grid + kXcds - 1) / kXcds * kXcds;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    // raise the dynamic LDS limit once per instantiation and device (the attribute belongs to
    // the device's copy of the kernel); concurrent first calls may both set it, which is harmless
    static std::atomic<bool> attr_set[kMaxDevices];
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    if (!attr_set[dev].load(std::memory_order_acquire)) {
        err = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm_lds<MODE, MT>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS);
        if (err != hipSuccess) return err;
        attr_set[dev].store(true, std::memory_order_release);
    }
    hipLaunchKernelGGL((k_gemm_lds<MODE, MT>), dim3((unsigned)grid), dim3(C::THREADS), C::LDS, stream, P);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gate_up_lds(const GateUpArgs& a, int rows, hipStream_t stream) {
    LdsGemmParams P{};
    P.a = a.xq; P.as = a.xs; P.gather = a.sorted_slot; P.K_top = a.K; P.src_rows = a.N;
    P.Kdim = a.d; P.Ndim = a.d_ff;
    P.w0 = a.wg; P.s0 = a.sg; P.w1 = a.wu; P.s1 = a.su;
    P.tiles = a.tiles; P.num_tiles = a.num_tiles;
    P.hq = a.hq; P.hs = a.hs;
    switch (rows) {
        case 128: return launch_lds<0, 4>(P, a.max_tiles, stream);
        case 192: return launch_lds<0, 6>(P, a.max_tiles, stream);
        case 224: return launch_lds<0, 7>(P, a.max_tiles, stream);
        default: return launch_lds<0, 8>(P, a.max_tiles, stream);
    }
}

hipError_t launch_down_lds(const DownArgs& a, int rows, hipStream_t stream) {
    LdsGemmParams P{};
    P.a = a.hq; P.as = a.hs; P.gather = nullptr; P.K_top = 1; P.src_rows = a.rows;
    P.Kdim = a.d_ff; P.Ndim = a.d;
    P.w0 = a.wd; P.s0 = a.sd;
    P.tiles = a.tiles; P.num_tiles = a.num_tiles;
    P.y = a.y; P.scatter = a.scatter; P.scatter_w = a.scatter_w; P.out_rows = a.out_rows;
    switch (rows) {
        case 128: return launch_lds<1, 4>(P, a.max_tiles, stream);
        case 192: return launch_lds<1, 6>(P, a.max_tiles, stream);
        case 224: return launch_lds<1, 7>(P, a.max_tiles, stream);
        default: return launch_lds<1, 8>(P, a.max_tiles, stream);
    }
}

}  // namespace moe
