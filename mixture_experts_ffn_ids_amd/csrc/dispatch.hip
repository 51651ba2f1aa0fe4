// Dispatch: per-expert histogram, prefix sum and stable permutation of the flat
// (token, choice) slots by expert ("Mixture of experts" page, Code: moe_infer --
// the scatter-of-ones column sum, the argsort of the flat ids and the running
// start/end index of each expert's slice).
//
// Integer-only and deterministic. Four launches:
//   1. k_hist:    slots are cut into chunks of 256; each workgroup counts its
//                 chunk per expert in LDS (integer LDS atomics -- the counts do not
//                 depend on their order) and writes chunk_counts[E][chunk].
//   2. k_colscan: one wave per expert turns its row of chunk counts into an exclusive
//                 prefix (the chunk's base inside the expert's slice) and writes
//                 counts[e].
//   3. k_offsets: one workgroup writes the exclusive scan offsets[E+1] of the counts.
//   4. k_permute: each slot's position is offsets[e] + chunk base + its rank among
//                 the earlier slots of the same expert in its chunk, so the order
//                 within an expert is ascending slot index (a stable sort).
// Also builds the GEMM tile lists (k_tiles) from offsets.
#include "moe_internal.h"

namespace moe {

__global__ __launch_bounds__(kDispatchChunk) void k_hist(const int32_t* __restrict__ ids, int64_t NK,
                                                         int K, int E, int nchunks,
                                                         int32_t* __restrict__ chunk_counts,
                                                         int32_t* __restrict__ err, int checked) {
    extern __shared__ int32_t cnt[];  // [E]
    for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
    __syncthreads();
    const int64_t s = (int64_t)blockIdx.x * kDispatchChunk + threadIdx.x;
    if (s < NK) {
        const int32_t e = ids[s];
        const bool in_range = e >= 0 && e < E;
        if (in_range) atomicAdd(&cnt[e], 1);
        if (checked) {
            if (!in_range) atomicOr(err, 1);
            const int64_t row = s / K;
            const int k = (int)(s - row * K);
            for (int j = 0; j < k; ++j)
                if (ids[row * K + j] == e) atomicOr(err, 2);
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) chunk_counts[(int64_t)e * nchunks + blockIdx.x] = cnt[e];
}

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

// Per expert (one wave each, four per workgroup): exclusive prefix of its chunk counts, in
// place, and its total. Lane L sums chunks [L per, (L+1) per), the lane sums are scanned
// across the wave, and each lane rewrites its chunks as running bases.
__global__ __launch_bounds__(256) void k_colscan(int32_t* __restrict__ chunk_counts, int nchunks, int E,
                                                 int32_t* __restrict__ counts) {
    const int lane = threadIdx.x & 63;
    const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (e >= E) return;  // uniform over the wave
    int32_t* row = chunk_counts + (int64_t)e * nchunks;
    const int per = (nchunks + 63) / 64;
    const int c0 = lane * per;
    const int c1 = c0 + per < nchunks ? c0 + per : nchunks;
    int32_t local = 0;
    for (int c = c0; c < c1; ++c) local += row[c];
    int32_t incl = local;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int32_t t = __shfl_up(incl, off, 64);
        if (lane >= off) incl += t;
    }
    int32_t run = incl - local;
    for (int c = c0; c < c1; ++c) {
        const int32_t v = row[c];
        row[c] = run;
        run += v;
    }
    if (lane == 63) counts[e] = incl;
}

// offsets[E+1]: exclusive scan of the per-expert counts (one workgroup; each thread owns a
// contiguous range of experts).
__global__ __launch_bounds__(1024) void k_offsets(const int32_t* __restrict__ counts, int E,
                                                  int32_t* __restrict__ offsets) {
    const int per = (E + blockDim.x - 1) / blockDim.x;
    const int e0 = threadIdx.x * per;
    int32_t local = 0;
    for (int e = e0; e < e0 + per && e < E; ++e) local += counts[e];
    int32_t total;
    int32_t run = block_exclusive_scan<int32_t>(local, &total);
    for (int e = e0; e < e0 + per && e < E; ++e) {
        offsets[e] = run;
        run += counts[e];
    }
    if (threadIdx.x == 0) offsets[E] = total;
}

__global__ __launch_bounds__(kDispatchChunk) void k_permute(const int32_t* __restrict__ ids, int64_t NK, int E,
                                                            int nchunks, const int32_t* __restrict__ chunk_base,
                                                            const int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ sorted_slot,
                                                            int32_t* __restrict__ slot_pos) {
    __shared__ int32_t sid[kDispatchChunk];
    const int64_t s = (int64_t)blockIdx.x * kDispatchChunk + threadIdx.x;
    const int32_t e = s < NK ? ids[s] : -1;
    sid[threadIdx.x] = e;
    __syncthreads();
    if (s >= NK) return;
    if (e < 0 || e >= E) {
        slot_pos[s] = -1;
        return;
    }
    int rank = 0;
    for (int j = 0; j < (int)threadIdx.x; ++j) rank += (sid[j] == e);
    const int32_t p = offsets[e] + chunk_base[(int64_t)e * nchunks + blockIdx.x] + rank;
    sorted_slot[p] = (int32_t)s;
    slot_pos[s] = p;
}

__global__ void k_fill_i32(int32_t* p, int64_t n, int32_t v) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

hipError_t launch_dispatch(const int32_t* ids, int64_t N, int K, int E, int32_t* counts,
                           int32_t* offsets, int32_t* sorted_slot, int32_t* slot_pos,
                           int32_t* chunk_counts, int32_t* err_flag, bool checked,
                           hipStream_t stream) {
    const int64_t NK = N * K;
    const int nchunks = (int)((NK + kDispatchChunk - 1) / kDispatchChunk);
    if (checked) hipLaunchKernelGGL(k_fill_i32, dim3(1), dim3(64), 0, stream, err_flag, (int64_t)1, 0);
    if (nchunks > 0) {
        hipLaunchKernelGGL(k_hist, dim3(nchunks), dim3(kDispatchChunk), E * sizeof(int32_t), stream, ids, NK,
                           K, E, nchunks, chunk_counts, err_flag, checked ? 1 : 0);
        hipLaunchKernelGGL(k_colscan, dim3((E + 3) / 4), dim3(256), 0, stream, chunk_counts, nchunks, E, counts);
    } else {
        hipLaunchKernelGGL(k_fill_i32, dim3((E + 255) / 256), dim3(256), 0, stream, counts, (int64_t)E, 0);
    }
    hipLaunchKernelGGL(k_offsets, dim3(1), dim3(1024), 0, stream, counts, E, offsets);
    if (nchunks > 0)
        hipLaunchKernelGGL(k_permute, dim3(nchunks), dim3(kDispatchChunk), 0, stream, ids, NK, E, nchunks,
                           chunk_counts, offsets, sorted_slot, slot_pos);
    return hipGetLastError();
}

// ---------------------------------------------------------------- tile lists
int64_t max_tiles(int64_t rows, int E, int BM) {
    // sum_e ceil(M_e / BM) <= rows / BM + (number of non-empty experts)
    const int64_t nonempty = rows < E ? rows : E;
    return rows / BM + nonempty + 1;
}

// num_tiles[0]: tiles written; num_tiles[1]: 1 when every expert with rows got one tile
__global__ __launch_bounds__(1024) void k_tiles(const int32_t* __restrict__ offsets, int E, int64_t rows,
                                                int BM, int64_t cap, Tile* __restrict__ tiles,
                                                int32_t* __restrict__ num_tiles) {
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

hipError_t launch_build_tiles(const int32_t* offsets, int E, int64_t rows, int BM, int64_t cap, Tile* tiles,
                              int32_t* num_tiles, hipStream_t stream) {
    hipLaunchKernelGGL(k_tiles, dim3(1), dim3(1024), 0, stream, offsets, E, rows, BM, cap, tiles, num_tiles);
    return hipGetLastError();
}

}  // namespace moe
