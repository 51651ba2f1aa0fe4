// Dispatch: per-expert histogram, prefix sum and stable permutation of the flat
// (token, choice) slots by expert ("Mixture of experts" page, Code: moe_infer --
// the scatter-of-ones column sum, the argsort of the flat ids and the running
// start/end index of each expert's slice).
//
// Integer-only and deterministic. Batches of at most kSmallDispatch slots take one
// launch (k_dispatch_small: one workgroup counts, scans and places every slot, walking the
// slots in order); larger ones take four:
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

// One workgroup of 1024 threads (16 waves) does the whole dispatch of a small batch.
//   1. counts in LDS (integer LDS atomics, one per expert and wave: the totals do not depend
//      on their order);
//   2. counts[e], and offsets[E+1] by a block scan; base[e] = offsets[e] in LDS;
//   3. the slots in rounds of 1024, in slot order. Each lane finds the lanes of its wave with
//      the same expert by one ballot per bit of the expert id; its rank among them gives its
//      place after the earlier lanes. The 16 waves of a round then take their places in wave
//      order, each advancing base[e] by its count of e, so positions follow slot order within
//      each expert (the stable sort).
// Out-of-range ids are not counted and get slot_pos = -1, as in the four-launch path.
__global__ __launch_bounds__(1024) void k_dispatch_small(const int32_t* __restrict__ ids, int NK, int E,
                                                         int nbits, int32_t* __restrict__ counts,
                                                         int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ sorted_slot,
                                                         int32_t* __restrict__ slot_pos) {
    extern __shared__ int32_t lds[];
    int32_t* const cnt = lds;       // [E]
    int32_t* const base = lds + E;  // [E]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int e = tid; e < E; e += 1024) cnt[e] = 0;
    __syncthreads();
    // lanes of this wave whose slot holds the same in-range expert as this lane's (valid lanes)
    auto same_expert = [&](int32_t e, bool valid) -> uint64_t {
        uint64_t match = __ballot(valid);
        for (int b = 0; b < nbits; ++b) {
            const bool bit = valid && ((e >> b) & 1);
            const uint64_t m = __ballot(bit);
            match &= bit ? m : ~m;
        }
        return match;
    };
    // one LDS atomic per expert and wave (the highest lane of each group adds the group's size),
    // so that many slots of one expert do not serialise on one address
    for (int r0 = 0; r0 < NK; r0 += 1024) {
        const int s = r0 + tid;
        const int32_t e = s < NK ? ids[s] : -1;
        const bool valid = e >= 0 && e < E;
        const uint64_t match = same_expert(e, valid);
        if (valid && (match >> lane) == 1ull) atomicAdd(&cnt[e], __popcll(match));
    }
    __syncthreads();
    // exclusive scan: thread tid owns experts [tid per, (tid+1) per)
    const int per = (E + 1023) / 1024;
    const int e0 = tid * per;
    int32_t local = 0;
    for (int e = e0; e < e0 + per && e < E; ++e) local += cnt[e];
    int32_t total;
    int32_t run = block_exclusive_scan<int32_t>(local, &total);
    for (int e = e0; e < e0 + per && e < E; ++e) {
        counts[e] = cnt[e];
        offsets[e] = run;
        base[e] = run;
        run += cnt[e];
    }
    if (tid == 0) offsets[E] = total;
    __syncthreads();
    const uint64_t below = (1ull << lane) - 1ull;
    for (int r0 = 0; r0 < NK; r0 += 1024) {
        const int s = r0 + tid;
        const int32_t e = s < NK ? ids[s] : -1;
        const bool valid = e >= 0 && e < E;
        const uint64_t match = same_expert(e, valid);
        const int rank = __popcll(match & below);
        const int n_same = __popcll(match);
        const bool last = valid && (match >> lane) == 1ull;   // highest lane of its group
        for (int w = 0; w < 16; ++w) {
            if (wave == w && valid) {
                const int32_t b0 = base[e];
                const int32_t p = b0 + rank;
                if (last) base[e] = b0 + n_same;
                sorted_slot[p] = s;
                slot_pos[s] = p;
            }
            __syncthreads();
        }
        if (s < NK && !valid) slot_pos[s] = -1;
    }
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
    if (!checked && NK <= kSmallDispatch && E <= kSmallDispatchExperts) {
        int nbits = 0;
        while ((1 << nbits) < E) ++nbits;   // ids 0..E-1 fit nbits bits
        hipLaunchKernelGGL(k_dispatch_small, dim3(1), dim3(1024), 2 * (size_t)E * sizeof(int32_t), stream, ids,
                           (int)NK, E, nbits, counts, offsets, sorted_slot, slot_pos);
        return hipGetLastError();
    }
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
__global__ __launch_bounds__(1024) void k_tiles(const int32_t* __restrict__ offsets, int E, int64_t rows,
                                                int BM, int64_t cap, Tile* __restrict__ tiles,
                                                int32_t* __restrict__ num_tiles) {
    build_tiles_block(offsets, E, rows, BM, cap, tiles, num_tiles);
}

hipError_t launch_build_tiles(const int32_t* offsets, int E, int64_t rows, int BM, int64_t cap, Tile* tiles,
                              int32_t* num_tiles, hipStream_t stream) {
    hipLaunchKernelGGL(k_tiles, dim3(1), dim3(1024), 0, stream, offsets, E, rows, BM, cap, tiles, num_tiles);
    return hipGetLastError();
}

}  // namespace moe
