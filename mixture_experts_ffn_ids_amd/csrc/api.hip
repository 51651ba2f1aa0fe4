// C ABI of libmoe: host-side validation, workspace layout, tile-list sizing, launches
// and the per-kernel event profiler. The declarations and their contracts are in
// include/moe.h. This file holds no kernels: it also builds for the host alone, which
// the sanitizer check of the host code uses.
#include <math.h>
#include <mutex>
#include <string.h>
#include <vector>

#include "moe.h"
#include "moe_internal.h"

namespace moe {

// ---------------------------------------------------------------- tile lists
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

int64_t max_tiles(int64_t rows, int E, int BM) {
    // sum_e ceil(M_e / BM) <= rows / BM + (number of non-empty experts)
    const int64_t nonempty = rows < E ? rows : E;
    return rows / BM + nonempty + 1;
}

}  // namespace moe

using namespace moe;

namespace {

thread_local int g_last_hip_error = 0;

moe_status hip_fail(hipError_t e) {
    g_last_hip_error = (int)e;
    return MOE_ERR_HIP;
}

}  // namespace

moe_status moe::record_hip_error(hipError_t e) { return hip_fail(e); }

namespace {

#define MOE_HIP(expr)                                 \
    do {                                              \
        hipError_t _e = (expr);                       \
        if (_e != hipSuccess) return hip_fail(_e);    \
    } while (0)

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// ---------------------------------------------------------------- device check
std::mutex g_dev_mu;
std::vector<int> g_dev_ok;  // per device: 0 unknown, 1 gfx950, -1 other

moe_status check_device() {
    int dev = 0;
    MOE_HIP(hipGetDevice(&dev));
    std::lock_guard<std::mutex> lk(g_dev_mu);
    if ((int)g_dev_ok.size() <= dev) g_dev_ok.resize(dev + 1, 0);
    if (g_dev_ok[dev] == 0) {
        hipDeviceProp_t prop;
        MOE_HIP(hipGetDeviceProperties(&prop, dev));
        g_dev_ok[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    }
    return g_dev_ok[dev] == 1 ? MOE_OK : MOE_ERR_DEVICE;
}

// ---------------------------------------------------------------- profiler
struct Pending {
    int kind;
    hipEvent_t a, b;
};
std::mutex g_prof_mu;
uint32_t g_prof_mask = 0;   // bit k: launches of kind k are timed
std::vector<hipEvent_t> g_prof_pool;
std::vector<Pending> g_prof_pending;
double g_prof_ms[MOE_KERNEL_KINDS] = {0};
int64_t g_prof_n[MOE_KERNEL_KINDS] = {0};

hipEvent_t prof_event() {
    if (!g_prof_pool.empty()) {
        hipEvent_t e = g_prof_pool.back();
        g_prof_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

// Records an event before a launch and one after it when profiling is on.
class ProfScope {
public:
    ProfScope(int kind, hipStream_t s) : kind_(kind), s_(s) {
        std::lock_guard<std::mutex> lk(g_prof_mu);
        if (kind < 0 || kind >= MOE_KERNEL_KINDS || !((g_prof_mask >> kind) & 1u)) return;
        a_ = prof_event();
        b_ = prof_event();
        if (!a_ || !b_ || hipEventRecord(a_, s_) != hipSuccess) release();
    }
    ~ProfScope() {
        std::lock_guard<std::mutex> lk(g_prof_mu);
        if (!a_ || !b_) return;
        if (hipEventRecord(b_, s_) != hipSuccess) {  // this launch goes untimed
            release();
            return;
        }
        g_prof_pending.push_back({kind_, a_, b_});
    }

private:
    // return the events to the pool (caller holds g_prof_mu)
    void release() {
        if (a_) g_prof_pool.push_back(a_);
        if (b_) g_prof_pool.push_back(b_);
        a_ = b_ = nullptr;
    }
    int kind_;
    hipStream_t s_;
    hipEvent_t a_ = nullptr, b_ = nullptr;
};

// ---------------------------------------------------------------- workspace layouts
struct DispatchWs {
    size_t chunk_counts, err, total;
};
DispatchWs dispatch_layout(int64_t N, int32_t K, int32_t E) {
    DispatchWs w;
    const int64_t nchunks = (N * K + kDispatchChunk - 1) / kDispatchChunk;
    w.chunk_counts = 0;
    w.err = align_up((size_t)nchunks * (size_t)E * sizeof(int32_t));
    w.total = w.err + kAlign;
    return w;
}

struct SwigluWs {
    size_t xq, xs, hq, hs, tiles, ntiles, total;
    int64_t tile_cap;
};
// with_x: room for the quantised activations (moe_grouped_swiglu); without it the caller
// passes them in (moe_grouped_swiglu_q)
SwigluWs swiglu_layout(int64_t N, int32_t K, int32_t E, int32_t d, int32_t d_ff, bool with_x = true) {
    SwigluWs w;
    const int64_t rows = N * K;
    size_t off = 0;
    w.xq = off; off = with_x ? align_up(off + (size_t)N * d) : off;
    w.xs = off; off = with_x ? align_up(off + (size_t)N * (d / kGroup) * sizeof(float)) : off;
    w.hq = off; off = align_up(off + (size_t)rows * d_ff);
    w.hs = off; off = align_up(off + (size_t)rows * (d_ff / kGroup) * sizeof(float));
    // sized for the smallest tile height, so every tile shape fits
    w.tile_cap = max_tiles(rows, E, tile_rows(TileShape::Rows16));
    w.tiles = off; off = align_up(off + (size_t)w.tile_cap * sizeof(Tile));
    w.ntiles = off; off = align_up(off + 2 * sizeof(int32_t));   // tile count, one-tile-per-expert flag
    w.total = off;
    return w;
}

bool dim_ok(int32_t v) { return v > 0 && v % kGroup == 0 && v <= MOE_MAX_DIM; }

// 0 <= N, 1 <= K <= MOE_MAX_TOPK and N*K < 2^31, tested without forming an overflowing product
bool slots_ok(int64_t N, int32_t K) {
    return N >= 0 && K >= 1 && K <= MOE_MAX_TOPK && N <= 0x7fffffffLL / K;
}

// The many-row kernels address activations with 32-bit byte offsets from a per-block base:
// token rows x d (gate|up) and sorted rows x d_ff (down) must stay below 2^32 bytes.
// Larger batches use the 16-row kernel, which addresses with 64 bits.
bool fits_32bit_offsets(int64_t N, int64_t rows, int32_t d, int32_t d_ff) {
    const int64_t lim = (int64_t)1 << 32;
    return N * (int64_t)d < lim && rows * (int64_t)d_ff < lim;
}

TileShape choose_shape(int64_t N, int64_t rows, int32_t E, int32_t d, int32_t d_ff, uint32_t flags) {
    if (!fits_32bit_offsets(N, rows, d, d_ff)) return TileShape::Rows16;
    switch (flags & MOE_FLAG_TILE_MASK) {
        case MOE_FLAG_TILE_16: return TileShape::Rows16;
        case MOE_FLAG_TILE_128: return TileShape::Rows128;
        case MOE_FLAG_TILE_192: return TileShape::Rows192;
        case MOE_FLAG_TILE_224: return TileShape::Rows224;
        case MOE_FLAG_TILE_256: return TileShape::Rows256;
        default: break;
    }
    const int64_t touched = rows < E ? rows : E;
    const int64_t per = touched > 0 ? rows / touched : 0;  // expected rows per touched expert
    // The 16-row kernel streams weights fastest, but it reads an expert's weights once per
    // 16-row tile, and above about 6 rows per expert the 128-row kernel, which reads them once,
    // is faster (measured at K2 shapes: 2.62 vs 2.63 ms at 5.3 rows, 2.68 vs 2.64 at 6.7, 5.35
    // vs 2.82 at 21).
    if (per < 6) return TileShape::Rows16;
    // Above that, the height whose tiles the experts' rows fill best: a tile costs its
    // expert's whole weight stream however few rows it holds, and the 224-row kernel does
    // more work per cycle than the 192-row one. Measured at K2 shapes (uniform top-8 routing
    // over 384 experts, 3,072-24,576 tokens), the fastest height was:
    //   128 up to about 107 rows per expert (one tile each);
    //   224 from 112 to 213 (one tile each; 2-4% faster than 192);
    //   128 from 224 to 256 (two full tiles; 224 leaves a second, nearly empty tile);
    //   192 from 267 to 320, 224 at 427, 192 at 512 and above (the shard's 1,365).
    // (The 256-row gate|up kernel, with its bf16 operands widened in registers, spills; it
    // remains for the flag only.)
    if (per < 110) return TileShape::Rows128;
    if (per < 220) return TileShape::Rows224;
    if (per < 262) return TileShape::Rows128;
    if (per < 380) return TileShape::Rows192;
    if (per < 460) return TileShape::Rows224;
    return TileShape::Rows192;
}

}  // namespace

extern "C" {

const char* moe_status_string(int status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_ERR_NULL: return "a required pointer is NULL";
        case MOE_ERR_SHAPE: return "a size is out of range";
        case MOE_ERR_ALIGN: return "a pointer is not suitably aligned";
        case MOE_ERR_WORKSPACE: return "workspace too small";
        case MOE_ERR_BAD_ID: return "an expert id is outside [0, E)";
        case MOE_ERR_DUP_ID: return "an expert id is repeated within a token";
        case MOE_ERR_HIP: return "a HIP runtime call failed";
        case MOE_ERR_DEVICE: return "the current device is not a gfx950 GPU";
        default: return "unknown status";
    }
}

int moe_last_hip_error(void) { return g_last_hip_error; }

size_t moe_dispatch_workspace_size(int64_t N, int32_t K, int32_t E) {
    if (!slots_ok(N, K) || E < 1 || E > MOE_MAX_EXPERTS || K > E) return 0;
    return dispatch_layout(N, K, E).total;
}

moe_status moe_dispatch(const int32_t* topk_ids, int64_t N, int32_t K, int32_t E, int32_t* counts,
                        int32_t* offsets, int32_t* sorted_slot, int32_t* slot_pos, void* workspace,
                        size_t workspace_bytes, uint32_t flags, void* stream) {
    if (!slots_ok(N, K) || E < 1 || E > MOE_MAX_EXPERTS || K > E) return MOE_ERR_SHAPE;
    if (!counts || !offsets || !workspace) return MOE_ERR_NULL;
    if (N > 0 && (!topk_ids || !sorted_slot || !slot_pos)) return MOE_ERR_NULL;
    if (!aligned(topk_ids, 4) || !aligned(counts, 4) || !aligned(offsets, 4) || !aligned(sorted_slot, 4) ||
        !aligned(slot_pos, 4) || !aligned(workspace, 16))
        return MOE_ERR_ALIGN;
    const DispatchWs L = dispatch_layout(N, K, E);
    if (workspace_bytes < L.total) return MOE_ERR_WORKSPACE;
    moe_status st = check_device();
    if (st != MOE_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    uint8_t* ws = (uint8_t*)workspace;
    int32_t* err = (int32_t*)(ws + L.err);
    const bool checked = (flags & MOE_FLAG_CHECKED) != 0;
    {
        ProfScope ps(MOE_KERNEL_DISPATCH, s);
        MOE_HIP(launch_dispatch(topk_ids, N, K, E, counts, offsets, sorted_slot, slot_pos,
                                (int32_t*)(ws + L.chunk_counts), err, checked, s));
    }
    if (checked) {
        int32_t h = 0;
        MOE_HIP(hipMemcpyAsync(&h, err, sizeof(h), hipMemcpyDeviceToHost, s));
        MOE_HIP(hipStreamSynchronize(s));
        if (h & 1) return MOE_ERR_BAD_ID;
        if (h & 2) return MOE_ERR_DUP_ID;
    }
    return MOE_OK;
}

size_t moe_swiglu_workspace_size(int64_t N, int32_t K, int32_t E, int32_t d, int32_t d_ff) {
    if (!slots_ok(N, K) || E < 1 || E > MOE_MAX_EXPERTS || K > E || !dim_ok(d) || !dim_ok(d_ff)) return 0;
    return swiglu_layout(N, K, E, d, d_ff).total;
}

size_t moe_swiglu_q_workspace_size(int64_t N, int32_t K, int32_t E, int32_t d, int32_t d_ff) {
    if (!slots_ok(N, K) || E < 1 || E > MOE_MAX_EXPERTS || K > E || !dim_ok(d) || !dim_ok(d_ff)) return 0;
    return swiglu_layout(N, K, E, d, d_ff, false).total;
}

}  // extern "C"

namespace {

// Shared by moe_grouped_swiglu (with_x: x is the bf16 input, quantised into the workspace),
// moe_grouped_swiglu_q (xq_in and xs_in are given) and moe_grouped_swiglu_top1 (top1_w
// given, K = 1: y_sorted is then the token-order output, written by the down epilogue).
moe_status grouped_swiglu(bool with_x, const uint16_t* x, const uint8_t* xq_in, const float* xs_in, int64_t N,
                          int32_t K, int32_t E, int32_t d, int32_t d_ff, const int32_t* offsets,
                          const int32_t* sorted_slot,
                          const uint8_t* w_gate, const float* s_gate, const uint8_t* w_up, const float* s_up,
                          const uint8_t* w_down, const float* s_down, uint16_t* y_sorted, void* workspace,
                          size_t workspace_bytes, uint32_t flags, void* stream, const float* top1_w = nullptr,
                          const int32_t* top1_slot_pos = nullptr, bool top1 = false) {
    if (!slots_ok(N, K) || E < 1 || E > MOE_MAX_EXPERTS || K > E || !dim_ok(d) || !dim_ok(d_ff))
        return MOE_ERR_SHAPE;
    if (N == 0) return MOE_OK;
    if ((with_x ? !x : (!xq_in || !xs_in)) || !offsets || !sorted_slot || !w_gate || !s_gate || !w_up || !s_up ||
        !w_down || !s_down || !y_sorted || !workspace || (top1 && (!top1_w || !top1_slot_pos)))
        return MOE_ERR_NULL;
    if (top1 && (!aligned(top1_w, 4) || !aligned(top1_slot_pos, 4))) return MOE_ERR_ALIGN;
    if ((with_x ? !aligned(x, 16) : (!aligned(xq_in, 16) || !aligned(xs_in, 4))) || !aligned(w_gate, 16) ||
        !aligned(w_up, 16) || !aligned(w_down, 16) || !aligned(y_sorted, 16) || !aligned(workspace, 16) ||
        !aligned(offsets, 4) || !aligned(sorted_slot, 4) || !aligned(s_gate, 4) || !aligned(s_up, 4) ||
        !aligned(s_down, 4))
        return MOE_ERR_ALIGN;
    const SwigluWs L = swiglu_layout(N, K, E, d, d_ff, with_x);
    if (workspace_bytes < L.total) return MOE_ERR_WORKSPACE;
    moe_status st = check_device();
    if (st != MOE_OK) return st;

    hipStream_t s = (hipStream_t)stream;
    uint8_t* ws = (uint8_t*)workspace;
    const uint8_t* xq = with_x ? ws + L.xq : xq_in;
    const float* xs = with_x ? (const float*)(ws + L.xs) : xs_in;
    uint8_t* hq = ws + L.hq;
    float* hs = (float*)(ws + L.hs);
    Tile* tiles = (Tile*)(ws + L.tiles);
    int32_t* ntiles = (int32_t*)(ws + L.ntiles);
    const int64_t rows = N * K;
    const TileShape shape = choose_shape(N, rows, E, d, d_ff, flags);
    const int BM = tile_rows(shape);
    const int64_t cap = max_tiles(rows, E, BM);

    if (with_x) {
        // the tile list is built by the last workgroup of the quantisation launch; for a top-1
        // call the same launch also writes the +0 rows of the tokens the dispatch left out
        const TileJob job{offsets, E, rows, BM, cap, tiles, ntiles};
        const ZeroRowsJob zero{top1_slot_pos, rows, y_sorted};
        ProfScope ps(MOE_KERNEL_QUANT, s);
        MOE_HIP(launch_quantize_rows(x, N, d, ws + L.xq, (float*)(ws + L.xs), s, &job, top1 ? &zero : nullptr));
    } else {
        ProfScope ps(MOE_KERNEL_DISPATCH, s);
        MOE_HIP(launch_build_tiles(offsets, E, rows, BM, cap, tiles, ntiles, s));
    }
    {
        GateUpArgs a{};
        a.xq = xq; a.xs = xs; a.sorted_slot = sorted_slot; a.N = N; a.K = K; a.rows = rows;
        a.d = d; a.d_ff = d_ff; a.wg = w_gate; a.sg = s_gate; a.wu = w_up; a.su = s_up;
        a.tiles = tiles; a.num_tiles = ntiles; a.max_tiles = cap; a.hq = hq; a.hs = hs;
        ProfScope ps(MOE_KERNEL_GATE_UP, s);
        MOE_HIP(launch_gate_up(a, shape, s));
    }
    {
        DownArgs a{};
        a.hq = hq; a.hs = hs; a.rows = rows; a.d = d; a.d_ff = d_ff; a.wd = w_down; a.sd = s_down;
        a.tiles = tiles; a.num_tiles = ntiles; a.max_tiles = cap; a.y = y_sorted;
        if (top1) {
            a.scatter = sorted_slot; a.scatter_w = top1_w; a.out_rows = N;
        }
        ProfScope ps(MOE_KERNEL_DOWN, s);
        MOE_HIP(launch_down(a, shape, s));
    }
    return MOE_OK;
}

moe_status combine(const uint16_t* y_sorted, const int32_t* slot_pos, const float* topk_w, const uint16_t* shared,
                   const uint16_t* residual, bool need_residual, int64_t N, int32_t K, int32_t d, uint16_t* out,
                   void* stream) {
    if (!slots_ok(N, K) || !dim_ok(d)) return MOE_ERR_SHAPE;
    if (N == 0) return MOE_OK;
    if (!y_sorted || !slot_pos || !topk_w || !out || (need_residual && !residual)) return MOE_ERR_NULL;
    if (!aligned(y_sorted, 16) || !aligned(out, 16) || (shared && !aligned(shared, 16)) ||
        (residual && !aligned(residual, 16)) || !aligned(slot_pos, 4) || !aligned(topk_w, 4))
        return MOE_ERR_ALIGN;
    moe_status st = check_device();
    if (st != MOE_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    ProfScope ps(MOE_KERNEL_COMBINE, s);
    MOE_HIP(launch_combine(y_sorted, slot_pos, topk_w, shared, residual, N, K, d, out, s));
    return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_grouped_swiglu(const uint16_t* x, int64_t N, int32_t K, int32_t E, int32_t d, int32_t d_ff,
                              const int32_t* offsets, const int32_t* sorted_slot, const uint8_t* w_gate,
                              const float* s_gate, const uint8_t* w_up, const float* s_up,
                              const uint8_t* w_down, const float* s_down, uint16_t* y_sorted, void* workspace,
                              size_t workspace_bytes, uint32_t flags, void* stream) {
    return grouped_swiglu(true, x, nullptr, nullptr, N, K, E, d, d_ff, offsets, sorted_slot, w_gate, s_gate, w_up,
                          s_up, w_down, s_down, y_sorted, workspace, workspace_bytes, flags, stream);
}

moe_status moe_grouped_swiglu_top1(const uint16_t* x, int64_t N, int32_t E, int32_t d, int32_t d_ff,
                                   const int32_t* offsets, const int32_t* sorted_slot, const int32_t* slot_pos,
                                   const float* topk_w, const uint8_t* w_gate, const float* s_gate,
                                   const uint8_t* w_up, const float* s_up, const uint8_t* w_down,
                                   const float* s_down, uint16_t* out, void* workspace, size_t workspace_bytes,
                                   uint32_t flags, void* stream) {
    return grouped_swiglu(true, x, nullptr, nullptr, N, 1, E, d, d_ff, offsets, sorted_slot, w_gate, s_gate, w_up,
                          s_up, w_down, s_down, out, workspace, workspace_bytes, flags, stream, topk_w, slot_pos,
                          true);
}

moe_status moe_grouped_swiglu_q(const uint8_t* xq, const float* xs, int64_t N, int32_t K, int32_t E, int32_t d,
                                int32_t d_ff, const int32_t* offsets, const int32_t* sorted_slot,
                                const uint8_t* w_gate, const float* s_gate, const uint8_t* w_up,
                                const float* s_up, const uint8_t* w_down, const float* s_down,
                                uint16_t* y_sorted, void* workspace, size_t workspace_bytes, uint32_t flags,
                                void* stream) {
    return grouped_swiglu(false, nullptr, xq, xs, N, K, E, d, d_ff, offsets, sorted_slot, w_gate, s_gate, w_up,
                          s_up, w_down, s_down, y_sorted, workspace, workspace_bytes, flags, stream);
}

moe_status moe_combine(const uint16_t* y_sorted, const int32_t* slot_pos, const float* topk_w,
                       const uint16_t* shared, int64_t N, int32_t K, int32_t d, uint16_t* out, void* stream) {
    return combine(y_sorted, slot_pos, topk_w, shared, nullptr, false, N, K, d, out, stream);
}

moe_status moe_combine_residual(const uint16_t* y_sorted, const int32_t* slot_pos, const float* topk_w,
                                const uint16_t* shared, const uint16_t* residual, int64_t N, int32_t K, int32_t d,
                                uint16_t* out, void* stream) {
    return combine(y_sorted, slot_pos, topk_w, shared, residual, true, N, K, d, out, stream);
}

moe_status moe_quantize_rows(const uint16_t* x, int64_t rows, int32_t cols, uint8_t* q, float* s_out,
                             void* stream) {
    if (rows < 0 || rows > 0x7fffffffLL || !dim_ok(cols)) return MOE_ERR_SHAPE;
    if (rows == 0) return MOE_OK;
    if (!x || !q || !s_out) return MOE_ERR_NULL;
    if (!aligned(x, 16) || !aligned(q, 16) || !aligned(s_out, 4)) return MOE_ERR_ALIGN;
    moe_status st = check_device();
    if (st != MOE_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    ProfScope ps(MOE_KERNEL_QUANT, s);
    MOE_HIP(launch_quantize_rows(x, rows, cols, q, s_out, s));
    return MOE_OK;
}

moe_status moe_rmsnorm_quantize_rows(const uint16_t* h, const uint16_t* gain, float eps, int64_t rows, int32_t cols,
                                     uint16_t* y, uint8_t* q, float* s_out, void* stream) {
    if (rows < 0 || rows > 0x7fffffffLL || !dim_ok(cols) || !(eps >= 0.0f) || eps == INFINITY) return MOE_ERR_SHAPE;
    if (rows == 0) return MOE_OK;
    if (!h || !gain || !q || !s_out) return MOE_ERR_NULL;
    if (!aligned(h, 16) || !aligned(gain, 16) || (y && !aligned(y, 16)) || !aligned(q, 16) || !aligned(s_out, 4))
        return MOE_ERR_ALIGN;
    moe_status st = check_device();
    if (st != MOE_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    ProfScope ps(MOE_KERNEL_QUANT, s);
    MOE_HIP(launch_rmsnorm_quantize(h, gain, eps, rows, cols, y, q, s_out, s));
    return MOE_OK;
}

moe_status moe_profile_enable(int on) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof_mask = on != 0 ? (1u << MOE_KERNEL_KINDS) - 1u : 0u;
    return MOE_OK;
}

moe_status moe_profile_enable_kinds(uint32_t kind_mask) {
    if (kind_mask >> MOE_KERNEL_KINDS) return MOE_ERR_SHAPE;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof_mask = kind_mask;
    return MOE_OK;
}

static moe_status drain_pending_locked() {
    for (const Pending& p : g_prof_pending) {
        hipError_t e = hipEventSynchronize(p.b);
        if (e != hipSuccess) return hip_fail(e);
        float ms = 0.f;
        e = hipEventElapsedTime(&ms, p.a, p.b);
        if (e != hipSuccess) return hip_fail(e);
        g_prof_ms[p.kind] += ms;
        g_prof_n[p.kind] += 1;
        g_prof_pool.push_back(p.a);
        g_prof_pool.push_back(p.b);
    }
    g_prof_pending.clear();
    return MOE_OK;
}

moe_status moe_profile_reset(void) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    moe_status st = drain_pending_locked();
    for (int i = 0; i < MOE_KERNEL_KINDS; ++i) {
        g_prof_ms[i] = 0;
        g_prof_n[i] = 0;
    }
    return st;
}

moe_status moe_profile_read(int kind, double* total_ms, int64_t* launches) {
    if (kind < 0 || kind >= MOE_KERNEL_KINDS) return MOE_ERR_SHAPE;
    if (!total_ms || !launches) return MOE_ERR_NULL;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    moe_status st = drain_pending_locked();
    *total_ms = g_prof_ms[kind];
    *launches = g_prof_n[kind];
    return st;
}

}  // extern "C"
