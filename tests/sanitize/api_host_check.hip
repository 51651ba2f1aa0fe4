// Host-side check of libmoe's C ABI under AddressSanitizer and UndefinedBehaviorSanitizer,
// without a GPU. Test infrastructure: built from the library's own api.hip compiled for the
// host only, linked with this file, which stands in for the kernel launchers and the few HIP
// runtime calls api.hip makes.
//
//   * The stand-in launchers read and write every byte the real kernels may touch, with the
//     sizes their arguments imply, so AddressSanitizer sees any pointer the host code computes
//     that runs past a buffer: buffers here are allocated with exactly the size the caller is
//     told to provide (the workspaces with exactly the *_workspace_size bytes).
//   * The regions a call carves out of its workspace (activation codes and scales, h codes and
//     scales, the tile list and its count, the dispatch counters and flag) are recorded with a
//     name each; a region of one name must start where every other use of that name starts,
//     and regions of different names must not overlap. (AddressSanitizer cannot see an overlap
//     inside one allocation.)
//   * Every host-side error path is driven (null, size, alignment, workspace, no device, a
//     device that is not gfx950, checked-mode id errors) and its status compared.
//   * The size queries are evaluated at the extremes of their arguments, where integer
//     overflow would be undefined behaviour.
// Exit status 0 when every check holds; a sanitizer report aborts the run.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <string>
#include <vector>

#include "moe.h"
#include "moe_internal.h"

using namespace moe;

// ---------------------------------------------------------------- stand-in HIP runtime
static int g_device = -1;        // device hipGetDevice reports; -1: no device
static int g_err_bits = 0;       // what the checked dispatch's device-side id check finds
static char g_events[4096][16];  // storage behind the stand-in events
static int g_nevents = 0;

hipError_t hipGetDevice(int* d) {
    if (g_device < 0) return hipErrorNoDevice;
    *d = g_device;
    return hipSuccess;
}
hipError_t hipGetDevicePropertiesR0600(hipDeviceProp_tR0600* prop, int device) {
    memset(prop, 0, sizeof(*prop));
    strcpy(prop->gcnArchName, device == 0 ? "gfx950:sramecc+:xnack-" : "gfx942:sramecc+:xnack-");
    return hipSuccess;
}
hipError_t hipEventCreate(hipEvent_t* e) {
    if (g_nevents >= 4096) return hipErrorOutOfMemory;
    *e = reinterpret_cast<hipEvent_t>(g_events[g_nevents++]);
    return hipSuccess;
}
hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }
hipError_t hipEventSynchronize(hipEvent_t) { return hipSuccess; }
hipError_t hipEventElapsedTime(float* ms, hipEvent_t, hipEvent_t) {
    *ms = 0.5f;
    return hipSuccess;
}
hipError_t hipMemcpyAsync(void* dst, const void* src, size_t n, hipMemcpyKind, hipStream_t) {
    memcpy(dst, src, n);
    return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }

// ---------------------------------------------------------------- touched regions
struct Region {
    std::string name;
    const uint8_t* p;
    size_t n;
};
static std::vector<Region> g_regions;
static int g_launches = 0;
static int g_gate_up_rows = -1;   // tile height of the last gate|up launch
static volatile uint8_t g_sink;

static void rd(const char* name, const void* p, size_t n) {
    if (!n) return;
    const uint8_t* b = static_cast<const uint8_t*>(p);
    uint8_t x = 0;
    for (size_t i = 0; i < n; ++i) x ^= b[i];
    g_sink = x;
    g_regions.push_back({name, b, n});
}
static void wr(const char* name, void* p, size_t n) {
    if (!n) return;
    memset(p, 0x5A, n);
    g_regions.push_back({name, static_cast<uint8_t*>(p), n});
}

namespace moe {

hipError_t launch_rmsnorm_quantize(const uint16_t* x, const uint16_t* gain, float, int64_t rows, int cols,
                                   uint16_t* y, uint8_t* q, float* s, hipStream_t) {
    ++g_launches;
    rd("rms.x", x, (size_t)rows * cols * 2);
    rd("rms.gain", gain, (size_t)cols * 2);
    if (y) wr("rms.y", y, (size_t)rows * cols * 2);
    wr("rms.q", q, (size_t)rows * cols);
    wr("rms.s", s, (size_t)rows * (cols / kGroup) * 4);
    return hipSuccess;
}

hipError_t launch_dispatch(const int32_t* ids, int64_t N, int K, int E, int32_t* counts, int32_t* offsets,
                           int32_t* sorted_slot, int32_t* slot_pos, int32_t* chunk_counts, int32_t* err_flag,
                           bool checked, hipStream_t) {
    ++g_launches;
    const int64_t NK = N * K;
    rd("ids", ids, (size_t)NK * 4);
    wr("counts", counts, (size_t)E * 4);
    wr("offsets", offsets, (size_t)(E + 1) * 4);
    wr("sorted_slot", sorted_slot, (size_t)NK * 4);
    wr("slot_pos", slot_pos, (size_t)NK * 4);
    const int64_t nchunks = (NK + kDispatchChunk - 1) / kDispatchChunk;
    wr("chunk_counts", chunk_counts, (size_t)nchunks * E * 4);
    wr("err", err_flag, 4);
    *err_flag = checked ? g_err_bits : 0;
    // a valid dispatch for what follows: every slot in order, expert offsets by counting
    for (int e = 0; e <= E; ++e) offsets[e] = 0;
    for (int64_t s = 0; s < NK; ++s) {
        const int e = ids[s] >= 0 && ids[s] < E ? ids[s] : 0;
        ++offsets[e + 1];
    }
    for (int e = 0; e < E; ++e) offsets[e + 1] += offsets[e];
    for (int64_t s = 0; s < NK; ++s) sorted_slot[s] = slot_pos[s] = (int32_t)s;
    return hipSuccess;
}

hipError_t launch_quantize_rows(const uint16_t* x, int64_t rows, int cols, uint8_t* q, float* s, hipStream_t,
                                const TileJob* tj, const ZeroRowsJob* zj) {
    ++g_launches;
    rd("x", x, (size_t)rows * cols * 2);
    wr("xq", q, (size_t)rows * cols);
    wr("xs", s, (size_t)rows * (cols / kGroup) * 4);
    if (tj && tj->tiles) {
        rd("offsets", tj->offsets, (size_t)(tj->E + 1) * 4);
        wr("tiles", tj->tiles, (size_t)tj->cap * sizeof(Tile));
        wr("ntiles", tj->num_tiles, 2 * 4);
    }
    if (zj && zj->out) {
        rd("slot_pos", zj->slot_pos, (size_t)rows * 4);
        wr("out", zj->out, (size_t)rows * cols * 2);
    }
    return hipSuccess;
}

hipError_t launch_build_tiles(const int32_t* offsets, int E, int64_t, int, int64_t cap, Tile* tiles,
                              int32_t* num_tiles, hipStream_t) {
    ++g_launches;
    rd("offsets", offsets, (size_t)(E + 1) * 4);
    wr("tiles", tiles, (size_t)cap * sizeof(Tile));
    wr("ntiles", num_tiles, 2 * 4);
    return hipSuccess;
}

hipError_t launch_gate_up(const GateUpArgs& a, TileShape shape, hipStream_t) {
    ++g_launches;
    g_gate_up_rows = tile_rows(shape);
    rd("xq", a.xq, (size_t)a.N * a.d);
    rd("xs", a.xs, (size_t)a.N * (a.d / kGroup) * 4);
    rd("sorted_slot", a.sorted_slot, (size_t)a.rows * 4);
    rd("tiles", a.tiles, (size_t)a.max_tiles * sizeof(Tile));
    rd("ntiles", a.num_tiles, 2 * 4);
    wr("hq", a.hq, (size_t)a.rows * a.d_ff);
    wr("hs", a.hs, (size_t)a.rows * (a.d_ff / kGroup) * 4);
    return hipSuccess;
}

hipError_t launch_down(const DownArgs& a, TileShape, hipStream_t) {
    ++g_launches;
    rd("hq", a.hq, (size_t)a.rows * a.d_ff);
    rd("hs", a.hs, (size_t)a.rows * (a.d_ff / kGroup) * 4);
    rd("tiles", a.tiles, (size_t)a.max_tiles * sizeof(Tile));
    rd("ntiles", a.num_tiles, 2 * 4);
    if (a.scatter) {
        rd("sorted_slot", a.scatter, (size_t)a.rows * 4);
        rd("topk_w", a.scatter_w, (size_t)a.out_rows * 4);
        wr("out", a.y, (size_t)a.out_rows * a.d * 2);
    } else {
        wr("y_sorted", a.y, (size_t)a.rows * a.d * 2);
    }
    return hipSuccess;
}

hipError_t launch_combine(const uint16_t* y, const int32_t* slot_pos, const float* w, const uint16_t* shared,
                          const uint16_t* residual, int64_t N, int K, int d, uint16_t* out, hipStream_t) {
    ++g_launches;
    rd("y_sorted", y, (size_t)N * K * d * 2);
    rd("slot_pos", slot_pos, (size_t)N * K * 4);
    rd("topk_w", w, (size_t)N * K * 4);
    if (shared) rd("shared", shared, (size_t)N * d * 2);
    if (residual) rd("residual", residual, (size_t)N * d * 2);
    wr("out", out, (size_t)N * d * 2);
    return hipSuccess;
}

}  // namespace moe

// ---------------------------------------------------------------- checks
static int g_checks = 0, g_fail = 0;
#define CHECK(cond, ...)                                     \
    do {                                                     \
        ++g_checks;                                          \
        if (!(cond)) {                                       \
            ++g_fail;                                        \
            printf("FAIL %s:%d: %s -- ", __FILE__, __LINE__, #cond); \
            printf(__VA_ARGS__);                             \
            printf("\n");                                    \
        }                                                    \
    } while (0)

// A buffer of exactly n bytes (256-byte aligned start), freed at scope end.
struct Buf {
    void* p = nullptr;
    size_t n = 0;
    explicit Buf(size_t bytes) : n(bytes) {
        if (posix_memalign(&p, 256, bytes ? bytes : 1) != 0) {
            printf("out of host memory\n");
            exit(3);
        }
    }
    ~Buf() { free(p); }
    Buf(const Buf&) = delete;
    Buf& operator=(const Buf&) = delete;
    template <typename T>
    T* as() const { return static_cast<T*>(p); }
};

// Workspace regions of the last call: named regions inside [ws, ws + bytes) must agree.
static void check_workspace(const char* what, const Buf& ws) {
    const uint8_t* lo = ws.as<uint8_t>();
    const uint8_t* hi = lo + ws.n;
    std::vector<Region> in;
    for (const Region& r : g_regions)
        if (r.p >= lo && r.p < hi) {
            CHECK(r.p + r.n <= hi, "%s: region %s ends past the workspace", what, r.name.c_str());
            in.push_back(r);
        }
    for (size_t i = 0; i < in.size(); ++i)
        for (size_t j = i + 1; j < in.size(); ++j) {
            const Region &a = in[i], &b = in[j];
            if (a.name == b.name) {
                CHECK(a.p == b.p, "%s: two uses of %s start at different offsets", what, a.name.c_str());
            } else {
                const bool disjoint = a.p + a.n <= b.p || b.p + b.n <= a.p;
                CHECK(disjoint, "%s: workspace regions %s and %s overlap", what, a.name.c_str(), b.name.c_str());
            }
        }
}

static void begin() {
    g_regions.clear();
    g_launches = 0;
}

struct Shape {
    int64_t N;
    int32_t K, E, d, d_ff;
};

static const uint32_t kTiles[] = {0, MOE_FLAG_TILE_16, MOE_FLAG_TILE_128, MOE_FLAG_TILE_192, MOE_FLAG_TILE_224,
                                  MOE_FLAG_TILE_256};

// Every entry point with valid arguments on exactly sized buffers.
static void valid_calls(const Shape& sh) {
    const int64_t N = sh.N, NK = sh.N * sh.K;
    const int32_t K = sh.K, E = sh.E, d = sh.d, F = sh.d_ff;
    char what[160];
    snprintf(what, sizeof what, "N=%lld K=%d E=%d d=%d d_ff=%d", (long long)N, K, E, d, F);
    Buf ids(NK * 4), counts(E * 4), offsets((E + 1) * 4), sorted(NK * 4), slot_pos(NK * 4);
    for (int64_t s = 0; s < NK; ++s) ids.as<int32_t>()[s] = (int32_t)((s * 7 + s / K) % E);
    Buf x(N * d * 2), topk_w(NK * 4), y_sorted(NK * d * 2), out(N * d * 2), shared(N * d * 2), resid(N * d * 2);
    Buf wg((size_t)E * F * d), wu((size_t)E * F * d), wd((size_t)E * d * F);
    Buf sg((size_t)E * (F / 128) * (d / 128) * 4), su(sg.n), sd(sg.n);
    Buf xq(N * d), xs(N * (d / 128) * 4), gain(d * 2), ynorm(N * d * 2);

    // dispatch, plain and checked
    for (int checked = 0; checked < 2; ++checked) {
        Buf ws(moe_dispatch_workspace_size(N, K, E));
        begin();
        const moe_status st = moe_dispatch(ids.as<int32_t>(), N, K, E, counts.as<int32_t>(), offsets.as<int32_t>(),
                                           sorted.as<int32_t>(), slot_pos.as<int32_t>(), ws.p, ws.n,
                                           checked ? MOE_FLAG_CHECKED : 0, nullptr);
        CHECK(st == MOE_OK, "%s: moe_dispatch checked=%d -> %d", what, checked, st);
        check_workspace(what, ws);
    }
    // grouped experts at every tile height
    for (uint32_t flags : kTiles) {
        Buf ws(moe_swiglu_workspace_size(N, K, E, d, F));
        begin();
        moe_status st = moe_grouped_swiglu(x.as<uint16_t>(), N, K, E, d, F, offsets.as<int32_t>(),
                                           sorted.as<int32_t>(), wg.as<uint8_t>(), sg.as<float>(), wu.as<uint8_t>(),
                                           su.as<float>(), wd.as<uint8_t>(), sd.as<float>(), y_sorted.as<uint16_t>(),
                                           ws.p, ws.n, flags, nullptr);
        CHECK(st == MOE_OK && g_launches == (N ? 3 : 0), "%s flags=%u: moe_grouped_swiglu -> %d (%d launches)", what,
              flags, st, g_launches);
        check_workspace(what, ws);

        Buf wsq(moe_swiglu_q_workspace_size(N, K, E, d, F));
        begin();
        st = moe_grouped_swiglu_q(xq.as<uint8_t>(), xs.as<float>(), N, K, E, d, F, offsets.as<int32_t>(),
                                  sorted.as<int32_t>(), wg.as<uint8_t>(), sg.as<float>(), wu.as<uint8_t>(),
                                  su.as<float>(), wd.as<uint8_t>(), sd.as<float>(), y_sorted.as<uint16_t>(), wsq.p,
                                  wsq.n, flags, nullptr);
        CHECK(st == MOE_OK, "%s flags=%u: moe_grouped_swiglu_q -> %d", what, flags, st);
        check_workspace(what, wsq);

        if (K == 1) {
            begin();
            st = moe_grouped_swiglu_top1(x.as<uint16_t>(), N, E, d, F, offsets.as<int32_t>(), sorted.as<int32_t>(),
                                         slot_pos.as<int32_t>(), topk_w.as<float>(), wg.as<uint8_t>(),
                                         sg.as<float>(), wu.as<uint8_t>(), su.as<float>(), wd.as<uint8_t>(),
                                         sd.as<float>(), out.as<uint16_t>(), ws.p, ws.n, flags, nullptr);
            CHECK(st == MOE_OK, "%s flags=%u: moe_grouped_swiglu_top1 -> %d", what, flags, st);
            check_workspace(what, ws);
        }
    }
    // combine, with a shared expert, with a residual, in place on the residual
    begin();
    CHECK(moe_combine(y_sorted.as<uint16_t>(), slot_pos.as<int32_t>(), topk_w.as<float>(), nullptr, N, K, d,
                      out.as<uint16_t>(), nullptr) == MOE_OK, "%s: moe_combine", what);
    CHECK(moe_combine(y_sorted.as<uint16_t>(), slot_pos.as<int32_t>(), topk_w.as<float>(), shared.as<uint16_t>(), N,
                      K, d, out.as<uint16_t>(), nullptr) == MOE_OK, "%s: moe_combine shared", what);
    CHECK(moe_combine_residual(y_sorted.as<uint16_t>(), slot_pos.as<int32_t>(), topk_w.as<float>(),
                               shared.as<uint16_t>(), resid.as<uint16_t>(), N, K, d, out.as<uint16_t>(),
                               nullptr) == MOE_OK, "%s: moe_combine_residual", what);
    CHECK(moe_combine_residual(y_sorted.as<uint16_t>(), slot_pos.as<int32_t>(), topk_w.as<float>(), nullptr,
                               resid.as<uint16_t>(), N, K, d, resid.as<uint16_t>(), nullptr) == MOE_OK,
          "%s: moe_combine_residual in place", what);
    // quantisation alone and with the RMSNorm, with and without the normalised rows
    CHECK(moe_quantize_rows(x.as<uint16_t>(), N, d, xq.as<uint8_t>(), xs.as<float>(), nullptr) == MOE_OK,
          "%s: moe_quantize_rows", what);
    CHECK(moe_rmsnorm_quantize_rows(x.as<uint16_t>(), gain.as<uint16_t>(), 1e-6f, N, d, nullptr, xq.as<uint8_t>(),
                                    xs.as<float>(), nullptr) == MOE_OK, "%s: moe_rmsnorm_quantize_rows", what);
    CHECK(moe_rmsnorm_quantize_rows(x.as<uint16_t>(), gain.as<uint16_t>(), 0.0f, N, d, ynorm.as<uint16_t>(),
                                    xq.as<uint8_t>(), xs.as<float>(), nullptr) == MOE_OK,
          "%s: moe_rmsnorm_quantize_rows keeping y", what);
}

// The host-side rejections of include/moe.h: each returns its status before any launch.
static void error_paths() {
    Buf b(1 << 16);
    uint8_t* p = b.as<uint8_t>();
    void* v = p;
    int32_t* i = b.as<int32_t>();
    float* f = b.as<float>();
    uint16_t* h = b.as<uint16_t>();
    uint8_t* mis2 = p + 2;
    auto none = [&](const char* what, moe_status st, moe_status want) {
        CHECK(st == want && g_launches == 0, "%s -> %d, want %d (%d launches)", what, st, want, g_launches);
    };
    begin();
    // dispatch: K > E, K < 1, E < 1, N < 0, E and K beyond the limits, N*K >= 2^31
    none("dispatch K>E", moe_dispatch(i, 4, 9, 8, i, i, i, i, v, 1 << 16, 0, nullptr), MOE_ERR_SHAPE);
    none("dispatch K<1", moe_dispatch(i, 4, 0, 8, i, i, i, i, v, 1 << 16, 0, nullptr), MOE_ERR_SHAPE);
    none("dispatch E<1", moe_dispatch(i, 4, 1, 0, i, i, i, i, v, 1 << 16, 0, nullptr), MOE_ERR_SHAPE);
    none("dispatch N<0", moe_dispatch(i, -1, 2, 8, i, i, i, i, v, 1 << 16, 0, nullptr), MOE_ERR_SHAPE);
    none("dispatch E>max", moe_dispatch(i, 4, 2, 8193, i, i, i, i, v, 1 << 16, 0, nullptr), MOE_ERR_SHAPE);
    none("dispatch K>max", moe_dispatch(i, 4, 65, 100, i, i, i, i, v, 1 << 16, 0, nullptr), MOE_ERR_SHAPE);
    none("dispatch NK", moe_dispatch(i, (int64_t)1 << 40, 8, 8, i, i, i, i, v, 1 << 16, 0, nullptr), MOE_ERR_SHAPE);
    none("dispatch null ids", moe_dispatch(nullptr, 4, 2, 8, i, i, i, i, v, 1 << 16, 0, nullptr), MOE_ERR_NULL);
    none("dispatch null counts", moe_dispatch(i, 4, 2, 8, nullptr, i, i, i, v, 1 << 16, 0, nullptr), MOE_ERR_NULL);
    none("dispatch null ws", moe_dispatch(i, 4, 2, 8, i, i, i, i, nullptr, 1 << 16, 0, nullptr), MOE_ERR_NULL);
    none("dispatch misaligned", moe_dispatch((int32_t*)mis2, 4, 2, 8, i, i, i, i, v, 1 << 16, 0, nullptr),
         MOE_ERR_ALIGN);
    const size_t dneed = moe_dispatch_workspace_size(4, 2, 8);
    CHECK(dneed > 0, "dispatch workspace size");
    none("dispatch small ws", moe_dispatch(i, 4, 2, 8, i, i, i, i, v, dneed - 1, 0, nullptr), MOE_ERR_WORKSPACE);
    // grouped experts: dims, null, misaligned, workspace
    none("swiglu d", moe_grouped_swiglu(h, 4, 2, 8, 100, 128, i, i, p, f, p, f, p, f, h, v, 1 << 16, 0, nullptr),
         MOE_ERR_SHAPE);
    none("swiglu d_ff", moe_grouped_swiglu(h, 4, 2, 8, 128, 0, i, i, p, f, p, f, p, f, h, v, 1 << 16, 0, nullptr),
         MOE_ERR_SHAPE);
    none("swiglu d>max", moe_grouped_swiglu(h, 4, 2, 8, 65536 + 128, 128, i, i, p, f, p, f, p, f, h, v, 1 << 16, 0,
                                            nullptr), MOE_ERR_SHAPE);
    none("swiglu N=0", moe_grouped_swiglu(nullptr, 0, 2, 8, 128, 128, nullptr, nullptr, nullptr, nullptr, nullptr,
                                          nullptr, nullptr, nullptr, nullptr, nullptr, 0, 0, nullptr), MOE_OK);
    none("swiglu null w", moe_grouped_swiglu(h, 4, 2, 8, 128, 128, i, i, p, f, nullptr, f, p, f, h, v, 1 << 16, 0,
                                             nullptr), MOE_ERR_NULL);
    none("swiglu misaligned x", moe_grouped_swiglu((uint16_t*)(p + 8), 4, 2, 8, 128, 128, i, i, p, f, p, f, p, f, h,
                                                   v, 1 << 16, 0, nullptr), MOE_ERR_ALIGN);
    const size_t sneed = moe_swiglu_workspace_size(4, 2, 8, 128, 128);
    none("swiglu small ws", moe_grouped_swiglu(h, 4, 2, 8, 128, 128, i, i, p, f, p, f, p, f, h, v, sneed - 1, 0,
                                               nullptr), MOE_ERR_WORKSPACE);
    const size_t qneed = moe_swiglu_q_workspace_size(4, 2, 8, 128, 128);
    CHECK(qneed > 0 && qneed < sneed, "q workspace %zu vs %zu", qneed, sneed);
    none("swiglu_q null xs", moe_grouped_swiglu_q(p, nullptr, 4, 2, 8, 128, 128, i, i, p, f, p, f, p, f, h, v,
                                                  1 << 16, 0, nullptr), MOE_ERR_NULL);
    none("swiglu_q misaligned", moe_grouped_swiglu_q(p + 4, f, 4, 2, 8, 128, 128, i, i, p, f, p, f, p, f, h, v,
                                                     1 << 16, 0, nullptr), MOE_ERR_ALIGN);
    none("swiglu_q small ws", moe_grouped_swiglu_q(p, f, 4, 2, 8, 128, 128, i, i, p, f, p, f, p, f, h, v, qneed - 1,
                                                   0, nullptr), MOE_ERR_WORKSPACE);
    // top-1: slot_pos and weights required and aligned; the K = 1 workspace
    none("top1 null w", moe_grouped_swiglu_top1(h, 4, 8, 128, 128, i, i, i, nullptr, p, f, p, f, p, f, h, v,
                                                1 << 16, 0, nullptr), MOE_ERR_NULL);
    none("top1 null slot_pos", moe_grouped_swiglu_top1(h, 4, 8, 128, 128, i, i, nullptr, f, p, f, p, f, p, f, h, v,
                                                       1 << 16, 0, nullptr), MOE_ERR_NULL);
    none("top1 misaligned w", moe_grouped_swiglu_top1(h, 4, 8, 128, 128, i, i, i, (float*)mis2, p, f, p, f, p, f,
                                                      h, v, 1 << 16, 0, nullptr), MOE_ERR_ALIGN);
    none("top1 misaligned slot_pos", moe_grouped_swiglu_top1(h, 4, 8, 128, 128, i, i, (int32_t*)mis2, f, p, f, p,
                                                             f, p, f, h, v, 1 << 16, 0, nullptr), MOE_ERR_ALIGN);
    const size_t tneed = moe_swiglu_workspace_size(4, 1, 8, 128, 128);
    none("top1 small ws", moe_grouped_swiglu_top1(h, 4, 8, 128, 128, i, i, i, f, p, f, p, f, p, f, h, v, tneed - 1,
                                                  0, nullptr), MOE_ERR_WORKSPACE);
    // combine
    none("combine d", moe_combine(h, i, f, nullptr, 4, 2, 130, h, nullptr), MOE_ERR_SHAPE);
    none("combine K", moe_combine(h, i, f, nullptr, 4, 65, 128, h, nullptr), MOE_ERR_SHAPE);
    none("combine null", moe_combine(nullptr, i, f, nullptr, 4, 2, 128, h, nullptr), MOE_ERR_NULL);
    none("combine N=0", moe_combine(h, i, f, nullptr, 0, 2, 128, nullptr, nullptr), MOE_OK);
    none("combine misaligned shared", moe_combine(h, i, f, (uint16_t*)mis2, 4, 2, 128, h, nullptr), MOE_ERR_ALIGN);
    none("residual null", moe_combine_residual(h, i, f, nullptr, nullptr, 4, 2, 128, h, nullptr), MOE_ERR_NULL);
    // quantisation
    none("quantize cols", moe_quantize_rows(h, 3, 96, p, f, nullptr), MOE_ERR_SHAPE);
    none("quantize null", moe_quantize_rows(nullptr, 3, 128, p, f, nullptr), MOE_ERR_NULL);
    none("quantize rows=0", moe_quantize_rows(h, 0, 128, nullptr, nullptr, nullptr), MOE_OK);
    none("quantize rows", moe_quantize_rows(h, (int64_t)1 << 31, 128, p, f, nullptr), MOE_ERR_SHAPE);
    none("quantize rows max", moe_quantize_rows(h, INT64_MAX, MOE_MAX_DIM, p, f, nullptr), MOE_ERR_SHAPE);
    none("rmsnorm eps<0", moe_rmsnorm_quantize_rows(h, h, -1.0f, 4, 128, nullptr, p, f, nullptr), MOE_ERR_SHAPE);
    none("rmsnorm eps inf", moe_rmsnorm_quantize_rows(h, h, INFINITY, 4, 128, nullptr, p, f, nullptr),
         MOE_ERR_SHAPE);
    none("rmsnorm eps nan", moe_rmsnorm_quantize_rows(h, h, NAN, 4, 128, nullptr, p, f, nullptr), MOE_ERR_SHAPE);
    none("rmsnorm null gain", moe_rmsnorm_quantize_rows(h, nullptr, 1e-6f, 4, 128, nullptr, p, f, nullptr),
         MOE_ERR_NULL);
    none("rmsnorm misaligned y", moe_rmsnorm_quantize_rows(h, h, 1e-6f, 4, 128, (uint16_t*)mis2, p, f, nullptr),
         MOE_ERR_ALIGN);
    // profiler and status strings
    double ms = 0;
    int64_t n = 0;
    CHECK(moe_profile_read(99, &ms, &n) == MOE_ERR_SHAPE, "profile kind");
    CHECK(moe_profile_read(0, nullptr, &n) == MOE_ERR_NULL, "profile null");
    CHECK(moe_profile_enable_kinds(1u << MOE_KERNEL_KINDS) == MOE_ERR_SHAPE, "profile mask");
    for (int s = -1; s <= 9; ++s) CHECK(moe_status_string(s) != nullptr, "status string %d", s);
}

// Size queries at the ends of their ranges: no overflow, zero for what the calls reject.
static void size_queries() {
    const int64_t big_n = 0x7fffffffLL;   // N*K at its largest with K = 1
    CHECK(moe_dispatch_workspace_size(big_n, 1, MOE_MAX_EXPERTS) > 0, "dispatch ws at the largest N*K");
    CHECK(moe_dispatch_workspace_size(big_n / MOE_MAX_TOPK, MOE_MAX_TOPK, MOE_MAX_EXPERTS) > 0, "dispatch ws, K max");
    CHECK(moe_dispatch_workspace_size(INT64_MAX, 8, 8) == 0, "dispatch ws, N*K past 2^31");
    CHECK(moe_dispatch_workspace_size(big_n, MOE_MAX_TOPK, 8) == 0, "dispatch ws, N*K past 2^31");
    CHECK(moe_dispatch_workspace_size(4, MOE_MAX_TOPK + 1, 100) == 0, "dispatch ws, K past the limit");
    CHECK(moe_dispatch_workspace_size(4, 2, MOE_MAX_EXPERTS + 1) == 0, "dispatch ws, E past the limit");
    CHECK(moe_swiglu_workspace_size(big_n, 1, MOE_MAX_EXPERTS, MOE_MAX_DIM, MOE_MAX_DIM) > 0, "swiglu ws at the ends");
    CHECK(moe_swiglu_workspace_size(INT64_MAX, 8, 8, 128, 128) == 0, "swiglu ws, N*K past 2^31");
    CHECK(moe_swiglu_q_workspace_size(INT64_MAX / 2, 4, 8, 128, 128) == 0, "swiglu_q ws, N*K past 2^31");
    CHECK(moe_swiglu_workspace_size(4, 2, 8, 7000, 128) == 0, "swiglu ws, d not a multiple of 128");
    CHECK(moe_swiglu_workspace_size(4, 9, 8, 128, 128) == 0, "swiglu ws, K > E");
}

// The automatic tile height against the expected rows per touched expert (K = 1 over E = 8
// experts, so N = 8 per): the measured bands -- 16 rows below 6 per expert, then 128, 224,
// 128, 192, 224 and 192 with edges at 110, 220, 262, 380 and 460 -- on both sides of each edge.
static void tile_rule() {
    struct Case {
        int64_t N;
        int rows;
    };
    const Case cases[] = {{4, 16},      {40, 16},     {48, 128},    {872, 128},   {880, 224},  {1752, 224},
                          {1760, 128},  {2088, 128},  {2096, 192},  {3032, 192},  {3040, 224}, {3672, 224},
                          {3680, 192},  {10920, 192}};
    const int32_t E = 8, d = 128, F = 128;
    for (const Case& c : cases) {
        const int64_t N = c.N;
        Buf x(N * d * 2), offsets((E + 1) * 4), sorted(N * 4), y(N * d * 2);
        Buf wg((size_t)E * F * d), wu(wg.n), wd(wg.n), sg((size_t)E * 4), su(sg.n), sd(sg.n);
        Buf ws(moe_swiglu_workspace_size(N, 1, E, d, F));
        begin();
        g_gate_up_rows = -1;
        const moe_status st = moe_grouped_swiglu(x.as<uint16_t>(), N, 1, E, d, F, offsets.as<int32_t>(),
                                                 sorted.as<int32_t>(), wg.as<uint8_t>(), sg.as<float>(),
                                                 wu.as<uint8_t>(), su.as<float>(), wd.as<uint8_t>(), sd.as<float>(),
                                                 y.as<uint16_t>(), ws.p, ws.n, 0, nullptr);
        CHECK(st == MOE_OK && g_gate_up_rows == c.rows, "N=%lld (%.1f rows per expert): %d-row tiles, want %d",
              (long long)N, N / 8.0, g_gate_up_rows, c.rows);
    }
}

int main() {
    // no device: a valid call reports the HIP error
    {
        Buf x(4 * 128 * 2), q(4 * 128), s(4 * 4);
        begin();
        const moe_status st = moe_quantize_rows(x.as<uint16_t>(), 4, 128, q.as<uint8_t>(), s.as<float>(), nullptr);
        CHECK(st == MOE_ERR_HIP && moe_last_hip_error() == hipErrorNoDevice && g_launches == 0,
              "no device -> %d (hip %d)", st, moe_last_hip_error());
        // a device that is not a gfx950
        g_device = 1;
        CHECK(moe_quantize_rows(x.as<uint16_t>(), 4, 128, q.as<uint8_t>(), s.as<float>(), nullptr) == MOE_ERR_DEVICE,
              "gfx942 device");
        g_device = 0;
    }
    error_paths();
    size_queries();
    const Shape shapes[] = {
        {64, 2, 8, 256, 128},     // the toy configuration
        {1, 8, 8, 128, 128},      // one token, every expert
        {0, 2, 8, 128, 128},      // no tokens
        {300, 3, 5, 384, 256},    // ragged tiles, a ragged down column block
        {700, 1, 5, 640, 256},    // top-1
        {4200, 2, 16, 128, 128},  // past the one-workgroup dispatch (8400 slots)
        {10, 1, 5000, 128, 128},  // more experts than the one-workgroup dispatch takes
        {3, 1, 1, 65536, 128},    // the largest hidden size
        {8192, 8, 384, 256, 128}, // 65536 sorted rows over 384 experts
        {40, 12, 16, 1536, 256},  // K = 12
    };
    for (const Shape& sh : shapes) valid_calls(sh);
    tile_rule();
    // checked dispatch reports what the device-side check found
    {
        const int64_t N = 6;
        Buf ids(N * 2 * 4), c(8 * 4), o(9 * 4), ss(N * 2 * 4), sp(N * 2 * 4), ws(moe_dispatch_workspace_size(N, 2, 8));
        memset(ids.p, 0, ids.n);
        for (int bits = 0; bits < 3; ++bits) {
            g_err_bits = bits;
            const moe_status st = moe_dispatch(ids.as<int32_t>(), N, 2, 8, c.as<int32_t>(), o.as<int32_t>(),
                                               ss.as<int32_t>(), sp.as<int32_t>(), ws.p, ws.n, MOE_FLAG_CHECKED,
                                               nullptr);
            const moe_status want = bits == 0 ? MOE_OK : bits == 1 ? MOE_ERR_BAD_ID : MOE_ERR_DUP_ID;
            CHECK(st == want, "checked dispatch bits %d -> %d", bits, st);
        }
        g_err_bits = 0;
    }
    // the profiler counts timed launches of the selected kinds
    {
        const Shape sh{16, 2, 4, 128, 128};
        CHECK(moe_profile_reset() == MOE_OK, "profile reset");
        CHECK(moe_profile_enable_kinds(1u << MOE_KERNEL_GATE_UP) == MOE_OK, "profile enable");
        valid_calls(sh);   // six tile heights: six gate|up launches with x, six more without
        double ms = 0;
        int64_t n = 0;
        CHECK(moe_profile_read(MOE_KERNEL_GATE_UP, &ms, &n) == MOE_OK && n == 12 && ms == 6.0,
              "gate|up launches timed: %lld, %.2f ms", (long long)n, ms);
        CHECK(moe_profile_read(MOE_KERNEL_DOWN, &ms, &n) == MOE_OK && n == 0, "down not timed");
        CHECK(moe_profile_enable(0) == MOE_OK && moe_profile_reset() == MOE_OK, "profile off");
    }
    printf("api host check: %d checks, %d failures\n", g_checks, g_fail);
    return g_fail ? 1 : 0;
}
