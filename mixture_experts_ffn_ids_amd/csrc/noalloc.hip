// moe_grouped_swiglu_noalloc: moe_grouped_swiglu with its workspace in a fixed device array of
// the library instead of a caller-provided buffer, for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The array is a file-scope __device__ variable: every GPU the library runs on holds its own
// copy, at its own address, for the life of the process. In host code the array's name is
// only a stand-in for the symbol, never a device address. Its address on a device is looked up
// once per device (hipGetSymbolAddress, with that device current, on the first call there), and
// only that address is handed to the kernels. Nothing here allocates.
//
// What the kernels keep in it (the e4m3 activations and their scales, the e4m3 product h and
// its scales, the tile list and its count) is written in full by each call before it is read,
// so nothing needs clearing between calls. Calls on one GPU share the array: calls that may
// overlap in time on one GPU (different streams without ordering) race on it.
#include <mutex>

#include "moe.h"
#include "moe_internal.h"

namespace {

constexpr size_t kScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices] = {};   // the array's device address, per device

// Device address of the array on the current device (looked up on the first call there), or
// the HIP error that prevented it.
hipError_t scratch_ptr(void** out) {
    int dev = -1;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        const hipError_t r = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (r != hipSuccess) return r;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" moe_status moe_grouped_swiglu_noalloc(const uint16_t* x, int64_t N, int32_t K, int32_t E, int32_t d,
                                                 int32_t d_ff, const int32_t* offsets, const int32_t* sorted_slot,
                                                 const uint8_t* w_gate, const float* s_gate, const uint8_t* w_up,
                                                 const float* s_up, const uint8_t* w_down, const float* s_down,
                                                 uint16_t* y_sorted, uint32_t flags, void* stream) {
    const size_t need = moe_swiglu_workspace_size(N, K, E, d, d_ff);
    if (N == 0 || need == 0)   // a no-op, or sizes the call rejects: its own status, no device work
        return moe_grouped_swiglu(x, N, K, E, d, d_ff, offsets, sorted_slot, w_gate, s_gate, w_up, s_up, w_down,
                                  s_down, y_sorted, nullptr, 0, flags, stream);
    if (need > kScratchBytes) return MOE_ERR_WORKSPACE;
    void* ws = nullptr;
    const hipError_t e = scratch_ptr(&ws);
    if (e != hipSuccess) return moe::record_hip_error(e);
    return moe_grouped_swiglu(x, N, K, E, d, d_ff, offsets, sorted_slot, w_gate, s_gate, w_up, s_up, w_down, s_down,
                              y_sorted, ws, kScratchBytes, flags, stream);
}
