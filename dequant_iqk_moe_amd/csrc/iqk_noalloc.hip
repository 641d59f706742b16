// iqk_noalloc.hip -- the routed projection for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, hosts
// that forbid allocation): iqk_moe_auto with its scratch (the routing
// arrays and the work plan of the grouped matvec and the fused prefill) in
// a fixed device array of this library instead of a caller's workspace.
//
// The array lives in the library's code object: each GPU the library runs
// on holds its own copy until the process ends, at its own address.  Host
// code takes that address once per device (hipGetSymbolAddress with the
// device current) and passes it to the kernels; the array's name itself is
// only a host-side stand-in and is never handed to a kernel or a copy.
#include <mutex>

#include "iqk_internal.h"
#include "iqk_status.h"

namespace {

constexpr size_t kScratchBytes = size_t(1) << 20;  // the most scratch one call may use
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};  // device address of `scratch` on each device

// The current device's copy of the scratch array (taken on the first call
// on that device), or null with the HIP error in *err.
void* device_scratch(hipError_t* err) {
    int dev = -1;
    *err = hipGetDevice(&dev);
    if (*err != hipSuccess) return nullptr;
    if (dev < 0 || dev >= kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (*err != hipSuccess) return nullptr;
        g_scratch[dev] = p;
    }
    return g_scratch[dev];
}

}  // namespace

extern "C" int iqk_moe_auto_noalloc(const iqk_weights* w, const float* values, const int8_t* grid, const void* x,
                                    int x_dtype, int x_slots, const int32_t* ids, int64_t T, int k, float* y,
                                    int* path, void* stream) {
    size_t need = 0;
    int rc = iqk_moe_auto_workspace(w, T, k, &need);
    if (rc) return rc;
    if (need > kScratchBytes)
        return iqk::fail(IQK_E_SIZE,
                         "this call needs %zu bytes of scratch; the allocation-free entry point holds %zu "
                         "(fewer token-expert pairs or experts per call)",
                         need, kScratchBytes);
    hipError_t e = hipSuccess;
    void* ws = device_scratch(&e);
    if (!ws) return iqk::fail(IQK_E_HIP, "scratch address: %s", hipGetErrorString(e));
    // every kernel of the path writes the scratch before reading it (counts,
    // offsets, permutation and plan are rebuilt by each call): nothing to clear
    return iqk_moe_auto(w, values, grid, x, x_dtype, x_slots, ids, T, k, ws, kScratchBytes, y, path, stream);
}
