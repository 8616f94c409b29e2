// noalloc.hip -- oproj_fused_noalloc: the whole path of oproj_fused with its
// workspace (FP8 codes, scales and, with wo_b, z) in a device array that this
// library holds for the life of the process, for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops).
//
// The array is a file-scope __device__ symbol: each GPU the library runs on
// holds its own copy at its own address.  That address is looked up once per
// device, with the device current, through hipGetSymbolAddress, and only the
// looked-up pointer is ever handed to a kernel (in host code the symbol's name
// is a host-side stand-in, not a device address).
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "oproj.h"

namespace {

constexpr size_t kScratchBytes = OPROJ_NOALLOC_SCRATCH_BYTES;
static __device__ __attribute__((aligned(256))) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// This device's copy of the scratch array (device address), looked up on the
// first call made with the device current.
oproj_status scratch_on_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return OPROJ_E_HIP;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return OPROJ_E_HIP;
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return OPROJ_OK;
}

}  // namespace

extern "C" oproj_status oproj_fused_noalloc(const oproj_shape* shape, int32_t scale_mode, const void* o,
                                            const int64_t* positions, const float* cos_sin,
                                            const void* w_codes, const void* w_scales, int32_t w_block,
                                            const void* wo_b, int64_t hidden, void* out, void* stream) {
    const size_t need = oproj_fused_workspace_bytes(shape, wo_b ? hidden : 0);
    if (need == 0)  // T == 0 (a no-op) or an invalid shape: oproj_fused reports which
        return oproj_fused(shape, scale_mode, o, positions, cos_sin, w_codes, w_scales, w_block, wo_b, hidden,
                           nullptr, 0, out, stream);
    if (need > kScratchBytes) return OPROJ_E_SCRATCH;
    // the recipe checks oproj_fused makes, before the device is touched
    const bool mode_ok = scale_mode == OPROJ_SCALE_FP32 || scale_mode == OPROJ_SCALE_POW2 ||
                         scale_mode == OPROJ_SCALE_E8M0;
    const bool block_ok = w_block == OPROJ_WBLOCK_128x128 || w_block == OPROJ_WBLOCK_1x128 ||
                          (w_block == OPROJ_WBLOCK_1x128_UE8M0 && scale_mode != OPROJ_SCALE_FP32);
    if (!mode_ok || !block_ok) return OPROJ_E_MODE;
    void* ws = nullptr;
    const oproj_status st = scratch_on_current_device(&ws);
    if (st != OPROJ_OK) return st;
    return oproj_fused(shape, scale_mode, o, positions, cos_sin, w_codes, w_scales, w_block, wo_b, hidden, ws,
                       kScratchBytes, out, stream);
}
