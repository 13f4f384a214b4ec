// ssd_combined_varlen for callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc): the same launches, with the workspace taken from a static device
// array of this library instead of a caller's buffer.
//
// The array exists once per GPU the library runs on and stays allocated until
// the process ends. Every call on one GPU uses that GPU's copy, so calls that
// overlap on one GPU (different streams, or threads) race on it; calls queued
// on one stream run one after the other and are safe. The workspace needs no
// clearing: every kernel writes what it later reads within the call.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "../../include/ssd_mi355x.h"

namespace {

constexpr size_t kScratchBytes = SSD_NOALLOC_SCRATCH_BYTES;

// The scratch array. In host code `scratch` names a host-side stand-in, not
// device memory: only the address hipGetSymbolAddress returns for the current
// device is ever passed on.
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void *g_scratch[kMaxDevices] = {};   // device address of `scratch` per device

// Device address of the current device's copy of `scratch`, looked up on the
// first call on that device (with that device current) and kept.
int scratch_of_current_device(void **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SSD_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (g_scratch[dev] == nullptr) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
            return SSD_ERR_HIP;
        g_scratch[dev] = ptr;
    }
    *out = g_scratch[dev];
    return SSD_OK;
}

}  // namespace

extern "C" {

size_t ssd_noalloc_scratch_bytes(void) { return kScratchBytes; }

int ssd_combined_varlen_noalloc(const ssd_problem *p, const void *x, const void *dt,
                                const float *A, const void *B, const void *C, const float *D,
                                const int32_t *cu_seqlens, void *state_cache,
                                const int32_t *state_indices, const uint8_t *has_initial_state,
                                void *y, void *checkpoints, void *stream)
{
    const size_t need = ssd_workspace_bytes(p);
    if (need == 0)   // an invalid problem: ssd_combined_varlen returns its status
        return ssd_combined_varlen(p, x, dt, A, B, C, D, cu_seqlens, state_cache, state_indices,
                                   has_initial_state, y, checkpoints, nullptr, 0, stream);
    if (need > kScratchBytes) return SSD_ERR_SCRATCH;
    void *ws = nullptr;
    const int rc = scratch_of_current_device(&ws);
    if (rc != SSD_OK) return rc;
    return ssd_combined_varlen(p, x, dt, A, B, C, D, cu_seqlens, state_cache, state_indices,
                               has_initial_state, y, checkpoints, ws, kScratchBytes, stream);
}

}  // extern "C"
