// bs_noalloc.hip -- bs_build_tables_noalloc: the per-tensor model from words
// in device memory, with no memory allocated by the call, for callers that
// cannot allocate (harnesses that forbid hipMalloc, serving loops that must
// not touch the allocator).
//
// The histogram's counters live in `scratch`, a file-scope device array that
// every GPU the library runs on holds for the life of the process.  Its
// device address comes from hipGetSymbolAddress, once per device with that
// device current; host code uses only that address, never the array's name
// (which in host code is a host-side stand-in, not a device address).  The
// counts are read back into a host array of the same size in static storage.
// One host lock covers a whole call, from clearing the counters to reading
// them back, so calls in one process do not overlap; the device array keeps
// the last call's counts.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <array>
#include <mutex>

#include "bs.h"
#include "bs_device.h"
#include "bs_encode_device.h"
#include "bs_internal.h"
#include "bs_model.h"

using namespace bs;

namespace {

constexpr uint64_t kScratchBytes = kHistCounters * sizeof(unsigned long long);   // 278,528 B
static __device__ __align__(256) unsigned long long scratch[kHistCounters];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void* g_scratch[kMaxDevices];      // device address of `scratch` on each device (under g_lock)
unsigned long long g_counts[kHistCounters];       // host copy of the counters (under g_lock)
std::array<uint64_t, 128> g_merged[kCandidates];  // model working memory (under g_lock)
uint64_t g_joint[512 * 8];                         // joint counts of layout 3 (under g_lock)

// the address of this device's copy of `scratch`, looked up on first use
bs_status scratch_of(int dev, void** out) {
    if (dev < 0 || dev >= kMaxDevices) { set_error("device %d: at most %d devices", dev, kMaxDevices); return BS_E_INVAL; }
    if (!g_scratch[dev]) {
        void* ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) {
            set_error("hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
            return BS_E_HIP;
        }
        g_scratch[dev] = ptr;
    }
    *out = g_scratch[dev];
    return BS_OK;
}

}  // namespace

extern "C" {

bs_status bs_build_tables_noalloc(const void* d_bf16, uint64_t n, const bs_params* p, void* stream, bs_tables* t) {
    if (!t || (!d_bf16 && n) || !params_ok(p)) {
        if (!t || (!d_bf16 && n)) set_error("NULL argument");
        return BS_E_INVAL;
    }
    if (n > BS_NOALLOC_MAX_WEIGHTS) {
        set_error("bs_build_tables_noalloc: %llu words, more than its maximum of %llu (2^36)", (unsigned long long)n,
                  (unsigned long long)BS_NOALLOC_MAX_WEIGHTS);
        return BS_E_INVAL;
    }
    std::lock_guard<std::mutex> hold(g_lock);
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) { set_error("hipGetDevice: %s", hipGetErrorString(e)); return BS_E_HIP; }
    void* d_cnt = nullptr;
    bs_status rc = scratch_of(dev, &d_cnt);
    if (rc != BS_OK) return rc;
    unsigned long long* cnt = (unsigned long long*)d_cnt;
    hipStream_t s = (hipStream_t)stream;
    if (n) {
        // cleared by a kernel (bsk_zero), not a memset node
        e = (hipError_t)bsk_zero(cnt, kScratchBytes, stream);
        if (e == hipSuccess) e = (hipError_t)bsk_hist((const uint16_t*)d_bf16, n, cnt, cnt + 256 * 128, stream);
        if (e == hipSuccess) e = hipMemcpyAsync(g_counts, cnt, kScratchBytes, hipMemcpyDeviceToHost, s);
        if (e == hipSuccess) e = hipStreamSynchronize(s);
        if (e != hipSuccess) { set_error("histogram: %s", hipGetErrorString(e)); return BS_E_HIP; }
    }
    return model_from_counts(*t, p, n, g_counts, g_merged, g_joint);
}

}  // extern "C"
