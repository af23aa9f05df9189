// Allocation-free prefill: ssd_chunked_scan with its workspace in a
// file-scope device array, for callers that cannot allocate device memory
// (code under stream capture, serving loops, harnesses that forbid it).
//
// Each device the library runs on holds one copy of `scratch` for the life
// of the process.  Its address on a device is taken once, on the first call
// with that device current, and kept per device; the kernels get that
// address, never the host-side name of the array.  Every call on a device
// shares its copy, so calls that overlap on one device (two host threads, or
// two streams without ordering between them) race.  Nothing in the array
// needs to start at zero: the prefill writes every workspace element it
// reads before reading it.
#include <atomic>

#include <hip/hip_runtime.h>

#include "ssd.h"
#include "ssd_internal.h"

#define SSD_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr size_t kScratchBytes = SSD_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::atomic<void*> g_scratch[kMaxDevices];

// The device address of this device's copy of `scratch` (looked up once per
// device; a concurrent first lookup by two threads stores the same address).
ssd_status scratch_on_current_device(void** out, int* dev_out) {
    int dev = -1;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0)
        return (ssd_status)ssd::set_error_detail(SSD_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    *dev_out = dev;
    if (dev >= kMaxDevices)
        return (ssd_status)ssd::set_error_detail(SSD_ERR_UNSUPPORTED, "device %d: at most %d devices", dev,
                                                 kMaxDevices);
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        const hipError_t g = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (g != hipSuccess || !p)
            return (ssd_status)ssd::set_error_detail(SSD_ERR_HIP, "hipGetSymbolAddress(scratch) failed: %s",
                                                     hipGetErrorString(g));
        g_scratch[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return SSD_OK;
}

}  // namespace

SSD_API ssd_status ssd_chunked_scan_noalloc(const void* x, const float* dt, const float* A, const void* B,
                                            const void* C, const float* D, int32_t chunk, const float* init_state,
                                            void* y, float* final_state, const ssd_shape* shape, void* stream) {
    size_t need = 0;
    // validates the shape and chunk as ssd_chunked_scan does
    ssd_status st = ssd_chunked_scan_workspace_size(shape, chunk, &need);
    if (st != SSD_OK) return st;
    if (need > kScratchBytes)
        return (ssd_status)ssd::set_error_detail(SSD_ERR_WORKSPACE,
                                                 "this shape needs %zu bytes of workspace; the static array holds %zu",
                                                 need, kScratchBytes);
    void* ws = nullptr;
    int dev = -1;
    st = scratch_on_current_device(&ws, &dev);
    if (st != SSD_OK) return st;
    return ssd_chunked_scan(x, dt, A, B, C, D, chunk, init_state, y, final_state, shape, ws, kScratchBytes, stream);
}
