// The library's own device scratch buffer, for the entry point that allocates
// nothing (ssd_chunk_scan_fwd_noalloc).
//
// `scratch` is a file-scope device array: every GPU the library runs on holds
// its own copy, at its own address, from the first use on that device until the
// process ends.  In host code the name `scratch` is only a host-side stand-in
// for the symbol, not a device address, so host code never passes it to a
// kernel or a copy: the device address comes from hipGetSymbolAddress, looked
// up once per device (with that device current) and cached here.
//
// Every call on one GPU shares that GPU's array and finds the previous call's
// contents in it.  Nothing here needs zeroing: each use writes every scratch
// value it later reads, except the flags of a cut last round, which a wait
// accepts only at the call's own 64-bit token and which the reading workgroup
// clears.  Calls that overlap in time on one GPU (two streams, or two host
// threads) race on the array.
#include <mutex>

#include "ssd_kernels.h"

namespace ssd {
namespace {

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t scratch_for_current_device(void **ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace ssd
