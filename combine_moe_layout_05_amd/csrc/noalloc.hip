// Static device scratch for the entry point that allocates nothing
// (moe_layout_noalloc): callers that may not call hipMalloc at all (code
// under graph capture, tight serving loops, harnesses that forbid it) pass
// their inputs and outputs, and the layout's per-tile histograms live here
// instead of in a context workspace.
//
// The array exists once per device for the life of the process. In host code
// its name is only a host-side stand-in, never a device address: the device
// address is looked up once per device with hipGetSymbolAddress, with that
// device current, and only that pointer is handed to kernels. Every call on
// one device shares the array, so calls that overlap on one device race
// (callers order them on one stream). Nothing in it needs to start at zero:
// the count launch writes every histogram row the rank launch reads.
#include <mutex>

#include "moe_kernels.h"

namespace moe {
namespace {

static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];

}  // namespace

hipError_t noalloc_scratch(void** out) {
    *out = nullptr;
    int dev = -1;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess) return err;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace moe
