// Device scratch of the weight gradient's entry point that allocates nothing
// (conv_bwd_dw_noalloc): the fp32 partials that conv_bwd_dw keeps in the
// caller's workspace live here instead, in a fixed array that every device
// the library runs on holds for the life of the process.
//
// In host code the array's name is only a stand-in for the device symbol, so
// its device address is looked up once per device (hipGetSymbolAddress, with
// that device current) and that address is what kernels receive.  Every call
// on a device shares the array: calls that overlap on one device race.
#include "kernels.hpp"

#include <atomic>

namespace convmi {

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
}  // namespace

hipError_t scratch_buffer(void** out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return hipSuccess;
}

}  // namespace convmi
