// Decode workspace for callers that cannot allocate device memory (code under
// HIP graph capture, serving loops that forbid hipMalloc): a file-scope
// device array that every GPU the library runs on holds from module load
// until the process ends.
//
// Host code never passes the array's name to a kernel or a copy: in host code
// that name is a host-side stand-in, not a device address.  The device
// address is looked up once per device with hipGetSymbolAddress (with that
// device current) and kept; kernels receive that pointer as their workspace.
#include <cstdint>
#include <mutex>

#include <hip/hip_runtime.h>

#include "fp4kv_internal.h"

namespace fp4kv {
namespace {

constexpr int kMaxDevices = 64;

__device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices];     // device address of `scratch`, per device (null: not looked up yet)

}  // namespace

hipError_t scratch_for_current_device(void **out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        if (!p)
            return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace fp4kv
