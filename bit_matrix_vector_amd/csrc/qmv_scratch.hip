// Library-held device scratch for the entry points that allocate nothing.
//
// One file-scope device array, of a fixed size, that every GPU the library
// runs on holds until the process ends. Host code never passes the array's
// name to a kernel (on the host that name is a stand-in, not a device
// address): the first request on a device, with that device current, asks the
// runtime for the array's address on that device, and every later request on
// the device returns the recorded address. Each device has its own copy at its
// own address.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <mutex>

#include "qmv_common.h"

namespace qmv {
namespace {

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kScratchDevices = 64;
void* g_scratch_ptr[kScratchDevices];

std::mutex& scratch_mutex() {
    static std::mutex m;
    return m;
}

}  // namespace

int scratch_for_current_device(void** out) {
    int d = 0;
    if (const hipError_t e = hipGetDevice(&d); e != hipSuccess) return (int)e;
    if (d < 0 || d >= kScratchDevices) return (int)hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(scratch_mutex());
    if (g_scratch_ptr[d] == nullptr) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return (int)e;
        if (p == nullptr) return (int)hipErrorInvalidSymbol;
        g_scratch_ptr[d] = p;
    }
    *out = g_scratch_ptr[d];
    return 0;
}

}  // namespace qmv
