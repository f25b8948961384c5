// scratch.hip -- the library's one static device workspace.
//
// lora_apply_noalloc serves callers that cannot allocate device memory at
// call time: its kernels take the per-call workspace (routing arrays, h parts,
// split-K partial sums) from this file-scope array instead of the pool's
// workspace.  The array's first SCRATCH_COUNTER_BYTES are the split tiles'
// counters, zeroed once here and left at 0 by every call.  Each device the library runs on holds its own copy of the array
// until the process ends.  In host code `scratch` names a host-side stand-in,
// not a device address: the device address comes from hipGetSymbolAddress,
// taken once per device with that device current, and only that address is
// ever handed to kernels.
#include <mutex>

#include "../../include/lora.h"
#include "internal.hpp"

namespace lora {

namespace {

__device__ __align__(256) char scratch[LORA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
char *g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t scratch_setup(int device) {
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_mu);
    if (g_ptr[device] != nullptr) return hipSuccess;
    void *p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    // The split counters start at 0 (the kernels leave them at 0).
    e = hipMemset(p, 0, SCRATCH_COUNTER_BYTES);
    if (e != hipSuccess) return e;
    g_ptr[device] = static_cast<char *>(p);
    return hipSuccess;
}

char *scratch_device_ptr(int device) {
    if (device < 0 || device >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lk(g_mu);
    return g_ptr[device] == nullptr ? nullptr : g_ptr[device] + SCRATCH_COUNTER_BYTES;
}

unsigned *scratch_split_counters(int device) {
    if (device < 0 || device >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lk(g_mu);
    return reinterpret_cast<unsigned *>(g_ptr[device]);
}

}  // namespace lora
