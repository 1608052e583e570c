// The library's one static device buffer: scratch memory for entry points
// that must not allocate (gspn_prop2d_4dir_ex_backward_noalloc).  Each GPU
// the library runs on holds its own copy of the array from module load until
// the process ends; host code reaches it only through the address that
// hipGetSymbolAddress returns for the current device.  Also here: the
// per-device CU counts that persistent grids are sized by.
#include "gspn_internal.h"

#include <mutex>

namespace gspn {
namespace {

constexpr int64_t kScratchBytes = int64_t{64} << 20;   // 64 MiB per GPU
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

// device address of `scratch` per device, looked up once per device with that
// device current (the array name in host code is a host-side stand-in, not a
// device address)
void* g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];
std::once_flag g_once[kMaxDevices];

// CUs per device, queried once per device
int g_cus[kMaxDevices];
hipError_t g_cus_err[kMaxDevices];
std::once_flag g_cus_once[kMaxDevices];

}  // namespace

int64_t noalloc_scratch_bytes() { return kScratchBytes; }

hipError_t device_cu_count(int* out) {
    int dev = 0;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::call_once(g_cus_once[dev], [dev] {
        g_cus_err[dev] = hipDeviceGetAttribute(&g_cus[dev], hipDeviceAttributeMultiprocessorCount, dev);
    });
    if (g_cus_err[dev] != hipSuccess) return g_cus_err[dev];
    *out = g_cus[dev] > 0 ? g_cus[dev] : 1;
    return hipSuccess;
}

hipError_t noalloc_scratch(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::call_once(g_once[dev], [dev] {
        void* p = nullptr;
        g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_ptr[dev] = p;
    });
    if (g_err[dev] != hipSuccess) return g_err[dev];
    *out = g_ptr[dev];
    return hipSuccess;
}

}  // namespace gspn
