// gdn_static.hip -- the scratch memory of gdn_tree_verify_static: a file-scope
// array in device memory that holds the plan's metadata (verdicts, depths,
// root-to-node paths, preorder) between the plan kernel and the verify kernels
// of one call, for callers that cannot allocate.  Each GPU the library runs on
// holds its own copy of the array until the process ends.
#include <mutex>

#include "gdn_internal.h"

namespace gdn {
constexpr size_t kStaticScratchBytes = size_t(32) << 20;  // 32 MiB per GPU
}  // namespace gdn

// In host code this name is only a stand-in for the device array, never an
// address: host code uses the per-device address that hipGetSymbolAddress
// returns (static_scratch below) and passes that to the kernels.
static __device__ __align__(256) unsigned char scratch[gdn::kStaticScratchBytes];

namespace gdn {
namespace {

constexpr int kScratchDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kScratchDevices];  // device address of `scratch` on each GPU

}  // namespace

size_t static_scratch_bytes() { return kStaticScratchBytes; }

// This GPU's address of `scratch`, looked up once per device, with that device
// current (the first call on each device does the lookup).
hipError_t static_scratch(void **out) {
    *out = nullptr;
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace gdn
