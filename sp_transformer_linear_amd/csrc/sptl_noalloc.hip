// Device scratch of agmm_chunked_noalloc: the chunk-ordered GEMM's landed flags, end counters
// and error word in one file-scope device array, so the call allocates nothing.
//
// Each GPU the library runs on holds its own copy of `scratch` (80 KiB) until the process
// ends.  Host code never uses the array's name as an address: set-up (sptl_create) resolves the
// address of the current device's copy once per device with hipGetSymbolAddress, and every
// later use goes through that pointer.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <string>

#include "sptl_internal.h"
#include "sptl_noalloc.h"

namespace sptl {
namespace {
constexpr size_t kFlagWords = kFlagSetWords;                         // 64 KiB of landed flags
constexpr size_t kCountWords = (size_t)kCallCountLines * kEndLine;  // a call's counters, 256 B apart
constexpr size_t kErrWords = 32;                                     // the error word's line
constexpr size_t kScratchWords = kFlagWords + kCountWords + kErrWords;
static_assert(kScratchWords * 8 <= 80 * 1024, "scratch budget");
constexpr int kDevices = 64;

struct DeviceScratch {
    uint64_t *base = nullptr;           // this device's copy of `scratch`
    std::atomic<uint64_t> epoch{0};     // landed-flag value of the last call (flags start at 0)
};
DeviceScratch g_dev[kDevices];
std::mutex g_mu;
}  // namespace
}  // namespace sptl

static __device__ __align__(256) uint64_t scratch[sptl::kScratchWords];

namespace sptl {

int noalloc_setup(int device, std::string *err) {
    if (device < 0 || device >= kDevices) {
        *err = "device index beyond the scratch table";
        return -1;
    }
    std::lock_guard<std::mutex> lk(g_mu);
    if (g_dev[device].base) return 0;
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
        *err = std::string("hipGetSymbolAddress of the scratch array failed: ") + hipGetErrorString(e);
        return -1;
    }
    g_dev[device].base = static_cast<uint64_t *>(p);
    return 0;
}

bool noalloc_scratch(int device, NoallocScratch *out) {
    if (device < 0 || device >= kDevices) return false;
    uint64_t *b = g_dev[device].base;
    if (!b) return false;
    out->flags = b;
    out->counts = b + kFlagWords;
    out->count_words = (int64_t)kCountWords;
    out->err = reinterpret_cast<int *>(b + kFlagWords + kCountWords);
    out->flag_epoch = g_dev[device].epoch.fetch_add(1, std::memory_order_relaxed) + 1;
    return true;
}

}  // namespace sptl
