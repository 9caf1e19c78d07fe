// The backward entry point that allocates nothing: for callers that cannot
// allocate device memory (code under stream capture, tight serving loops,
// harnesses that forbid allocation).  Every buffer a call needs beyond its
// inputs and outputs (the XCD probe words, the schedule table, the fp32 dQ
// accumulator, D and lse*log2(e), flags and counters) lives in `scratch`, a
// fixed device array of the library that each device holds for the life of
// the process.
#include <hip/hip_runtime.h>

#include <map>
#include <mutex>

#include "attn_bwd.h"
#include "internal.h"

namespace attn {

// 64 MiB: enough for b*h*s*d up to about 15.7M elements of accumulator (for
// example b=4, h=16, s=2048, d=64) together with its schedule table.
constexpr size_t kScratchBytes = 64u << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// The device address of `scratch` on each device, looked up once per device
// with that device current (the host-side name `scratch` is only a stand-in
// and must never be passed to a kernel or a copy).
static std::mutex g_scratch_mutex;
static std::map<int, char*> g_scratch_ptr;

static int scratch_address(int dev, char** out) {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    auto it = g_scratch_ptr.find(dev);
    if (it != g_scratch_ptr.end()) {
        *out = it->second;
        return ATTN_OK;
    }
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) return fail(ATTN_ERR_HIP, "hipGetSymbolAddress(scratch) failed");
    g_scratch_ptr[dev] = static_cast<char*>(ptr);
    *out = static_cast<char*>(ptr);
    return ATTN_OK;
}

}  // namespace attn

using namespace attn;

extern "C" size_t attn_bwd_noalloc_capacity(void) { return kScratchBytes; }

extern "C" int attn_bwd_deterministic_noalloc(const void* q, const void* k, const void* v, const void* o,
                                              const void* dO, const float* lse, void* dq, void* dk, void* dv,
                                              int b, int h, int s, int d, int causal, int schedule, int dtype,
                                              float scale, void* stream) {
    return guarded([&]() -> int {
        int dev = 0;
        const hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return fail(ATTN_ERR_HIP, "hipGetDevice failed");
        char* base = nullptr;
        const int rc = scratch_address(dev, &base);
        if (rc != ATTN_OK) return rc;
        const NoAllocArea na{base, kScratchBytes};
        return backward(q, k, v, o, dO, lse, dq, dk, dv, b, h, s, d, causal, schedule, dtype, scale, nullptr, 0,
                        stream, &na);
    });
}
