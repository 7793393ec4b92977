// Static device scratch of qgemm_w4a16_noalloc, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation).
//
// `scratch` is a file-scope device array of QG_NOALLOC_SCRATCH_BYTES bytes:
// every GPU the library runs on holds its own copy, at its own address, until
// the process ends.  In host code the array's name is only a host-side
// stand-in, so its device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and kept; host code then
// uses that address and never the name.  The first call on a device also
// clears the scratch's split-K counter region with a fill kernel on the
// call's stream (no memset node, so the call stays safe to capture in a
// graph); every W4A16 call leaves those counters at zero again.  All calls on
// one GPU share the one array, which keeps the last call's contents: calls
// that overlap in time on one GPU race.
#include "qgemm.h"
#include "qg_launch.h"

#include <mutex>

namespace qg {

static __device__ __align__(256) unsigned char scratch[QG_NOALLOC_SCRATCH_BYTES];

__global__ __launch_bounds__(256) void zero_words_kernel(unsigned *__restrict__ p, unsigned n)
{
    const unsigned i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0u;
}

hipError_t noalloc_scratch(hipStream_t st, void **out)
{
    static_assert(QG_NOALLOC_SCRATCH_BYTES >= W4A16_WS_COUNTER_BYTES, "counter region fits");
    constexpr int MAX_DEVICES = 64;
    static std::mutex mu;
    static void *addr[MAX_DEVICES];
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        const unsigned words = (unsigned)(W4A16_WS_COUNTER_BYTES / sizeof(unsigned));
        hipLaunchKernelGGL(zero_words_kernel, dim3((words + 255) / 256), dim3(256), 0, st,
                           static_cast<unsigned *>(p), words);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        addr[dev] = p;
    }
    *out = addr[dev];
    return hipSuccess;
}

} // namespace qg
