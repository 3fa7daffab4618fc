// kda_chunk_fwd_noalloc: kda_chunk_fwd with the workspace taken from a fixed scratch array that
// the library owns, for callers that cannot allocate device memory (code under stream capture,
// tight serving loops, harnesses that forbid allocation). See include/kda.h for the contract.
//
// The array is a file-scope __device__ symbol: each device the library runs on holds its own copy
// (allocated when this file's code object is loaded on that device) until the process ends. Host
// code never uses the symbol's name as an address: the device address of each device's copy is
// looked up once per device with hipGetSymbolAddress, with that device current, and kept here.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kda.h"
#include "kda_internal.h"
#include "kda_plan.h"

namespace {

static __device__ __align__(256) unsigned char scratch[KDA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices];
std::once_flag g_once[kMaxDevices];
hipError_t g_status[kMaxDevices];

// Device address of `dev`'s copy of the scratch array, or NULL if the lookup failed.
void* scratch_of(int dev) {
    if (dev < 0 || dev >= kMaxDevices) return nullptr;
    std::call_once(g_once[dev], [dev] {
        int cur = 0;
        hipError_t e = hipGetDevice(&cur);
        if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
        void* ptr = nullptr;
        if (e == hipSuccess) e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (cur != dev) (void)hipSetDevice(cur);
        g_status[dev] = e;
        g_scratch[dev] = e == hipSuccess ? ptr : nullptr;
    });
    return g_scratch[dev];
}

}  // namespace

extern "C" kda_status kda_chunk_fwd_noalloc(const kda_chunk_desc* desc, const void* q, const void* k,
                                            const void* v, const void* log_alpha, const void* beta,
                                            const float* S0, void* o, float* S_T, void* stream) {
    return kda::chunk_fwd_impl(desc, q, k, v, log_alpha, beta, S0, o, S_T, nullptr, 0, stream, scratch_of);
}
