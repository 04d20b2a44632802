// The static device scratch behind kda_fwd_noalloc: the forward's schedule
// (task order, sequence offsets, segment list) lives in a file-scope device
// array instead of library-allocated memory, so that the call allocates
// nothing.  One copy per device, held until the process ends; every
// kda_fwd_noalloc call on a device overwrites it, so calls that overlap on one
// device (other streams, other threads) race.
#include <hip/hip_runtime.h>

#include <cstring>
#include <map>
#include <mutex>

#include "../../include/libkda.h"
#include "kda_kernels.h"

// The scratch array itself (file scope, one copy per device).
static __device__ __align__(256) unsigned char scratch[KDA_NOALLOC_SCRATCH_BYTES];

namespace kda {

namespace {

// Data words per upload launch: the kernel argument block stays under 4 KiB.
constexpr unsigned kUploadWords = 960;

struct UploadBlock {
    unsigned offset;  // bytes into the scratch
    unsigned words;   // 32-bit words to store (<= kUploadWords)
    unsigned data[kUploadWords];
};

__global__ __launch_bounds__(256) void upload_kernel(unsigned char* base, UploadBlock b) {
    unsigned* dst = reinterpret_cast<unsigned*>(base + b.offset);
    for (unsigned i = threadIdx.x; i < b.words; i += blockDim.x) dst[i] = b.data[i];
}

std::mutex g_mu;
std::map<int, void*> g_addr;  // device -> address of its scratch copy

}  // namespace

hipError_t noalloc_scratch(int dev, void** ptr) {
    std::lock_guard<std::mutex> lock(g_mu);
    auto it = g_addr.find(dev);
    if (it != g_addr.end()) {
        *ptr = it->second;
        return hipSuccess;
    }
    // the caller made `dev` current; in host code the array's name is only a
    // handle, the device address comes from the runtime
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_addr[dev] = p;
    *ptr = p;
    return hipSuccess;
}

hipError_t upload_to_scratch(void* dst, const void* host, size_t bytes, hipStream_t s) {
    if (bytes % 4 != 0 || bytes > (size_t)KDA_NOALLOC_SCRATCH_BYTES) return hipErrorInvalidValue;
    const unsigned* src = static_cast<const unsigned*>(host);
    const size_t words = bytes / 4;
    UploadBlock b;
    for (size_t w = 0; w < words; w += kUploadWords) {
        b.offset = (unsigned)(w * 4);
        b.words = (unsigned)(words - w < kUploadWords ? words - w : kUploadWords);
        std::memcpy(b.data, src + w, b.words * 4);
        hipLaunchKernelGGL(upload_kernel, dim3(1), dim3(256), 0, s, static_cast<unsigned char*>(dst), b);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace kda
