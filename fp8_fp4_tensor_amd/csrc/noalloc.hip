// noalloc.hip -- fq_quantize_noalloc: fq_quantize without a caller-provided
// workspace, for callers that cannot allocate device memory (code under HIP
// graph capture, tight serving loops, harnesses that forbid allocation).
//
// The scratch fq_quantize takes from its workspace argument -- the amax
// partials of per-tensor current scaling and NVFP4, one fp32 per workgroup of
// the amax pass, at most 1024 of them -- lives here in a file-scope device
// array instead: one copy per GPU, held until the process ends. On the host
// the array's name is only a stand-in for the device symbol, never an
// address: the device address is looked up once per device, with that device
// current, by hipGetSymbolAddress, kept, and passed to the kernels as the
// workspace pointer.
//
// Every call on one GPU shares that GPU's array, and the array keeps the
// last call's contents. Calls on one stream are ordered and safe; calls that
// overlap in time on one GPU (unordered streams, or several host threads)
// race on the array and give wrong results. Nothing needs clearing between
// calls: the amax pass writes every partial that its consumers read.
#include "fq.h"

#include <hip/hip_runtime.h>

#include <atomic>

#include "launch.hpp"

namespace {

constexpr size_t kScratchBytes = 4096;
static_assert(kScratchBytes >= fq::kPartialsBytes, "the amax partials must fit the scratch array");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];

// The device address of `scratch` on the device that runs `stream`.
fq_status scratch_address(hipStream_t stream, void** out)
{
    int cur = 0, dev = 0;
    if (hipGetDevice(&cur) != hipSuccess)
        return FQ_E_HIP;
    if (hipStreamGetDevice(stream, &dev) != hipSuccess)
        return FQ_E_HIP;
    if (dev < 0 || dev >= kMaxDevices)
        return FQ_E_UNSUPPORTED;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (p) {
        *out = p;
        return FQ_OK;
    }
    // first call on this device: look the symbol up with the device current
    if (dev != cur && hipSetDevice(dev) != hipSuccess)
        return FQ_E_HIP;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur && hipSetDevice(cur) != hipSuccess)
        return FQ_E_HIP;
    if (e != hipSuccess || !p)
        return FQ_E_HIP;
    g_scratch[dev].store(p, std::memory_order_release);
    *out = p;
    return FQ_OK;
}

}  // namespace

extern "C" fq_status fq_quantize_noalloc(const fq_desc* d, const void* x, const fq_quantized* out,
                                         hipStream_t stream)
{
    size_t need = 0;
    fq_status s = fq_sizes(d, nullptr, nullptr, nullptr, nullptr, &need);
    if (s != FQ_OK)
        return s;
    if (need > kScratchBytes)
        return FQ_E_WORKSPACE;  // more scratch than the static array holds
    void* ws = nullptr;
    if ((s = scratch_address(stream, &ws)) != FQ_OK)
        return s;
    return fq_quantize(d, x, out, ws, kScratchBytes, stream);
}
