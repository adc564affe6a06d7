// kda_prefill for callers that cannot allocate: the operand-block workspace
// lives in a file-scope device array instead of a caller buffer.
//
// The array is `scratch` below, kNoallocScratchBytes per GPU (held from the
// moment the library's code is loaded on that GPU until the process ends).
// In host code its name stands for a host-side shadow, not a device address,
// so its device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and kept; every launch
// takes that address.  Calls on one GPU share its array: calls whose work
// overlaps in time (different streams, or host threads without ordering
// between them) race on it, so the caller orders them.  Nothing in the array
// needs to start at zero: each segment's blocks are written by the prepare
// launch before the walk launch reads them.
#include <algorithm>
#include <mutex>

#include "kda_launch.hpp"

namespace kda {

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
void *g_scratch_ptr[kMaxDevices] = {};
std::mutex g_scratch_mu;

// Device address of this device's scratch array (looked up on the first
// call on the device); nullptr with *err set when the lookup fails.
void *scratch_ptr(hipError_t *err)
{
    int dev = 0;
    *err = hipGetDevice(&dev);
    if (*err != hipSuccess) return nullptr;
    if (dev < 0 || dev >= kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void *p = nullptr;
        *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (*err != hipSuccess) return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

hipError_t launch_kda_prefill_noalloc(const float *q, const float *k, const float *v,
                                      const float *gate, const float *beta, float *state,
                                      float *core, int T, int heads, int head_dim, int chunk,
                                      float scale, hipStream_t stream)
{
    // as many chunks per segment as the array holds, never more than the
    // cache-sized segments of kda_prefill; the chunk boundaries, and so the
    // bits, are the same for every segment length
    const size_t per_chunk = prefill_workspace_bytes(chunk, heads, head_dim, chunk);
    if (per_chunk == 0 || per_chunk > kNoallocScratchBytes) return hipErrorInvalidValue;
    const int fit = (int)std::min<size_t>(kNoallocScratchBytes / per_chunk, 1 << 30);
    const int seg = std::min(fit, prefill_segment_chunks(T, heads, head_dim, chunk));
    hipError_t e = hipSuccess;
    void *ws = scratch_ptr(&e);
    if (ws == nullptr) return e;
    return launch_kda_prefill_segments(q, k, v, gate, beta, state, core, T, heads, head_dim, chunk,
                                       scale, ws, seg, stream);
}

}  // namespace kda
