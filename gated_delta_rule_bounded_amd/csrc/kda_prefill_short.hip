// The one-chunk forward instance of the chunked prefill (every walk of the
// launch is a single chunk: all sequences at most C rows), in a translation
// unit of its own.  The same products in the same order as the load-ahead
// instance, so the same bits.
//
// Such a walk is a short latency chain (state in, one chunk, state out).
// With many (sequence, head) pairs in the launch, what it costs is the head's
// operand block being pulled into every workgroup that walks part of the
// head, so a workgroup then takes all D / 16 column tiles of its head (the
// whole state; the block is read once per head and sequence instead of once
// per 16 columns), one workgroup per CU.  Fewer pairs than CUs keep the
// 16-column workgroups, which spread the few heads over more CUs.
#include "kda_prefill_kernels.hpp"

namespace kda {

template <int D, int C>
hipError_t fwd_split_one_chunk(dim3 grid, const float *ws, float *state, float *core, int T,
                               int NC, int H, float scale, const Varlen &vl, hipStream_t stream)
{
    constexpr int NJ = D / 16;
    if ((int64_t)H * grid.y >= 256)
        hipLaunchKernelGGL((kda_chunk_fwd_split_kernel<D, C, false, NJ>), dim3(H, grid.y),
                           dim3(2 * PrefCfg<D, C>::kThreads), 0, stream, ws, state, core, T, NC,
                           H, scale, vl);
    else
        hipLaunchKernelGGL((kda_chunk_fwd_split_kernel<D, C, false>), grid,
                           dim3(2 * PrefCfg<D, C>::kThreads), 0, stream, ws, state, core, T, NC,
                           H, scale, vl);
    return hipGetLastError();
}

template hipError_t fwd_split_one_chunk<128, 64>(dim3, const float *, float *, float *, int, int,
                                                 int, float, const Varlen &, hipStream_t);

}  // namespace kda
