// The one-chunk forward instance of the chunked prefill (every walk of the
// launch is a single chunk: all sequences at most C rows), in a translation
// unit of its own.  The same products in the same order as the load-ahead
// instance, so the same bits.
#include "kda_prefill_kernels.hpp"

namespace kda {

template <int D, int C>
hipError_t fwd_split_one_chunk(dim3 grid, const float *ws, float *state, float *core, int T,
                               int NC, int H, float scale, const Varlen &vl, hipStream_t stream)
{
    hipLaunchKernelGGL((kda_chunk_fwd_split_kernel<D, C, false>), grid,
                       dim3(2 * PrefCfg<D, C>::kThreads), 0, stream, ws, state, core, T, NC, H,
                       scale, vl);
    return hipGetLastError();
}

template hipError_t fwd_split_one_chunk<128, 64>(dim3, const float *, float *, float *, int, int,
                                                 int, float, const Varlen &, hipStream_t);

}  // namespace kda
