// The chunked prefill of launches in which every walk is a single chunk (all
// sequences at most C rows), in a translation unit of its own so that the
// kernels of kda_prefill.hip keep their place in that file's module.
//
// Such a walk is a short chain (state in, one chunk, state out) with nothing
// to hand on between chunks, so a workgroup takes a whole head (walk1_split):
// the head's operand block is read once, not once per 16 value columns.
//   fwd_split_one_chunk  the forward pass alone, over operand blocks that a
//                        prepare launch wrote;
//   prefill_one_chunk    prepare and walk of each (sequence, head) in one
//                        workgroup: the operand block is written and read
//                        back by the same workgroup right away, instead of
//                        being written by one launch and fetched again by the
//                        next.
// Both run the products of the two-launch path in the same order, so every
// core row and state is the same bits.
#include "kda_prefill_kernels.hpp"

namespace kda {

template <int D, int C>
__global__ __launch_bounds__(C / 16 * 64) __attribute__((amdgpu_waves_per_eu(2))) void kda_chunk_walk1_kernel(
    const float *__restrict__ ws, float *__restrict__ state, float *__restrict__ core, int T,
    int H, float scale, const Varlen vl)
{
    using B = Blk<D, C>;
    const int h = blockIdx.x;
    if (vl.cu) {   // the blockIdx.y-th sequence of the segment, one chunk long
        int s;
        SeqSpan sp;
        if (!walker_span<C>(vl, blockIdx.y, s, sp) || sp.nch != 1 || sp.chunk0 < vl.seg_lo)
            return;   // uniform over the workgroup
        state = vl.states[s];
        core += sp.row0 * H * D;
        ws += (sp.chunk0 - vl.seg_lo) * H * B::kSize;
        T = sp.T;
    }
    __shared__ Walk1Lds<D, C> L;
    walk1_split<D, C>(ws + (int64_t)h * B::kSize, state + (int64_t)h * D * D, core, T, H, scale, h,
                      (int)threadIdx.x, L);
}

template <int D, int C>
__global__ __launch_bounds__(C / 16 * 64) __attribute__((amdgpu_waves_per_eu(2))) void kda_chunk_fused1_kernel(
    QkvSrc<false> src, const float *__restrict__ gate, const float *__restrict__ beta, int H,
    float *__restrict__ ws, float *__restrict__ core, float scale, const Varlen vl)
{
    using B = Blk<D, C>;
    // one workgroup per (head, walked sequence): every walked sequence is one
    // chunk, prepared and walked here
    const int h = blockIdx.x;
    if (vl.plan == nullptr && blockIdx.x == 0 && blockIdx.y == 0)
        wave_report(vl, wave_seq<C>(vl), true);
    int s;
    SeqSpan sp;
    if (!walker_span<C>(vl, blockIdx.y, s, sp) || sp.nch != 1 || sp.chunk0 < vl.seg_lo)
        return;   // uniform over the workgroup
    src.advance(sp.row0);
    float *blk = ws + ((sp.chunk0 - vl.seg_lo) * H + h) * B::kSize;
    __shared__ union {
        PrepSplitLds<D, C> prep;
        Walk1Lds<D, C> walk;
    } L;
    // W and U' stay in the prepare's LDS; the rest of the block goes through
    // the workspace (written, then read back by this workgroup)
    prep_split_unit<D, C, false, true>(src, gate + sp.row0 * H * D, beta + sp.row0 * H, sp.T, H,
                                       blk, 0, h, vl.rows - 1 - sp.row0, (int)threadIdx.x, L.prep);
    // the block's global stores and W and U' in LDS visible to every wave of
    // the workgroup
    __syncthreads();
    walk1_split<D, C, true>(blk, vl.states[s] + (int64_t)h * D * D, core + sp.row0 * H * D, sp.T, H,
                            scale, h, (int)threadIdx.x, L.walk, &L.prep.s_M[0][0], L.prep.s_xbuf);
}

template <int D, int C>
hipError_t fwd_split_one_chunk(dim3 grid, const float *ws, float *state, float *core, int T,
                               int NC, int H, float scale, const Varlen &vl, hipStream_t stream)
{
    // Few (sequence, head) pairs keep the 16-column workgroups, which spread
    // the heads over more CUs; many take a whole head per workgroup.
    if ((int64_t)H * grid.y >= 256)
        hipLaunchKernelGGL((kda_chunk_walk1_kernel<D, C>), dim3(H, grid.y), dim3(PrefCfg<D, C>::kThreads),
                           0, stream, ws, state, core, T, H, scale, vl);
    else
        hipLaunchKernelGGL((kda_chunk_fwd_split_kernel<D, C, false>), grid,
                           dim3(2 * PrefCfg<D, C>::kThreads), 0, stream, ws, state, core, T, NC,
                           H, scale, vl);
    return hipGetLastError();
}

template <int D, int C>
hipError_t prefill_one_chunk(const float *q, const float *k, const float *v, const float *gate,
                             const float *beta, float *core, int H, float scale, void *workspace,
                             const Varlen &vl, hipStream_t stream)
{
    const QkvSrc<false> src{q, k, v, (int64_t)H * D};
    hipLaunchKernelGGL((kda_chunk_fused1_kernel<D, C>), dim3(H, std::min(vl.B, vl.seg_hi - vl.seg_lo)),
                       dim3(PrefCfg<D, C>::kThreads),
                       0, stream, src, gate, beta, H, static_cast<float *>(workspace), core, scale,
                       vl);
    return hipGetLastError();
}

template hipError_t fwd_split_one_chunk<128, 64>(dim3, const float *, float *, float *, int, int,
                                                 int, float, const Varlen &, hipStream_t);
template hipError_t prefill_one_chunk<128, 64>(const float *, const float *, const float *,
                                               const float *, const float *, float *, int, float,
                                               void *, const Varlen &, hipStream_t);

}  // namespace kda
