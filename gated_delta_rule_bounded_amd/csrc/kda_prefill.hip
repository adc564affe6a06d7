// Host side of the chunked KDA prefill: workspace sizing, the segment loop and
// the launches of the kernels in kda_prefill_kernels.hpp.
#include "kda_prefill_kernels.hpp"

namespace kda {

size_t prefill_workspace_bytes(int T_pad, int heads, int head_dim, int chunk)
{
    // one operand block per (chunk, head): 4*C*D + C*C + D fp32
    const size_t blk = 4 * (size_t)chunk * head_dim + (size_t)chunk * chunk + head_dim;
    return (size_t)(T_pad / chunk) * heads * blk * sizeof(float);
}

int prefill_segment_chunks(int T, int heads, int head_dim, int chunk)
{
    constexpr size_t kCacheBudget = size_t(160) << 20;   // of MI355X's 256 MiB last-level cache
    const int NC = std::max(1, (T + chunk - 1) / chunk);
    const size_t per_chunk = prefill_workspace_bytes(chunk, heads, head_dim, chunk);
    const int nseg = (int)std::max<size_t>(1, (NC * per_chunk + kCacheBudget - 1) / kCacheBudget);
    return (NC + nseg - 1) / nseg;
}

constexpr int kMaxChunksPerLaunch = 65535;   // grid y

template <int D, int C, bool BF>
static hipError_t prepare_src(const QkvSrc<BF> &src, const float *gate, const float *beta, int T,
                              int H, void *workspace, const Varlen &vl, int B, hipStream_t stream)
{
    const dim3 grid = vl.cu ? dim3(vl.max_chunks, H, B) : dim3((T + C - 1) / C, H);
    // the split kernel takes the chunks in y (heads fastest); the callers
    // launch at most kMaxChunksPerLaunch chunks at a time
    const dim3 grid_split = vl.cu ? dim3(H, vl.max_chunks, B) : dim3(H, (T + C - 1) / C);
    if constexpr (Blk<D, C>::kSplit)
        hipLaunchKernelGGL((kda_chunk_prep_split_kernel<D, C, BF>), grid_split,
                           dim3(PrefCfg<D, C>::kThreads), 0, stream, src, gate, beta, T, H,
                           static_cast<float *>(workspace), vl);
    else
        hipLaunchKernelGGL((kda_chunk_prep_kernel<D, C, BF>), grid,
                           dim3(PrefCfg<D, C>::kThreads), 0, stream, src, gate, beta, T, H,
                           static_cast<float *>(workspace), vl);
    return hipGetLastError();
}

template <int D, int C>
static hipError_t prepare_t(const float *q, const float *k, const float *v, const float *gate,
                            const float *beta, int T, int H, void *workspace, const Varlen &vl,
                            int B, hipStream_t stream)
{
    const QkvSrc<false> src{q, k, v, (int64_t)H * D};
    return prepare_src<D, C, false>(src, gate, beta, T, H, workspace, vl, B, stream);
}

// q | k | v read from bf16 rows (row stride ldqkv elements)
template <int D, int C>
static hipError_t prepare_bf16_t(const uint16_t *qkv, int64_t ldqkv, const float *gate,
                                 const float *beta, int T, int H, void *workspace,
                                 hipStream_t stream)
{
    const int64_t qw = (int64_t)H * D;
    const QkvSrc<true> src{qkv, qkv + qw, qkv + 2 * qw, ldqkv};
    return prepare_src<D, C, true>(src, gate, beta, T, H, workspace, Varlen{}, 1, stream);
}

template <int D, int C>
static hipError_t forward_t(float *state, float *core, int T, int H, float scale,
                            const void *workspace, const Varlen &vl, int B, hipStream_t stream)
{
    const int NC = (T + C - 1) / C;
    const dim3 grid(H * PrefCfg<D, C>::kDT, vl.cu ? B : 1);
    // every walk one chunk (sequences longer than max_chunks are skipped by
    // the kernels): the instance without the load-ahead register set
    const bool one = vl.cu ? vl.max_chunks <= 1 : NC <= 1;
    if constexpr (Blk<D, C>::kSplit) {
        if (!one) {
            // Several sequences: a workgroup may take NJ column tiles of its
            // head (the head's operand block read once for all of them; the
            // same bits for any NJ).  Per chunk a workgroup's time is set by
            // the block it reads, so fewer, wider workgroups finish a
            // segment's walks in fewer rounds, as long as they still cover
            // the CUs: the widest NJ of 1, 2, 4 that launches at least 256
            // workgroups for the sequences a segment holds (estimated from the
            // mean chunks per sequence).  Measured at 4096 tokens, 32 heads:
            // 8 x 512 tokens 231 -> 188 us, 16 x 256 257 -> 202 us, 4 x 1024
            // 216 -> 189 us (NJ = 2), 2 x 2048 best at NJ = 1.
            int nj = 1;
            if (vl.cu) {
                const int64_t seg = vl.seg_hi - vl.seg_lo;
                const int64_t seqs = std::max<int64_t>(
                    1, std::min<int64_t>(B, (int64_t)B * seg / std::max(1, vl.total_chunks)));
                const int64_t tiles = seqs * H * PrefCfg<D, C>::kDT;
                for (int c = 4; c > 1 && nj == 1; c /= 2)
                    if (PrefCfg<D, C>::kDT % c == 0 && tiles / c >= 256) nj = c;
            }
            const dim3 g(H * PrefCfg<D, C>::kDT / nj, grid.y);
            const dim3 blk(2 * PrefCfg<D, C>::kThreads);
            const float *ws = static_cast<const float *>(workspace);
            if constexpr (PrefCfg<D, C>::kDT % 4 == 0) {
                if (nj == 4) {
                    hipLaunchKernelGGL((kda_chunk_fwd_split_kernel<D, C, true, 4>), g, blk, 0, stream,
                                       ws, state, core, T, NC, H, scale, vl);
                    return hipGetLastError();
                }
            }
            if constexpr (PrefCfg<D, C>::kDT % 2 == 0) {
                if (nj == 2) {
                    hipLaunchKernelGGL((kda_chunk_fwd_split_kernel<D, C, true, 2>), g, blk, 0, stream,
                                       ws, state, core, T, NC, H, scale, vl);
                    return hipGetLastError();
                }
            }
            hipLaunchKernelGGL((kda_chunk_fwd_split_kernel<D, C, true>), g, blk, 0, stream, ws,
                               state, core, T, NC, H, scale, vl);
            return hipGetLastError();
        }
        return fwd_split_one_chunk<D, C>(grid, static_cast<const float *>(workspace), state, core,
                                         T, NC, H, scale, vl, stream);
    } else
        hipLaunchKernelGGL((kda_chunk_fwd_kernel<D, C>), grid,
                           dim3(PrefCfg<D, C>::kThreads), 0, stream,
                           static_cast<const float *>(workspace), state, core, T, NC, H, scale, vl);
    return hipGetLastError();
}

#define KDA_PREFILL_DISPATCH(FN, ...)                                        \
    (head_dim == 128 && chunk == 64)   ? FN<128, 64>(__VA_ARGS__)            \
    : (head_dim == 128 && chunk == 16) ? FN<128, 16>(__VA_ARGS__)            \
    : (head_dim == 16 && chunk == 64)  ? FN<16, 64>(__VA_ARGS__)             \
                                       : FN<16, 16>(__VA_ARGS__)

hipError_t launch_kda_prefill_prepare(const float *q, const float *k, const float *v,
                                      const float *gate, const float *beta, int T, int heads,
                                      int head_dim, int chunk, void *workspace,
                                      hipStream_t stream)
{
    // chunks are independent here: a long sequence is prepared in pieces of
    // at most kMaxChunksPerLaunch chunks (a grid dimension's limit), each
    // into its own blocks of the one-pass layout
    const int NC = (T + chunk - 1) / chunk;
    const int64_t HD = (int64_t)heads * head_dim;
    const size_t chunk_bytes = prefill_workspace_bytes(chunk, heads, head_dim, chunk);
    for (int c0 = 0; c0 < NC; c0 += kMaxChunksPerLaunch) {
        const int64_t r0 = (int64_t)c0 * chunk;
        const int Ts = (int)std::min<int64_t>((int64_t)T - r0, (int64_t)kMaxChunksPerLaunch * chunk);
        void *ws = static_cast<char *>(workspace) + (size_t)c0 * chunk_bytes;
        const hipError_t e = KDA_PREFILL_DISPATCH(prepare_t, q + r0 * HD, k + r0 * HD, v + r0 * HD,
                                                  gate + r0 * HD, beta + r0 * heads, Ts, heads,
                                                  ws, Varlen{}, 1, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_kda_prefill_forward(float *state, float *core, int T, int heads, int head_dim,
                                      int chunk, float scale, const void *workspace,
                                      hipStream_t stream)
{
    return KDA_PREFILL_DISPATCH(forward_t, state, core, T, heads, scale, workspace, Varlen{}, 1,
                                stream);
}

hipError_t launch_kda_prefill(const float *q, const float *k, const float *v,
                              const float *gate, const float *beta, float *state,
                              float *core, int T, int heads, int head_dim, int chunk,
                              float scale, void *workspace, hipStream_t stream)
{
    return launch_kda_prefill_segments(q, k, v, gate, beta, state, core, T, heads, head_dim,
                                       chunk, scale, workspace,
                                       prefill_segment_chunks(T, heads, head_dim, chunk), stream);
}

hipError_t launch_kda_prefill_segments(const float *q, const float *k, const float *v,
                                       const float *gate, const float *beta, float *state,
                                       float *core, int T, int heads, int head_dim, int chunk,
                                       float scale, void *workspace, int seg, hipStream_t stream)
{
    // Segments of `seg` chunks, each prepared into the start of the workspace
    // and walked at once: a segment's operand blocks (at most the cache
    // budget) are still in the last-level cache when the walk reads them.
    // Chunk boundaries and the carried state are those of one long pass, so
    // the result is bitwise the same.
    const int NC = (T + chunk - 1) / chunk;
    const int64_t HD = (int64_t)heads * head_dim;
    for (int c0 = 0; c0 < NC; c0 += seg) {
        const int64_t r0 = (int64_t)c0 * chunk;
        const int Ts = (int)std::min<int64_t>((int64_t)T - r0, (int64_t)seg * chunk);
        hipError_t e = launch_kda_prefill_prepare(q + r0 * HD, k + r0 * HD, v + r0 * HD,
                                                  gate + r0 * HD, beta + r0 * heads, Ts, heads,
                                                  head_dim, chunk, workspace, stream);
        if (e != hipSuccess) return e;
        e = launch_kda_prefill_forward(state, core + r0 * HD, Ts, heads, head_dim, chunk, scale,
                                       workspace, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_kda_prefill_bf16(const uint16_t *qkv, int64_t ldqkv, const float *gate,
                                   const float *beta, float *state, float *core, int T,
                                   int heads, int head_dim, int chunk, float scale,
                                   void *workspace, hipStream_t stream)
{
    // the segments of launch_kda_prefill, reading q | k | v from bf16 rows
    const int NC = (T + chunk - 1) / chunk;
    const int seg = prefill_segment_chunks(T, heads, head_dim, chunk);
    const int64_t HD = (int64_t)heads * head_dim;
    for (int c0 = 0; c0 < NC; c0 += seg) {
        const int64_t r0 = (int64_t)c0 * chunk;
        const int Ts = (int)std::min<int64_t>((int64_t)T - r0, (int64_t)seg * chunk);
        hipError_t e = KDA_PREFILL_DISPATCH(prepare_bf16_t, qkv + r0 * ldqkv, ldqkv,
                                            gate + r0 * HD, beta + r0 * heads, Ts, heads,
                                            workspace, stream);
        if (e != hipSuccess) return e;
        e = launch_kda_prefill_forward(state, core + r0 * HD, Ts, heads, head_dim, chunk, scale,
                                       workspace, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_kda_prefill_varlen(const float *q, const float *k, const float *v,
                                     const float *gate, const float *beta, float *const *state,
                                     float *core, const int32_t *cu_seqlens, int B, int64_t rows,
                                     int max_chunks, int total_chunks, int heads, int head_dim,
                                     int chunk, float scale, void *workspace, int32_t *status,
                                     hipStream_t stream)
{
    // Segments of global chunks sized as kda_prefill's: each is prepared into
    // the start of the workspace and walked at once (one walk per sequence,
    // head and value slice that has chunks in it), so the forward pass reads
    // operand blocks the prepare pass has just left in the last-level cache.
    if (max_chunks <= 1 && head_dim == 128 && chunk == 64) {
        // every sequence one chunk: prepare and walk in one kernel, which
        // reads each operand block back at once, so one launch over all
        // chunks (no cache-sized segments; each block at its own place)
        const Varlen vl{cu_seqlens, state, rows, max_chunks, total_chunks, 0, total_chunks,
                        status};
        return prefill_one_chunk<128, 64>(q, k, v, gate, beta, core, heads, scale, workspace, vl,
                                          B, stream);
    }
    const int seg = prefill_segment_chunks(total_chunks * chunk, heads, head_dim, chunk);
    for (int lo = 0; lo < total_chunks; lo += seg) {
        const Varlen vl{cu_seqlens, state, rows, max_chunks, total_chunks, lo,
                        std::min(lo + seg, total_chunks), status};
        hipError_t e = KDA_PREFILL_DISPATCH(prepare_t, q, k, v, gate, beta, 0, heads, workspace,
                                            vl, B, stream);
        if (e != hipSuccess) return e;
        e = KDA_PREFILL_DISPATCH(forward_t, nullptr, core, 0, heads, scale, workspace, vl, B,
                                 stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace kda
