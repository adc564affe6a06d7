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

// The plan tables of a several-sequence call (layout above), and its report
// bits (the KDA_REPORT_* values of kda.h): a sequence skipped because its
// chunks do not fit max_chunks / total_chunks, and offsets that had to be
// clamped, ORed into the caller's word with a vector atomic.  One workgroup of
// kPlanThreads walks the sequences in blocks of kPlanThreads, carrying the
// chunk and rank counts from block to block.
constexpr int kPlanThreads = 1024;

__global__ __launch_bounds__(kPlanThreads) void kda_varlen_plan_kernel(
    const int32_t *__restrict__ cu, int B, int64_t rows, int C, int max_chunks,
    int total_chunks, int32_t *__restrict__ plan, int32_t *status)
{
    constexpr int NWV = kPlanThreads / kWave;
    int32_t *seq_of = plan, *chunk0 = plan + total_chunks, *rank = chunk0 + B;
    int32_t *by_rank = rank + B + 1;
    __shared__ int32_t s_c0[kPlanThreads];   // this block's chunk offsets (clamped)
    __shared__ int64_t s_wc[NWV];
    __shared__ int32_t s_wr[NWV];
    __shared__ int32_t s_bits;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    if (tid == 0) s_bits = 0;
    const int64_t cap = (int64_t)total_chunks + 1;
    int64_t base_c = 0;   // chunks of the sequences before this block
    int32_t base_r = 0;   // walked sequences before this block
    int32_t bits = 0;
    for (int s0 = 0; s0 < B; s0 += kPlanThreads) {
        const int s = s0 + tid, n = min(kPlanThreads, B - s0);
        int64_t nch = 0;
        if (s < B) {
            int64_t lo, hi;
            seq_rows(cu, rows, s, lo, hi);
            nch = (hi - lo + C - 1) / C;
            const int64_t a = cu[s], b = cu[s + 1];
            if (a < 0 || b < a || b > rows) bits |= kReportRowsClamped;
        }
        // exclusive prefix of the chunk counts over the block
        int64_t inc = nch;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const int64_t t = __shfl_up(inc, o);
            if (lane >= o) inc += t;
        }
        if (lane == kWave - 1) s_wc[wv] = inc;
        __syncthreads();
        int64_t before = 0, total = 0;
        for (int i = 0; i < NWV; ++i) {
            before += i < wv ? s_wc[i] : 0;
            total += s_wc[i];
        }
        const int64_t c0 = base_c + before + inc - nch;
        const bool ok = nch <= max_chunks && c0 + nch <= total_chunks;
        const int32_t walk = s < B && ok && nch > 0;
        if (s < B && !ok) bits |= kReportSeqSkipped;
        // exclusive prefix of the walked flags
        int32_t rinc = walk;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const int32_t t = __shfl_up(rinc, o);
            if (lane >= o) rinc += t;
        }
        if (lane == kWave - 1) s_wr[wv] = rinc;
        s_c0[tid] = (int32_t)min(c0, cap);
        __syncthreads();
        int32_t rbefore = 0, rtotal = 0;
        for (int i = 0; i < NWV; ++i) {
            rbefore += i < wv ? s_wr[i] : 0;
            rtotal += s_wr[i];
        }
        const int32_t r = base_r + rbefore + rinc - walk;
        if (s < B) {
            chunk0[s] = s_c0[tid];
            rank[s] = r;
            if (walk) by_rank[r] = s;
        }
        // the owner of every global chunk of this block: the last sequence
        // whose first chunk is at or before it (a sequence without chunks
        // shares its first chunk only with sequences after it)
        const int64_t g_end = min(base_c + total, (int64_t)total_chunks);
        for (int64_t g = base_c + tid; g < g_end; g += kPlanThreads) {
            int lo = 0, hi = n;   // s_c0[lo] <= g < s_c0[hi] (s_c0[n] taken as the end)
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (s_c0[mid] <= g) lo = mid; else hi = mid;
            }
            seq_of[g] = s0 + lo;
        }
        base_c += total;
        base_r += rtotal;
        __syncthreads();   // s_c0, s_wc, s_wr reused by the next block
    }
    for (int64_t g = min(base_c, (int64_t)total_chunks) + tid; g < total_chunks; g += kPlanThreads)
        seq_of[g] = -1;
    if (tid == 0) rank[B] = base_r;
    if (status) {
        if (bits) atomicOr(&s_bits, bits);
        __syncthreads();
        if (tid == 0 && s_bits) atomicOr(status, s_bits);
    }
}

size_t prefill_varlen_workspace_bytes(int B, int total_chunks, int heads, int head_dim, int chunk)
{
    const size_t plan = (varlen_plan_ints(B, total_chunks) * sizeof(int32_t) + 255) & ~size_t(255);
    return prefill_workspace_bytes(total_chunks * chunk, heads, head_dim, chunk) + plan;
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
                              int H, void *workspace, const Varlen &vl, hipStream_t stream)
{
    // one workgroup per (chunk, head); for several sequences the chunks are
    // those of the segment.  The split kernel takes the chunks in y (heads
    // fastest); the callers launch at most kMaxChunksPerLaunch chunks at a time
    const int nc = vl.cu ? vl.seg_hi - vl.seg_lo : (T + C - 1) / C;
    const dim3 grid(nc, H), grid_split(H, nc);
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
                            hipStream_t stream)
{
    const QkvSrc<false> src{q, k, v, (int64_t)H * D};
    return prepare_src<D, C, false>(src, gate, beta, T, H, workspace, vl, stream);
}

// q | k | v read from bf16 rows (row stride ldqkv elements)
template <int D, int C>
static hipError_t prepare_bf16_t(const uint16_t *qkv, int64_t ldqkv, const float *gate,
                                 const float *beta, int T, int H, void *workspace,
                                 hipStream_t stream)
{
    const int64_t qw = (int64_t)H * D;
    const QkvSrc<true> src{qkv, qkv + qw, qkv + 2 * qw, ldqkv};
    return prepare_src<D, C, true>(src, gate, beta, T, H, workspace, Varlen{}, stream);
}

template <int D, int C>
static hipError_t forward_t(float *state, float *core, int T, int H, float scale,
                            const void *workspace, const Varlen &vl, int B, hipStream_t stream)
{
    const int NC = (T + C - 1) / C;
    // several sequences: one row of workgroups per sequence of the segment
    // (at most one per chunk)
    const dim3 grid(H * PrefCfg<D, C>::kDT, vl.cu ? std::min(B, vl.seg_hi - vl.seg_lo) : 1);
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
                                                  ws, Varlen{}, stream);
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
    // More than a wave of sequences: the sequence tables after the operand
    // blocks, written first (the plan kernel reports).  Then segments of
    // global chunks sized as kda_prefill's, each prepared into the start of
    // the workspace and walked at once (one walk per sequence, head and value
    // slice that has chunks in it), so the forward pass reads operand blocks
    // the prepare pass has just left in the last-level cache.
    int32_t *plan = nullptr;
    if (B > kWave) {
        plan = reinterpret_cast<int32_t *>(
            static_cast<char *>(workspace) +
            prefill_workspace_bytes(total_chunks * chunk, heads, head_dim, chunk));
        hipLaunchKernelGGL(kda_varlen_plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream,
                           cu_seqlens, B, rows, chunk, max_chunks, total_chunks, plan, status);
        if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
        status = nullptr;
    }
    if (max_chunks <= 1 && head_dim == 128 && chunk == 64) {
        // every sequence one chunk: prepare and walk in one kernel, which
        // reads each operand block back at once, so one launch over all
        // chunks (no cache-sized segments; each block at its own place)
        const Varlen vl{cu_seqlens, state, rows, B, max_chunks, total_chunks, 0, total_chunks,
                        plan, status};
        return prefill_one_chunk<128, 64>(q, k, v, gate, beta, core, heads, scale, workspace, vl,
                                          stream);
    }
    const int seg = std::min(prefill_segment_chunks(total_chunks * chunk, heads, head_dim, chunk),
                             kMaxChunksPerLaunch);
    for (int lo = 0; lo < total_chunks; lo += seg) {
        const Varlen vl{cu_seqlens, state, rows, B, max_chunks, total_chunks, lo,
                        std::min(lo + seg, total_chunks), plan, status};
        hipError_t e = KDA_PREFILL_DISPATCH(prepare_t, q, k, v, gate, beta, 0, heads, workspace,
                                            vl, stream);
        if (e != hipSuccess) return e;
        e = KDA_PREFILL_DISPATCH(forward_t, nullptr, core, 0, heads, scale, workspace, vl, B,
                                 stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace kda
