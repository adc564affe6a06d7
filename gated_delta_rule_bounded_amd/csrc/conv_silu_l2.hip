// conv_silu_l2: short causal depthwise conv + SiLU + per-head L2 of q and k
// ("Glm5NextKdaWorkspace" page, fields qkv_proj, conv_out and q_f32;
// "Glm5NextKdaWeights" page, field conv; "Glm5NextKdaLayer" page, decode and
// decode_k for the carried conv state and its per-row snapshots).
//
// For each row t and channel c (window = the last KC pre-conv rows, newest
// last; it starts from the carried conv state):
//   pre = sum_j w[c][j] * window[j][c]       (tap KC-1 meets row t)
//   s   = pre * sigmoid(pre)   (exp, reciprocal and rsqrt on the
//                               transcendental unit, ~1 ulp each)
//   q and k sections: s /= sqrt(sum over the head's D channels of s^2 + eps)
//   y   = bf16(s)  (one rounding), optional exact fp32 copies of q, k, v.
//
// Mapping: a thread owns 8 consecutive channels (one 16-byte bf16 load per
// row) and walks a tile of consecutive rows with the window in registers, so
// each input row is read once.  The D/8 threads of one head are adjacent
// lanes; the L2 sum reduces among them by xor-shuffles in a fixed order.  The
// per-row arithmetic does not depend on the tiling, so the K-row snapshot
// mode is bit-identical to K single-row calls.  Only row tile 0 of a sequence
// reads the old conv state, and the same threads write the new state after
// reading it, so no other workgroup can observe a half-updated state.
#include "kda_device.hpp"
#include "kda_launch.hpp"
#include "kda_rows.hpp"

namespace kda {

constexpr int kConvThreads = 256;
// kConvRowsPerTile (kda_launch.hpp): 8 rows per tile (128 VGPRs, four waves
// per SIMD) measured fastest at 8192 rows x 12288 channels: 84 us against
// 88 us for 4 rows, 98 us for 16 (160 VGPRs, three waves) and 126 us for 32
// (two waves)

template <int D, int RPT>
__global__ __launch_bounds__(kConvThreads) void conv_silu_l2_kernel(
    const uint16_t *__restrict__ x, int64_t ldx, const uint16_t *__restrict__ w,
    uint16_t *const *__restrict__ conv_state, uint16_t *const *__restrict__ conv_snap,
    int rows, int H, int ntiles, float eps_l2, uint16_t *__restrict__ y, int64_t ldy,
    float *__restrict__ q32, float *__restrict__ k32, float *__restrict__ v32, bool write_state)
{
    constexpr int KC = kConvKC;
    constexpr int LANES_PER_HEAD = D / 8;
    const int qkv = H * D;
    const int conv_dim = 3 * qkv;
    const int grp = blockIdx.x * kConvThreads + threadIdx.x;
    const bool active = grp < conv_dim / 8;
    const int c0 = active ? grp * 8 : 0;
    const int tile = blockIdx.y;
    const int seq = blockIdx.z;
    const int t0 = tile * RPT;
    const int t1 = min(rows, t0 + RPT);
    const int64_t row0 = (int64_t)seq * rows;   // first row of this sequence
    const uint16_t *__restrict__ st = conv_state ? conv_state[seq] : nullptr;

    // taps for the 8 channels: w[c][0..KC-1]
    float wt[8][KC];
    conv_taps(w, c0, wt);

    // window: win[j] holds input row (t - KC + 1 + j) once row t is loaded
    uint4 win[KC];
#pragma unroll
    for (int j = 1; j < KC; ++j) {
        const int r = t0 - KC + j;   // sequence-local row index, may be < 0
        if (r >= 0)
            win[j] = *reinterpret_cast<const uint4 *>(x + (row0 + r) * ldx + c0);
        else if (st != nullptr)
            win[j] = gload16(st + (int64_t)(KC + r) * conv_dim + c0);
        else
            win[j] = make_uint4(0u, 0u, 0u, 0u);
    }
    win[0] = make_uint4(0u, 0u, 0u, 0u);

    const int section = c0 / qkv;           // 0 = q, 1 = k, 2 = v
    const int cs = c0 - section * qkv;      // channel within the section

    // the tile's rows are all loaded up front (many 16-byte loads in flight
    // per wave), then computed in order
    uint4 rowv[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i)
        if (t0 + i < t1) rowv[i] = *reinterpret_cast<const uint4 *>(x + (row0 + t0 + i) * ldx + c0);
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int t = t0 + i;
        if (t >= t1) break;
#pragma unroll
        for (int j = 0; j + 1 < KC; ++j) win[j] = win[j + 1];
        win[KC - 1] = rowv[i];

        const uint4 packed = conv_row<LANES_PER_HEAD>(win, wt, section < 2, eps_l2);
        if (active) {
            *reinterpret_cast<uint4 *>(y + (row0 + t) * ldy + c0) = packed;
            if (q32 != nullptr) {
                float *dst = (section == 0 ? q32 : section == 1 ? k32 : v32) +
                             (row0 + t) * qkv + cs;
                float f[8];
                unpack8(packed, f);
                reinterpret_cast<float4 *>(dst)[0] = make_float4(f[0], f[1], f[2], f[3]);
                reinterpret_cast<float4 *>(dst)[1] = make_float4(f[4], f[5], f[6], f[7]);
            }
            if (conv_snap != nullptr && t + 1 < rows) {
                uint16_t *dst = conv_snap[row0 - seq + t];   // seq*(rows-1) + t
#pragma unroll
                for (int j = 0; j < KC; ++j)
                    gstore16(dst + (int64_t)j * conv_dim + c0, win[j]);
            }
        }
    }

    // new conv state = the window after the sequence's last row (launched
    // with write_state only when RPT >= KC, so that tile 0 is the only one
    // that reads the old state)
    if (write_state && tile == 0 && st != nullptr && active) {
        uint16_t *dst = conv_state[seq];
        if (ntiles == 1) {
#pragma unroll
            for (int j = 0; j < KC; ++j) gstore16(dst + (int64_t)j * conv_dim + c0, win[j]);
        } else {
            // rows >= kConvRowsPerTile >= KC: the window is the last KC rows of x
#pragma unroll
            for (int j = 0; j < KC; ++j)
                gstore16(dst + (int64_t)j * conv_dim + c0,
                         *reinterpret_cast<const uint4 *>(x + (row0 + rows - KC + j) * ldx + c0));
        }
    }
}

// Write-on-accept for the conv window ("Glm5NextLayer" page,
// LayerWriteOnAccept): after a verify that left the conv states untouched,
// sequence b's window moves past its first n = n_accept[b] pre-conv rows
// (clamped to [0, K]): the new window is the last KC rows of [old window;
// rows b*K .. b*K + n - 1 of x], exactly the snapshot a K-row conv call writes
// after row n - 1.  A thread owns 8 channels and reads its whole old window
// before writing any of it.
__global__ __launch_bounds__(kConvThreads) void conv_fold_kernel(
    const uint16_t *__restrict__ x, int64_t ldx, uint16_t *const *__restrict__ conv_state,
    const int32_t *__restrict__ n_accept, int K, int conv_dim)
{
    constexpr int KC = kConvKC;
    const int grp = blockIdx.x * kConvThreads + threadIdx.x;
    const int b = blockIdx.y;
    const int n = min(max(n_accept[b], 0), K);
    if (grp >= conv_dim / 8 || n == 0) return;
    const int c0 = grp * 8;
    uint16_t *__restrict__ st = conv_state[b];
    uint4 old[KC];
#pragma unroll
    for (int j = 0; j < KC; ++j) old[j] = gload16(st + (int64_t)j * conv_dim + c0);
#pragma unroll
    for (int j = 0; j < KC; ++j) {
        const int idx = n + j;   // position in [old window; accepted rows]
        // the accepted row idx - KC (a row of this sequence whatever idx is:
        // clamped, and used only when idx >= KC), and old[idx] picked by
        // selects over the unrolled window, word by word (an indexed register
        // array, or a select between the two addresses, would go through
        // scratch memory)
        const uint4 xr = *reinterpret_cast<const uint4 *>(
            x + ((int64_t)b * K + max(idx - KC, 0)) * ldx + c0);
        uint32_t o[4] = {old[KC - 1].x, old[KC - 1].y, old[KC - 1].z, old[KC - 1].w};
#pragma unroll
        for (int i = KC - 2; i >= 0; --i) {
            o[0] = idx == i ? old[i].x : o[0];
            o[1] = idx == i ? old[i].y : o[1];
            o[2] = idx == i ? old[i].z : o[2];
            o[3] = idx == i ? old[i].w : o[3];
        }
        const bool own = idx < KC;
        gstore16(st + (int64_t)j * conv_dim + c0,
                 make_uint4(own ? o[0] : xr.x, own ? o[1] : xr.y, own ? o[2] : xr.z,
                            own ? o[3] : xr.w));
    }
}

hipError_t launch_conv_fold(const uint16_t *x, int64_t ldx, uint16_t *const *conv_state,
                            const int32_t *n_accept, int B, int K, int heads, int head_dim,
                            hipStream_t stream)
{
    const int conv_dim = 3 * heads * head_dim;
    const dim3 grid((conv_dim / 8 + kConvThreads - 1) / kConvThreads, B);
    hipLaunchKernelGGL(conv_fold_kernel, grid, dim3(kConvThreads), 0, stream, x, ldx, conv_state,
                       n_accept, K, conv_dim);
    return hipGetLastError();
}

hipError_t launch_conv_silu_l2(const uint16_t *x, int64_t ldx, const uint16_t *w,
                               uint16_t *const *conv_state, uint16_t *const *conv_snap,
                               int n_seq, int rows, int heads, int head_dim, float eps_l2,
                               uint16_t *y, int64_t ldy, float *q32, float *k32, float *v32,
                               hipStream_t stream, bool write_state)
{
    const int conv_dim = 3 * heads * head_dim;
    // A few rows that leave the conv state alone (a verify): one row per
    // tile, so the rows run side by side instead of one after another in
    // each thread (each tile reads its own window; the per-row arithmetic is
    // the same, so are the bits).  Otherwise tiles of kConvRowsPerTile rows.
    const bool by_row = !write_state && rows <= kConvRowsPerTile;
    const int rpt = by_row ? 1 : kConvRowsPerTile;
    const int ntiles = (rows + rpt - 1) / rpt;
    const dim3 grid((conv_dim / 8 + kConvThreads - 1) / kConvThreads, ntiles, n_seq);
#define KDA_CONV_LAUNCH(DH, RPT)                                                              \
    hipLaunchKernelGGL((conv_silu_l2_kernel<DH, RPT>), grid, dim3(kConvThreads), 0, stream, x, \
                       ldx, w, conv_state, conv_snap, rows, heads, ntiles, eps_l2, y, ldy, q32, \
                       k32, v32, write_state)
    if (head_dim == 128) {
        if (by_row) KDA_CONV_LAUNCH(128, 1);
        else KDA_CONV_LAUNCH(128, kConvRowsPerTile);
    } else {
        if (by_row) KDA_CONV_LAUNCH(16, 1);
        else KDA_CONV_LAUNCH(16, kConvRowsPerTile);
    }
#undef KDA_CONV_LAUNCH
    return hipGetLastError();
}

}  // namespace kda
