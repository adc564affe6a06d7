// dense_gemv_bf16_batchm: y[m][n] = bf16( sum_k x[m][k] * w[n][k] ) for a few
// rows m ("Glm5NextKdaLayer" page, decode_k: the projections of K rows run
// once over all rows, and each row must come out exactly as it would alone).
//
// Row-order exactness.  Every output element is accumulated in the same
// order whatever M is and wherever its row sits:
//   * the contraction is cut into 32-deep steps; wave w of the workgroup takes
//     the w-th quarter of them and chains them through one bf16 16x16x32 MFMA
//     accumulator in an order set by the output column's tile alone (the
//     same for every kernel instance below, whatever its load depth);
//   * the four waves' partial sums meet in LDS and are added as
//     ((p0 + p1) + p2) + p3, then rounded to bf16 (nearest, ties to even).
// A row enters an MFMA only as its own A-operand row, and the matrix unit
// forms each output element from that row and one weight row alone, so the
// other rows of the tile (other tokens, or zeros past M) never touch it.
//
// Layout.  w is torch Linear layout [N][Kd] bf16 (row stride Kd), x [M][Kd]
// with row stride ldx, y [M][N] with row stride ldy.  One workgroup owns 16
// output columns and up to 64 rows (grid.y covers further rows), so at the
// block's shapes the weights, which dominate the traffic, are read from HBM
// exactly once per call.  Several products that share M run in one launch as
// segments (the front projections of a KDA block all read the same hidden
// rows).
#include "kda_device.hpp"
#include "kda_gemv.hpp"
#include "kda_launch.hpp"

namespace kda {
namespace {

constexpr int kColTile = kGemvColTile;   // output columns per workgroup
constexpr int kWaves = kGemvQuarters;    // one wave per contraction quarter

struct Seg {
    const uint16_t *x;
    const uint16_t *w;
    uint16_t *y;
    int64_t ldx, ldy;
    int32_t N, Kd;
    int32_t tile0;  // first workgroup of this segment in the grid
    int32_t epi, head_dim;
    float *act;
    const float *a_log, *dt_bias;
    int32_t ksplit;  // contraction chunks (workgroups per column tile)
    float *part;     // chunk sums when ksplit > 1
};

// Store one result: its bf16 rounding, and the segment's activation of it.
__device__ __forceinline__ void store_out(const Seg &g, int m, int n, float v)
{
    const uint32_t u = f32_to_bf16(v);
    g.y[(int64_t)m * g.ldy + n] = (uint16_t)u;
    if (g.epi == kEpiGate)
        g.act[(int64_t)m * g.N + n] =
            log_decay(bf16_to_f32(u), g.dt_bias[n], decay_rate(g.a_log[n / g.head_dim]));
    else if (g.epi == kEpiBeta)
        g.act[(int64_t)m * g.N + n] = sigmoid_fast(bf16_to_f32(u));
}

struct Args {
    Seg seg[kGemvMaxSegs];
    int32_t nseg;
    int32_t M;
};

// Operands of SIF contraction steps (the wave's visited steps v0 .. v0 +
// SIF - 1) for RT row tiles.  Every load is issued unconditionally, so the
// compiler can count the loads in flight exactly and wait for one stage while
// the next is still coming: slots past the wave's last step re-read its first
// one (their products are skipped).
//
// Weights.  The MFMA's B operand wants, in lane (r, kg), 16 bytes of weight
// row r at a 64-byte step: loaded that way, each instruction would touch 16
// rows in 64-byte pieces, which the vector-memory path serves at about a
// quarter of its rate for contiguous spans.  So a stage's weights are loaded
// per row instead: a row's SIF steps are SIF * 64 consecutive bytes (unless
// the visit wraps around inside the stage), and lane l of load i takes
// 16-byte chunk l % (4 SIF) of row i * (16 / SIF) + l / (4 SIF), so one
// instruction covers 16 / SIF rows with contiguous spans.  The chunks go
// through the wave's own LDS rows into the operand layout; the values and
// their order of use are exactly those of per-step loads.
//
// x is read through a buffer resource bounded by the rows that exist: lanes
// of rows past M carry an offset beyond the bound, which the hardware answers
// with zeros and no memory traffic.
template <int RT, int SIF>
struct Stage {
    uintx4 w[SIF];
    uint4 x[SIF][RT];
};

constexpr uint32_t kOutOfRange = 0x80000000u;

__device__ __forceinline__ uint4 load_x(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// LDS rows of a wave's staged weights: 16 rows of 4 SIF chunks, padded by one
// chunk against bank conflicts on the operand reads.
template <int SIF>
using WRows = uintx4[16][4 * SIF + 1];
// With XL the x rows go the same way (16 RT rows: each row's stage is one
// contiguous span, instead of 16 rows' 64-byte pieces per load).
template <int RT, int SIF>
using XRows = uintx4[16 * RT][4 * SIF + 1];

template <int RT, int SIF, bool NT, bool XL>
__device__ __forceinline__ void load_stage(Stage<RT, SIF> &S, const uint16_t *__restrict__ w,
                                           const int64_t (&wrow)[SIF], int lane,
                                           __amdgpu_buffer_rsrc_t xr, const uint32_t (&xoff)[RT],
                                           uint32_t xrows, const GemvVisit &vs, int v0)
{
    constexpr int CPR = 4 * SIF, RPI = 16 / SIF;   // 16-byte chunks per row, rows per load
    const int c = lane % CPR;
    const int vj = v0 + c / 4;     // visited step of this lane's chunk
    const int stc = vj < vs.cnt ? vs.step(vj) : vs.beg;   // past the end: a valid dummy
#pragma unroll
    for (int i = 0; i < SIF; ++i)
    {
        const uintx4 *p = reinterpret_cast<const uintx4 *>(w + wrow[i] + 32 * stc + 8 * (c % 4));
        S.w[i] = NT ? __builtin_nontemporal_load(p) : *p;
    }
    if constexpr (XL) {
        // load i: rows i RPI + lane / CPR, this lane's chunk of their stage;
        // xoff[0] is the byte offset of row lane / CPR (out of range past the
        // rows), xrows the bytes of RPI rows
        const uint32_t o = xoff[0] + 2u * (uint32_t)(32 * stc + 8 * (c % 4));
#pragma unroll
        for (int i = 0; i < SIF * RT; ++i) S.x[i / RT][i % RT] = load_x(xr, o + xrows * (uint32_t)i);
    } else {
#pragma unroll
        for (int j = 0; j < SIF; ++j) {
            const int st = v0 + j < vs.cnt ? vs.step(v0 + j) : vs.beg;
#pragma unroll
            for (int t = 0; t < RT; ++t) S.x[j][t] = load_x(xr, xoff[t] + 64u * st);
        }
    }
}

// the staged weights (and with XL the x rows) into the wave's LDS rows
// (after the stage before them has been read from there: the wave's own LDS
// accesses complete in order)
template <int RT, int SIF, bool XL>
__device__ __forceinline__ void put_stage(const Stage<RT, SIF> &S, WRows<SIF> &L,
                                          XRows<RT, SIF> &X, int lane)
{
    constexpr int CPR = 4 * SIF, RPI = 16 / SIF;
#pragma unroll
    for (int i = 0; i < SIF; ++i) L[i * RPI + lane / CPR][lane % CPR] = S.w[i];
    if constexpr (XL) {
#pragma unroll
        for (int i = 0; i < SIF * RT; ++i)
            X[i * RPI + lane / CPR][lane % CPR] = __builtin_bit_cast(uintx4, S.x[i / RT][i % RT]);
    }
}

template <int RT, int SIF, bool XL>
__device__ __forceinline__ void mma_stage(const Stage<RT, SIF> &S, const WRows<SIF> &L,
                                          const XRows<RT, SIF> &X, floatx4 (&acc)[RT],
                                          const GemvVisit &vs, int v0, int r, int kg)
{
#pragma unroll
    for (int j = 0; j < SIF; ++j) {
        if (v0 + j >= vs.cnt) break;
        const bf16x8 b = __builtin_bit_cast(bf16x8, L[r][4 * j + kg]);
#pragma unroll
        for (int t = 0; t < RT; ++t) {
            const bf16x8 xa = XL ? __builtin_bit_cast(bf16x8, X[16 * t + r][4 * j + kg])
                                 : __builtin_bit_cast(bf16x8, S.x[j][t]);
            acc[t] = mfma_bf16(xa, b, acc[t]);
        }
    }
}

// RT 16-row tiles per workgroup (grid.y covers the rest of M); SIF steps per
// load stage, two stages in flight; NT marks the weight loads non-temporal
// (streaming).  None of these changes any element's order of accumulation,
// only how many rows a workgroup carries and how its loads run.
template <int RT, int SIF, bool NT, bool XL>
__global__ __launch_bounds__(256) void gemv_bf16_batchm(const Args a)
{
    __shared__ float part[kWaves][RT][16][17];
    __shared__ WRows<SIF> s_w[kWaves];
    __shared__ XRows<RT, SIF> s_x[XL ? kWaves : 1];   // with XL only

    // segment of this column tile (uniform scalar search over a handful)
    int s = 0;
#pragma unroll 1
    for (int i = 1; i < a.nseg; ++i)
        if ((int)blockIdx.x >= a.seg[i].tile0) s = i;
    const Seg g = a.seg[s];
    // column tile, and the contraction chunk [k0, k0 + kc) of a split segment
    const int unit = (int)blockIdx.x - g.tile0;
    const int chunk = unit % g.ksplit;
    const int n0 = unit / g.ksplit * kColTile;
    const int kc = g.Kd / g.ksplit, k0 = chunk * kc;
    const int m0 = (int)blockIdx.y * (RT * 16);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int r = lane & 15, kg = lane >> 4;
    const int nsteps = kc >> 5;

    // the weight rows this lane loads (element offsets; columns past N read
    // row 0 and are never stored)
    int64_t wrow[SIF];
#pragma unroll
    for (int i = 0; i < SIF; ++i) {
        const int n = n0 + i * (16 / SIF) + lane / (4 * SIF);
        wrow[i] = (int64_t)(n < g.N ? n : 0) * g.Kd + k0;
    }
    // this lane's x rows, one per 16-row tile: byte offsets from the chunk's
    // first column of the workgroup's first row, or out of range for rows
    // past M (with XL: xoff[0] the row lane / (4 SIF) of the contiguous row
    // loads, xrows the bytes of 16 / SIF rows; rows past M then lie past the
    // bound by themselves)
    const int rows = min(a.M - m0, RT * 16);
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(g.x + (int64_t)m0 * g.ldx + k0), (short)0,
        (int)((int64_t)rows * g.ldx * 2 - (int64_t)k0 * 2), 0x00020000);
    uint32_t xoff[RT] = {}, xrows = 0;
    if constexpr (XL) {
        xoff[0] = (uint32_t)((int64_t)(lane / (4 * SIF)) * g.ldx * 2);
        xrows = (uint32_t)((int64_t)(16 / SIF) * g.ldx * 2);
    } else {
#pragma unroll
        for (int t = 0; t < RT; ++t) {
            const int m = 16 * t + r;
            xoff[t] = m < rows ? (uint32_t)(((int64_t)m * g.ldx + 8 * kg) * 2) : kOutOfRange;
        }
    }

    floatx4 acc[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) acc[t] = floatx4{0.f, 0.f, 0.f, 0.f};

    const GemvVisit vs = gemv_visit(wave, nsteps, n0 / kColTile);
    if (vs.cnt > 0) {
        WRows<SIF> &L = s_w[wave];
        XRows<RT, SIF> &X = s_x[XL ? wave : 0];
        Stage<RT, SIF> A, B;
        load_stage<RT, SIF, NT, XL>(A, g.w, wrow, lane, xr, xoff, xrows, vs, 0);
        load_stage<RT, SIF, NT, XL>(B, g.w, wrow, lane, xr, xoff, xrows, vs, SIF);
        put_stage<RT, SIF, XL>(A, L, X, lane);
#pragma unroll 1
        for (int v = 0; v < vs.cnt; v += 2 * SIF) {
            mma_stage<RT, SIF, XL>(A, L, X, acc, vs, v, r, kg);
            load_stage<RT, SIF, NT, XL>(A, g.w, wrow, lane, xr, xoff, xrows, vs, v + 2 * SIF);
            put_stage<RT, SIF, XL>(B, L, X, lane);
            mma_stage<RT, SIF, XL>(B, L, X, acc, vs, v + SIF, r, kg);
            load_stage<RT, SIF, NT, XL>(B, g.w, wrow, lane, xr, xoff, xrows, vs, v + 3 * SIF);
            put_stage<RT, SIF, XL>(A, L, X, lane);
        }
    }

    // lane holds rows 4*kg + i of each tile at column r
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) part[wave][t][4 * kg + i][r] = acc[t][i];
    __syncthreads();

    // one thread per (row, column) of a tile: fixed-order sum of the 4 waves
    const int tr = threadIdx.x >> 4, tc = threadIdx.x & 15;
    if (n0 + tc < g.N) {
#pragma unroll
        for (int t = 0; t < RT; ++t) {
            const int m = m0 + 16 * t + tr;
            if (m < a.M) {
                const float v = ((part[0][t][tr][tc] + part[1][t][tr][tc]) + part[2][t][tr][tc]) +
                                part[3][t][tr][tc];
                if (g.ksplit > 1)
                    g.part[((int64_t)chunk * a.M + m) * g.N + n0 + tc] = v;
                else
                    store_out(g, m, n0 + tc, v);
            }
        }
    }
}

// The low-rank products of a block split along the contraction: each
// (row, column) of f_a, g_a (rank columns) and b_proj (heads columns) summed
// from its chunks, rounded to bf16, and beta = sigmoid(b_raw) formed as the
// b_proj epilogue forms it.
__global__ __launch_bounds__(256) void lowrank_finish_kernel(
    const float *__restrict__ part, int ks, int M, int rank, int heads, uint16_t *__restrict__ fa,
    uint16_t *__restrict__ ga, uint16_t *__restrict__ b_raw, float *__restrict__ beta)
{
    const int ncol = 2 * rank + heads;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)M * ncol) return;
    const int m = (int)(i / ncol), n = (int)(i % ncol);
    if (n < 2 * rank) {
        const int which = n / rank, j = n % rank;
        const uint32_t u = f32_to_bf16(split_sum(part + (int64_t)which * ks * M * rank, ks, M, m, rank, j));
        (which == 0 ? fa : ga)[(int64_t)m * rank + j] = (uint16_t)u;
    } else {
        const int j = n - 2 * rank;
        const uint32_t u = f32_to_bf16(split_sum(part + (int64_t)2 * ks * M * rank, ks, M, m, heads, j));
        b_raw[(int64_t)m * heads + j] = (uint16_t)u;
        beta[(int64_t)m * heads + j] = sigmoid_fast(bf16_to_f32(u));
    }
}

}  // namespace

hipError_t launch_lowrank_finish(const float *part, int ks, int M, int rank, int heads,
                                 uint16_t *fa, uint16_t *ga, uint16_t *b_raw, float *beta,
                                 hipStream_t stream)
{
    const int64_t n = (int64_t)M * (2 * rank + heads);
    hipLaunchKernelGGL(lowrank_finish_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                       stream, part, ks, M, rank, heads, fa, ga, b_raw, beta);
    return hipGetLastError();
}

hipError_t launch_gemv_bf16_batchm(const GemvSeg *segs, int nseg, int M, hipStream_t stream)
{
    if (M <= 0 || nseg <= 0) return hipSuccess;
    Args a = {};
    int tiles = 0;
    for (int i = 0; i < nseg; ++i) {
        a.seg[i] = Seg{segs[i].x,     segs[i].w,        segs[i].y,   segs[i].ldx,
                       segs[i].ldy,   segs[i].N,        segs[i].Kd,  tiles,
                       segs[i].epi,   segs[i].head_dim, segs[i].act, segs[i].a_log,
                       segs[i].dt_bias, max(segs[i].ksplit, 1), segs[i].part};
        tiles += (segs[i].N + kColTile - 1) / kColTile * max(segs[i].ksplit, 1);
    }
    a.nseg = nseg;
    a.M = M;
    // up to 16 rows: one row tile, deeper loads; more rows: four row tiles.
    // A wave's steps at Kd = 4096 (32) are a whole number of load pairs at
    // both depths, so no slot of the last pass is a dummy: measured on weights
    // streamed from HBM, 4 steps per stage beat 6 (which leaves dummies) by
    // about 10 %, and 8 (fewer resident workgroups) by about 6 %.
    // Non-temporal weight loads measured 6 % faster for launches of more
    // tiles than CUs (the q|k|v product: 20.7 against 22.1 us) and 3 % slower
    // at one tile per CU (o_proj), so only the former take them.
    const bool nt = tiles > 256;
    // past 8 rows the x rows (then as many bytes as a tile's weights, or
    // several times) are read as contiguous row spans through LDS, as the
    // weights are, against 16 rows' 64-byte pieces per load: q|k|v at 16
    // rows 25.4 -> 22.4 us, at 64 rows 64.5 -> 39.8 us; 17 to 32 rows take
    // two row tiles a workgroup (at 17 rows 31.0 -> 24.6 us against four)
    if (M <= 8) {
        if (nt)
            hipLaunchKernelGGL((gemv_bf16_batchm<1, 4, true, false>), dim3(tiles, 1), dim3(256), 0,
                               stream, a);
        else
            hipLaunchKernelGGL((gemv_bf16_batchm<1, 4, false, false>), dim3(tiles, 1), dim3(256),
                               0, stream, a);
    } else if (M <= 16) {
        if (nt)
            hipLaunchKernelGGL((gemv_bf16_batchm<1, 4, true, true>), dim3(tiles, 1), dim3(256), 0,
                               stream, a);
        else
            hipLaunchKernelGGL((gemv_bf16_batchm<1, 4, false, true>), dim3(tiles, 1), dim3(256),
                               0, stream, a);
    } else if (M <= 32) {
        if (nt)
            hipLaunchKernelGGL((gemv_bf16_batchm<2, 2, true, true>), dim3(tiles, (M + 31) / 32),
                               dim3(256), 0, stream, a);
        else
            hipLaunchKernelGGL((gemv_bf16_batchm<2, 2, false, true>), dim3(tiles, (M + 31) / 32),
                               dim3(256), 0, stream, a);
    } else {
        const dim3 grid(tiles, (M + 63) / 64);
        if (nt)
            hipLaunchKernelGGL((gemv_bf16_batchm<4, 2, true, true>), grid, dim3(256), 0, stream,
                               a);
        else
            hipLaunchKernelGGL((gemv_bf16_batchm<4, 2, false, true>), grid, dim3(256), 0, stream,
                               a);
    }
    return hipGetLastError();
}

}  // namespace kda
