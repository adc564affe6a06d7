// dense_gemv_bf16_batchm: y[m][n] = bf16( sum_k x[m][k] * w[n][k] ) for a few
// rows m ("Glm5NextKdaLayer" page, decode_k: the projections of K rows run
// once over all rows, and each row must come out exactly as it would alone).
//
// Row-order exactness.  Every output element is accumulated in the same
// order whatever M is and wherever its row sits:
//   * the contraction is cut into 32-deep steps; wave w of the workgroup takes
//     steps w, w+4, w+8, ... and chains them through one bf16 16x16x32 MFMA
//     accumulator in increasing order;
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
#include "kda_launch.hpp"

namespace kda {
namespace {

constexpr int kColTile = 16;       // output columns per workgroup
constexpr int kRowTiles = 4;       // 16-row tiles per workgroup (64 rows)
constexpr int kWaves = 4;
constexpr int kStepsInFlight = 4;  // contraction steps loaded ahead per wave

struct Seg {
    const uint16_t *x;
    const uint16_t *w;
    uint16_t *y;
    int64_t ldx, ldy;
    int32_t N, Kd;
    int32_t tile0;  // first column tile of this segment in the grid
};

struct Args {
    Seg seg[kGemvMaxSegs];
    int32_t nseg;
    int32_t M;
};

__global__ __launch_bounds__(256) void gemv_bf16_batchm(const Args a)
{
    __shared__ float part[kWaves][kRowTiles][16][17];

    // segment of this column tile (uniform scalar search over a handful)
    int s = 0;
#pragma unroll 1
    for (int i = 1; i < a.nseg; ++i)
        if ((int)blockIdx.x >= a.seg[i].tile0) s = i;
    const Seg g = a.seg[s];
    const int n0 = ((int)blockIdx.x - g.tile0) * kColTile;
    const int m0 = (int)blockIdx.y * (kRowTiles * 16);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int r = lane & 15, kg = lane >> 4;
    const int nsteps = g.Kd >> 5;
    const int ntiles = min(kRowTiles, (a.M - m0 + 15) >> 4);

    // this lane's weight row (columns past N read row 0 and are never stored)
    const int n = n0 + r;
    const uint16_t *wrow = g.w + (int64_t)(n < g.N ? n : 0) * g.Kd + 8 * kg;
    // this lane's x rows, one per 16-row tile (rows past M give zero operands)
    const uint16_t *xrow[kRowTiles];
    bool xok[kRowTiles];
#pragma unroll
    for (int t = 0; t < kRowTiles; ++t) {
        const int m = m0 + 16 * t + r;
        xok[t] = m < a.M;
        xrow[t] = g.x + (int64_t)(xok[t] ? m : 0) * g.ldx + 8 * kg;
    }

    floatx4 acc[kRowTiles];
#pragma unroll
    for (int t = 0; t < kRowTiles; ++t) acc[t] = floatx4{0.f, 0.f, 0.f, 0.f};

    // steps wave, wave+4, ...: operands of kStepsInFlight steps loaded at once
#pragma unroll 1
    for (int s0 = wave; s0 < nsteps; s0 += kWaves * kStepsInFlight) {
        uint4 wb[kStepsInFlight], xb[kStepsInFlight][kRowTiles];
#pragma unroll
        for (int j = 0; j < kStepsInFlight; ++j) {
            const int st = s0 + kWaves * j;
            const bool ok = st < nsteps;
            wb[j] = ok ? *reinterpret_cast<const uint4 *>(wrow + 32 * st) : make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int t = 0; t < kRowTiles; ++t)
                xb[j][t] = (ok && t < ntiles && xok[t])
                               ? *reinterpret_cast<const uint4 *>(xrow[t] + 32 * st)
                               : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < kStepsInFlight; ++j) {
            if (s0 + kWaves * j >= nsteps) break;
            const bf16x8 b = __builtin_bit_cast(bf16x8, wb[j]);
#pragma unroll
            for (int t = 0; t < kRowTiles; ++t) {
                if (t >= ntiles) break;
                acc[t] = mfma_bf16(__builtin_bit_cast(bf16x8, xb[j][t]), b, acc[t]);
            }
        }
    }

    // lane holds rows 4*kg + i of each tile at column r
#pragma unroll
    for (int t = 0; t < kRowTiles; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) part[wave][t][4 * kg + i][r] = acc[t][i];
    __syncthreads();

    // one thread per (row, column) of a tile: fixed-order sum of the 4 waves
    const int tr = threadIdx.x >> 4, tc = threadIdx.x & 15;
    if (n0 + tc < g.N) {
#pragma unroll
        for (int t = 0; t < kRowTiles; ++t) {
            const int m = m0 + 16 * t + tr;
            if (t < ntiles && m < a.M) {
                const float v = ((part[0][t][tr][tc] + part[1][t][tr][tc]) + part[2][t][tr][tc]) +
                                part[3][t][tr][tc];
                g.y[(int64_t)m * g.ldy + n0 + tc] = (uint16_t)f32_to_bf16(v);
            }
        }
    }
}

}  // namespace

hipError_t launch_gemv_bf16_batchm(const GemvSeg *segs, int nseg, int M, hipStream_t stream)
{
    if (M <= 0 || nseg <= 0) return hipSuccess;
    Args a = {};
    int tiles = 0;
    for (int i = 0; i < nseg; ++i) {
        a.seg[i] = Seg{segs[i].x, segs[i].w, segs[i].y, segs[i].ldx, segs[i].ldy,
                       segs[i].N, segs[i].Kd, tiles};
        tiles += (segs[i].N + kColTile - 1) / kColTile;
    }
    a.nseg = nseg;
    a.M = M;
    const dim3 grid(tiles, (M + kRowTiles * 16 - 1) / (kRowTiles * 16));
    hipLaunchKernelGGL(gemv_bf16_batchm, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace kda
