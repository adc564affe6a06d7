// Accumulation order of the row-order-exact bf16 products (dense_gemv_bf16_batchm),
// shared by the projection kernel and the fused block-decode kernel, which
// forms the head's slice of the two rank-R products itself and must give the
// projection kernel's bits.
//
// Every output element y[m][n] = sum_k x[m][k] w[n][k] is formed as follows,
// whatever the number of rows:
//   * the contraction is cut into 32-deep steps (one bf16 16x16x32 MFMA each;
//     A = 16 x rows, B = the 16 weight rows of the column tile);
//   * quarter q = 0..3 of the column tile owns the contiguous steps
//     [beg, beg + cnt) and chains them through one fp32 accumulator started at
//     zero, in the order given by gemv_visit (it depends on the column tile
//     and the quarter alone);
//   * the quarters' sums are added as ((p0 + p1) + p2) + p3 and rounded to
//     bf16 (nearest, ties to even).
#pragma once

#include "kda_device.hpp"

namespace kda {

constexpr int kGemvColTile = 16;   // output columns per tile
constexpr int kGemvQuarters = 4;   // contraction quarters per tile

// Quarter q owns the steps [beg, beg + cnt) and visits them starting at beg
// + rho, wrapping around, rho = 12 x (column tile) mod cnt: the workgroups in
// flight read different parts of their weight rows rather than all the same
// offset.
struct GemvVisit {
    int beg, cnt, rho;
    __device__ __forceinline__ int step(int v) const {   // v-th visited step, v < 2 cnt
        const int q = rho + v;
        return beg + (q >= cnt ? q - cnt : q);
    }
};

__device__ __forceinline__ GemvVisit gemv_visit(int quarter, int nsteps, int tile)
{
    const int per = (nsteps + kGemvQuarters - 1) / kGemvQuarters;
    GemvVisit vs;
    vs.beg = min(quarter * per, nsteps);
    vs.cnt = min(vs.beg + per, nsteps) - vs.beg;
    vs.rho = vs.cnt > 0 ? (12 * tile) % vs.cnt : 0;
    return vs;
}

// An element of a product split along the contraction (GemvSeg::ksplit):
// the chunk sums part[(c M + m) N + n] added in chunk order from the first.
__device__ __forceinline__ float split_sum(const float *__restrict__ part, int ks, int64_t M,
                                           int64_t m, int N, int n)
{
    float v = part[m * N + n];
    for (int c = 1; c < ks; ++c) v = v + part[((int64_t)c * M + m) * N + n];
    return v;
}

}  // namespace kda
