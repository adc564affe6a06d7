// kda_gate: bounded per-channel log-decay and beta ("Glm5NextKdaWorkspace"
// page, fields g_raw, gate and beta; "Glm5NextKdaWeights" page, fields a_log,
// per head, and dt_bias, per channel).
//   gate[t,h,d] = -exp(a_log[h]) * softplus(g_raw[t, h*D+d] + dt_bias[h*D+d])
//   beta[t,h]   = sigmoid(b_raw[t,h])
// Element-wise and HBM-bound: each thread reads 8 bf16 (one 16-byte load) and
// writes 8 fp32 (two 16-byte stores); consecutive threads cover consecutive
// channels of a row.  Exponentials and logarithms run on the transcendental
// unit (relative error near 1e-7, far inside the fp32 tolerance).
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

constexpr int kGateThreads = 256;

// Grid (rows, channel groups of 8 per row / kGateThreads): no integer
// division on the way to the element; blocks with blockIdx.x >= T compute
// beta, kGateThreads * gridDim.y elements of the [T, H] array each.
__global__ __launch_bounds__(kGateThreads) void kda_gate_kernel(
    const uint16_t *__restrict__ g_raw, int64_t ldg, const uint16_t *__restrict__ b_raw,
    int64_t ldb, const float *__restrict__ a_log, const float *__restrict__ dt_bias,
    int T, int H, int D, float *__restrict__ gate, float *__restrict__ beta)
{
    const int qkv = H * D;
    const int row = blockIdx.x;
    if (row < T) {
        const int c0 = (blockIdx.y * kGateThreads + threadIdx.x) * 8;
        if (c0 >= qkv) return;
        const int h = c0 / D;
        float x[8];
        unpack8(*reinterpret_cast<const uint4 *>(g_raw + (int64_t)row * ldg + c0), x);
        const float4 b0 = *reinterpret_cast<const float4 *>(dt_bias + c0);
        const float4 b1 = *reinterpret_cast<const float4 *>(dt_bias + c0 + 4);
        const float bias[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
        const float A = decay_rate(a_log[h]);
        float g[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) g[e] = log_decay(x[e], bias[e], A);
        float4 *dst = reinterpret_cast<float4 *>(gate + (int64_t)row * qkv + c0);
        dst[0] = make_float4(g[0], g[1], g[2], g[3]);
        dst[1] = make_float4(g[4], g[5], g[6], g[7]);
    } else {
        // beta: elements (row - T) * per + [0, per) of the [T, H] array, one
        // per thread, per = gridDim.y * kGateThreads
        const int per = gridDim.y * kGateThreads;
        const int64_t idx = (int64_t)(row - T) * per + blockIdx.y * kGateThreads + threadIdx.x;
        if (idx >= (int64_t)T * H) return;
        const int t = (int)(idx / H), hh = (int)(idx - (int64_t)t * H);
        beta[idx] = sigmoid_fast(bf16_to_f32(b_raw[(int64_t)t * ldb + hh]));
    }
}

hipError_t launch_kda_gate(const uint16_t *g_raw, int64_t ldg, const uint16_t *b_raw,
                           int64_t ldb, const float *a_log, const float *dt_bias, int T,
                           int heads, int head_dim, float *gate, float *beta,
                           hipStream_t stream)
{
    const int groups_per_row = heads * head_dim / 8;
    const int gx = (groups_per_row + kGateThreads - 1) / kGateThreads;
    const int64_t per = (int64_t)gx * kGateThreads;
    const int beta_rows = b_raw ? (int)(((int64_t)T * heads + per - 1) / per) : 0;
    hipLaunchKernelGGL(kda_gate_kernel, dim3(T + beta_rows, gx), dim3(kGateThreads), 0, stream,
                       g_raw, ldg, b_raw, ldb, a_log, dt_bias, T, heads, head_dim, gate, beta);
    return hipGetLastError();
}

}  // namespace kda
