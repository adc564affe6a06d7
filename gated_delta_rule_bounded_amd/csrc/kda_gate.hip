// kda_gate: bounded per-channel log-decay and beta ("Glm5NextKdaWorkspace"
// page, fields g_raw, gate and beta; "Glm5NextKdaWeights" page, fields a_log,
// per head, and dt_bias, per channel).
//   gate[t,h,d] = -exp(a_log[h]) * softplus(g_raw[t, h*D+d] + dt_bias[h*D+d])
//   beta[t,h]   = sigmoid(b_raw[t,h])
// Element-wise and HBM-bound: each thread reads 8 bf16 (one 16-byte load) and
// writes 8 fp32 (two 16-byte stores); consecutive threads cover consecutive
// channels of a row.  Blocks past the gate range compute beta.
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

constexpr int kGateThreads = 256;

__global__ __launch_bounds__(kGateThreads) void kda_gate_kernel(
    const uint16_t *__restrict__ g_raw, int64_t ldg, const uint16_t *__restrict__ b_raw,
    int64_t ldb, const float *__restrict__ a_log, const float *__restrict__ dt_bias,
    int T, int H, int D, int gate_blocks, float *__restrict__ gate, float *__restrict__ beta)
{
    const int qkv = H * D;
    if ((int)blockIdx.x < gate_blocks) {
        const int groups_per_row = qkv / 8;
        const int64_t gidx = (int64_t)blockIdx.x * kGateThreads + threadIdx.x;
        if (gidx >= (int64_t)T * groups_per_row) return;
        const int t = (int)(gidx / groups_per_row);
        const int c0 = (int)(gidx % groups_per_row) * 8;
        const int h = c0 / D;
        float x[8];
        unpack8(*reinterpret_cast<const uint4 *>(g_raw + (int64_t)t * ldg + c0), x);
        const float4 b0 = *reinterpret_cast<const float4 *>(dt_bias + c0);
        const float4 b1 = *reinterpret_cast<const float4 *>(dt_bias + c0 + 4);
        const float bias[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
        const float A = expf(a_log[h]);
        float g[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float z = x[e] + bias[e];
            const float sp = z > 20.0f ? z : log1pf(expf(z));
            g[e] = -A * sp;
        }
        float4 *dst = reinterpret_cast<float4 *>(gate + (int64_t)t * qkv + c0);
        dst[0] = make_float4(g[0], g[1], g[2], g[3]);
        dst[1] = make_float4(g[4], g[5], g[6], g[7]);
    } else {
        const int64_t idx = (int64_t)(blockIdx.x - gate_blocks) * kGateThreads + threadIdx.x;
        if (idx >= (int64_t)T * H) return;
        const int t = (int)(idx / H), h = (int)(idx % H);
        const float z = bf16_to_f32(b_raw[(int64_t)t * ldb + h]);
        beta[idx] = 1.0f / (1.0f + expf(-z));
    }
}

hipError_t launch_kda_gate(const uint16_t *g_raw, int64_t ldg, const uint16_t *b_raw,
                           int64_t ldb, const float *a_log, const float *dt_bias, int T,
                           int heads, int head_dim, float *gate, float *beta,
                           hipStream_t stream)
{
    const int64_t groups = (int64_t)T * heads * head_dim / 8;
    const int gate_blocks = (int)((groups + kGateThreads - 1) / kGateThreads);
    const int beta_blocks =
        b_raw ? (int)(((int64_t)T * heads + kGateThreads - 1) / kGateThreads) : 0;
    hipLaunchKernelGGL(kda_gate_kernel, dim3(gate_blocks + beta_blocks), dim3(kGateThreads), 0,
                       stream, g_raw, ldg, b_raw, ldb, a_log, dt_bias, T, heads, head_dim,
                       gate_blocks, gate, beta);
    return hipGetLastError();
}

}  // namespace kda
