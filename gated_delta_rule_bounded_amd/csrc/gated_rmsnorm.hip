// gated_rmsnorm: sigmoid-gated RMSNorm of the core output per (token, head)
// ("Glm5NextKdaWorkspace" page, fields core, out_gate and o_norm_out;
// "Glm5NextKdaWeights" page, field o_norm).
//   out[t, h*D+d] = bf16( x_d * rsqrt(mean_d x^2 + eps) * w[d] * sigmoid(gate[t, h*D+d]) )
// HBM-bound: each thread owns 8 consecutive channels (two 16-byte fp32 loads,
// one 16-byte bf16 gate load, one 16-byte store); the D/8 threads of a head are
// adjacent lanes and reduce the sum of squares by xor-shuffles.
#include "kda_device.hpp"
#include "kda_launch.hpp"
#include "kda_rows.hpp"

namespace kda {

constexpr int kNormThreads = 256;

// Grid (rows, channel groups of 8 / kNormThreads): no integer division on
// the way to the element.  rsqrt, exp and the reciprocal run on the
// transcendental unit (~1 ulp each, far inside the bf16 output rounding).
template <int D>
__global__ __launch_bounds__(kNormThreads) void gated_rmsnorm_kernel(
    const float *__restrict__ core, int64_t ldc, const uint16_t *__restrict__ out_gate,
    int64_t ldo, const uint16_t *__restrict__ w, int T, int H, float eps,
    uint16_t *__restrict__ out, int64_t ldy)
{
    const int t = blockIdx.x;
    const int cg = blockIdx.y * kNormThreads + threadIdx.x;
    const bool active = cg < H * D / 8;
    const int c0 = active ? cg * 8 : 0;
    const int d0 = c0 % D;
    const float4 a = *reinterpret_cast<const float4 *>(core + (int64_t)t * ldc + c0);
    const float4 b = *reinterpret_cast<const float4 *>(core + (int64_t)t * ldc + c0 + 4);
    const float xv[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    const uint4 o = gated_norm8<D>(xv, *reinterpret_cast<const uint4 *>(out_gate + (int64_t)t * ldo + c0),
                                   *reinterpret_cast<const uint4 *>(w + d0), eps);
    if (active) *reinterpret_cast<uint4 *>(out + (int64_t)t * ldy + c0) = o;
}

hipError_t launch_gated_rmsnorm(const float *core, int64_t ldc, const uint16_t *out_gate,
                                int64_t ldo, const uint16_t *w, int T, int heads,
                                int head_dim, float eps, uint16_t *out, int64_t ldy,
                                hipStream_t stream)
{
    const int groups_per_row = heads * head_dim / 8;
    const dim3 grid(T, (groups_per_row + kNormThreads - 1) / kNormThreads);
    if (head_dim == 128)
        hipLaunchKernelGGL(gated_rmsnorm_kernel<128>, grid, dim3(kNormThreads), 0, stream, core,
                           ldc, out_gate, ldo, w, T, heads, eps, out, ldy);
    else
        hipLaunchKernelGGL(gated_rmsnorm_kernel<16>, grid, dim3(kNormThreads), 0, stream, core,
                           ldc, out_gate, ldo, w, T, heads, eps, out, ldy);
    return hipGetLastError();
}

}  // namespace kda
