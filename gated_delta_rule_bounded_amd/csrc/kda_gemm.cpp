// The block's projections: plain bf16 GEMMs y = x W^T with fp32 accumulation,
// run by the vendor library (hipBLASLt).  Weights are in torch Linear layout
// [out, in] ("Glm5NextKdaWeights" page); every output is a bf16 buffer.
//
// Library state, kept per device for the life of the process: one hipBLASLt
// handle and one plan (descriptors + the algorithm the heuristic picked) per
// distinct GEMM shape.  Both are created on the first call that needs them;
// no call allocates device memory for its own use (the GEMM workspace is the
// caller's).
#include <hipblaslt/hipblaslt.h>

#include <map>
#include <mutex>
#include <tuple>

#include "kda_launch.hpp"

namespace kda {
namespace {

struct GemmPlan {
    hipblasLtMatmulDesc_t desc = nullptr;
    hipblasLtMatrixLayout_t a = nullptr, b = nullptr, c = nullptr;
    hipblasLtMatmulAlgo_t algo{};
};

using PlanKey = std::tuple<int, int, int, int64_t, int64_t, int64_t, size_t>;

struct DeviceGemm {
    hipblasLtHandle_t handle = nullptr;
    std::map<PlanKey, GemmPlan> plans;
};

std::mutex g_mu;
std::map<int, DeviceGemm> g_dev;

const char *status_name(hipblasStatus_t s) {
    switch (s) {
    case HIPBLAS_STATUS_SUCCESS: return "success";
    case HIPBLAS_STATUS_NOT_INITIALIZED: return "not initialized";
    case HIPBLAS_STATUS_ALLOC_FAILED: return "alloc failed";
    case HIPBLAS_STATUS_INVALID_VALUE: return "invalid value";
    case HIPBLAS_STATUS_ARCH_MISMATCH: return "arch mismatch";
    case HIPBLAS_STATUS_EXECUTION_FAILED: return "execution failed";
    case HIPBLAS_STATUS_INTERNAL_ERROR: return "internal error";
    case HIPBLAS_STATUS_NOT_SUPPORTED: return "not supported";
    default: return "error";
    }
}

// Descriptors for the column-major view of y = x W^T:
//   D (n_out x rows, ld ldy) = op(A) op(B),  A = W stored (n_in x n_out, ld ldw)
//   and transposed, B = x stored (n_in x rows, ld ldx).
hipblasStatus_t make_plan(hipblasLtHandle_t h, int rows, int n_out, int n_in, int64_t ldx,
                          int64_t ldw, int64_t ldy, size_t ws_bytes, GemmPlan &p)
{
    hipblasStatus_t s;
    if ((s = hipblasLtMatmulDescCreate(&p.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F))) return s;
    const hipblasOperation_t ta = HIPBLAS_OP_T, tb = HIPBLAS_OP_N;
    if ((s = hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &ta, sizeof ta)))
        return s;
    if ((s = hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &tb, sizeof tb)))
        return s;
    if ((s = hipblasLtMatrixLayoutCreate(&p.a, HIP_R_16BF, n_in, n_out, ldw))) return s;
    if ((s = hipblasLtMatrixLayoutCreate(&p.b, HIP_R_16BF, n_in, rows, ldx))) return s;
    if ((s = hipblasLtMatrixLayoutCreate(&p.c, HIP_R_16BF, n_out, rows, ldy))) return s;
    hipblasLtMatmulPreference_t pref;
    if ((s = hipblasLtMatmulPreferenceCreate(&pref))) return s;
    const uint64_t ws = ws_bytes;
    s = hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES,
                                              &ws, sizeof ws);
    hipblasLtMatmulHeuristicResult_t res[1];
    int n = 0;
    if (!s)
        s = hipblasLtMatmulAlgoGetHeuristic(h, p.desc, p.a, p.b, p.c, p.c, pref, 1, res, &n);
    hipblasLtMatmulPreferenceDestroy(pref);
    if (s) return s;
    if (n < 1 || res[0].state != HIPBLAS_STATUS_SUCCESS) return HIPBLAS_STATUS_NOT_SUPPORTED;
    p.algo = res[0].algo;
    return HIPBLAS_STATUS_SUCCESS;
}

}  // namespace

int gemm_bf16_xwT(const uint16_t *x, int64_t ldx, const uint16_t *w, int64_t ldw, uint16_t *y,
                  int64_t ldy, int rows, int n_out, int n_in, void *ws, size_t ws_bytes,
                  hipStream_t stream, const char **what)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        *what = "hipGetDevice failed";
        return 1;
    }
    const GemmPlan *plan = nullptr;
    hipblasLtHandle_t handle = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_mu);
        DeviceGemm &d = g_dev[dev];
        if (!d.handle && hipblasLtCreate(&d.handle) != HIPBLAS_STATUS_SUCCESS) {
            d.handle = nullptr;
            *what = "hipblasLtCreate failed";
            return 1;
        }
        handle = d.handle;
        const PlanKey key{rows, n_out, n_in, ldx, ldw, ldy, ws_bytes};
        auto it = d.plans.find(key);
        if (it == d.plans.end()) {
            GemmPlan p;
            const hipblasStatus_t s = make_plan(handle, rows, n_out, n_in, ldx, ldw, ldy, ws_bytes, p);
            if (s != HIPBLAS_STATUS_SUCCESS) {
                if (p.a) hipblasLtMatrixLayoutDestroy(p.a);
                if (p.b) hipblasLtMatrixLayoutDestroy(p.b);
                if (p.c) hipblasLtMatrixLayoutDestroy(p.c);
                if (p.desc) hipblasLtMatmulDescDestroy(p.desc);
                *what = status_name(s);
                return 1;
            }
            it = d.plans.emplace(key, p).first;
        }
        plan = &it->second;
        // enqueue under the lock: the handle is shared by every caller on this device
        const float alpha = 1.0f, beta = 0.0f;
        const hipblasStatus_t s =
            hipblasLtMatmul(handle, plan->desc, &alpha, w, plan->a, x, plan->b, &beta, y, plan->c,
                            y, plan->c, &plan->algo, ws, ws_bytes, stream);
        if (s != HIPBLAS_STATUS_SUCCESS) {
            *what = status_name(s);
            return 1;
        }
    }
    return 0;
}

// Column ranges of a row-major bf16 matrix x [rows][ldx] copied to their own
// buffers: y_r[t][0 .. n_r) = x[t][c_r .. c_r + n_r), for up to three ranges
// (n_r multiples of 8), 16 bytes per thread.
struct ColSplit {
    uint16_t *y[3];
    int32_t c[3], n[3];
    int32_t chunks;   // 16-byte pieces per row over all ranges
};

__global__ __launch_bounds__(256) void split_cols_kernel(const uint16_t *__restrict__ x,
                                                         int64_t ldx, int64_t rows,
                                                         const ColSplit s)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= rows * s.chunks) return;
    const int64_t t = i / s.chunks;
    int p = (int)(i % s.chunks) * 8;   // element offset within the ranges
    int r = 0;
    while (p >= s.n[r]) p -= s.n[r++];
    *reinterpret_cast<uint4 *>(s.y[r] + t * s.n[r] + p) =
        *reinterpret_cast<const uint4 *>(x + t * ldx + s.c[r] + p);
}

hipError_t launch_split_cols(const uint16_t *x, int64_t ldx, int64_t rows, int nr,
                             uint16_t *const *y, const int *c, const int *n, hipStream_t stream)
{
    ColSplit s{};
    int chunks = 0;
    for (int r = 0; r < nr; ++r) {
        s.y[r] = y[r];
        s.c[r] = c[r];
        s.n[r] = n[r];
        chunks += n[r] / 8;
    }
    s.chunks = chunks;
    const int64_t total = rows * chunks;
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(split_cols_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream,
                       x, ldx, rows, s);
    return hipGetLastError();
}

}  // namespace kda

