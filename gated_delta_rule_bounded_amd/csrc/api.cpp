// C entry points of libkda: argument validation, error reporting, dispatch to
// the kernel launchers.  The library allocates nothing and never synchronises.
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/kda.h"
#include "kda_launch.hpp"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_err[0] = '\0';
    return KDA_OK;
}

int hip_status(hipError_t e, const char *what) {
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

bool head_dim_ok(int d) { return d == 16 || d == 128; }

// largest grid extent along y and z of a launch
constexpr int64_t kMaxGridYZ = 65535;

// [lo, hi) byte ranges overlap
bool overlap(const void *a, size_t na, const void *b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const char *pa = static_cast<const char *>(a), *pb = static_cast<const char *>(b);
    return pa < pb + nb && pb < pa + na;
}

}  // namespace

extern "C" {

const char *kda_last_error(void) { return g_err; }

int conv_silu_l2(const uint16_t *x, int64_t ldx, const uint16_t *w,
                 uint16_t *const *conv_state, uint16_t *const *conv_snap, int32_t n_seq,
                 int32_t rows, int32_t heads, int32_t head_dim, int32_t kc, float eps_l2,
                 uint16_t *y, int64_t ldy, float *q32, float *k32, float *v32,
                 hipStream_t stream)
{
    if (n_seq < 0 || rows < 0 || heads <= 0 || n_seq > kMaxGridYZ ||
        ((int64_t)rows + kda::kConvRowsPerTile - 1) / kda::kConvRowsPerTile > kMaxGridYZ)
        return fail(KDA_ERR_SHAPE, "conv_silu_l2: n_seq=%d rows=%d heads=%d", n_seq, rows, heads);
    if (!head_dim_ok(head_dim) || kc != 4)
        return fail(KDA_ERR_UNSUPPORTED, "conv_silu_l2: head_dim=%d kc=%d (need 16|128, 4)",
                    head_dim, kc);
    if (n_seq == 0 || rows == 0) return ok();
    if (!x || !w || !y) return fail(KDA_ERR_NULL, "conv_silu_l2: x, w and y are required");
    const int64_t conv_dim = 3LL * heads * head_dim;
    if (ldx < conv_dim || ldy < conv_dim || ldx % 8 || ldy % 8)
        return fail(KDA_ERR_SHAPE, "conv_silu_l2: ldx=%lld ldy=%lld conv_dim=%lld",
                    (long long)ldx, (long long)ldy, (long long)conv_dim);
    const bool any32 = q32 || k32 || v32;
    if (any32 && !(q32 && k32 && v32))
        return fail(KDA_ERR_NULL, "conv_silu_l2: q32, k32, v32 must all be given or all NULL");
    if (!aligned16(x) || !aligned16(w) || !aligned16(y) ||
        (any32 && (!aligned16(q32) || !aligned16(k32) || !aligned16(v32))))
        return fail(KDA_ERR_SHAPE, "conv_silu_l2: pointers must be 16-byte aligned");
    const int64_t nrows = (int64_t)n_seq * rows;
    if (overlap(x, (size_t)((nrows - 1) * ldx + conv_dim) * 2, y,
                (size_t)((nrows - 1) * ldy + conv_dim) * 2))
        return fail(KDA_ERR_ALIAS, "conv_silu_l2: y overlaps x");
    return hip_status(kda::launch_conv_silu_l2(x, ldx, w, conv_state, conv_snap, n_seq, rows,
                                               heads, head_dim, eps_l2, y, ldy, q32, k32, v32,
                                               stream),
                      "conv_silu_l2 launch");
}

int kda_gate(const uint16_t *g_raw, int64_t ldg, const uint16_t *b_raw, int64_t ldb,
             const float *a_log, const float *dt_bias, int32_t T, int32_t heads,
             int32_t head_dim, float *gate, float *beta, hipStream_t stream)
{
    if (T < 0 || T > (1 << 24) || heads <= 0)
        return fail(KDA_ERR_SHAPE, "kda_gate: T=%d heads=%d", T, heads);
    if (!head_dim_ok(head_dim))
        return fail(KDA_ERR_UNSUPPORTED, "kda_gate: head_dim=%d", head_dim);
    if (T == 0) return ok();
    if (!g_raw || !a_log || !dt_bias || !gate || (b_raw && !beta))
        return fail(KDA_ERR_NULL, "kda_gate: g_raw, a_log, dt_bias, gate (and beta with b_raw) required");
    const int64_t qkv = (int64_t)heads * head_dim;
    if (ldg < qkv || ldg % 8 || (b_raw && ldb < heads))
        return fail(KDA_ERR_SHAPE, "kda_gate: ldg=%lld ldb=%lld", (long long)ldg, (long long)ldb);
    if (!aligned16(g_raw) || !aligned16(dt_bias) || !aligned16(gate))
        return fail(KDA_ERR_SHAPE, "kda_gate: g_raw, dt_bias, gate must be 16-byte aligned");
    if (overlap(gate, (size_t)T * qkv * 4, g_raw, (size_t)((T - 1) * ldg + qkv) * 2) ||
        (b_raw && overlap(beta, (size_t)T * heads * 4, b_raw, (size_t)((T - 1) * ldb + heads) * 2)))
        return fail(KDA_ERR_ALIAS, "kda_gate: an output overlaps an input");
    return hip_status(kda::launch_kda_gate(g_raw, ldg, b_raw, ldb, a_log, dt_bias, T, heads,
                                           head_dim, gate, beta, stream),
                      "kda_gate launch");
}

size_t kda_prefill_workspace_bytes(int32_t T_pad, int32_t heads, int32_t head_dim, int32_t chunk)
{
    if (T_pad < 0 || heads <= 0 || !(chunk == 16 || chunk == 64) || T_pad % chunk) return 0;
    return kda::prefill_workspace_bytes(T_pad, heads, head_dim, chunk);
}

size_t kda_prefill_varlen_workspace_bytes(int32_t B, int32_t total_chunks, int32_t heads,
                                          int32_t head_dim, int32_t chunk)
{
    if (B < 0 || B > 65535 || total_chunks < 0 || heads <= 0 || !(chunk == 16 || chunk == 64) ||
        (int64_t)total_chunks * chunk > (int64_t)1 << 30)
        return 0;
    return kda::prefill_varlen_workspace_bytes(B, total_chunks, heads, head_dim, chunk);
}

int32_t kda_prefill_segment_chunks(int32_t T, int32_t heads, int32_t head_dim, int32_t chunk)
{
    if (T < 0 || heads <= 0 || !head_dim_ok(head_dim) || !(chunk == 16 || chunk == 64)) return 0;
    return kda::prefill_segment_chunks(T, heads, head_dim, chunk);
}

// Shared validation of the prefill family; v may be NULL for prepare, beta
// NULL for forward, state/core NULL for prepare.
static int check_prefill(const char *who, const float *q, const float *k, const float *v,
                         const float *gate, const float *beta, const float *state,
                         const float *core, int32_t T, int32_t T_pad, int32_t heads,
                         int32_t head_dim, int32_t chunk, const void *workspace,
                         size_t workspace_bytes, bool need_v, bool need_beta, bool need_out,
                         bool own_ws = false)
{
    if (!head_dim_ok(head_dim) || !(chunk == 16 || chunk == 64))
        return fail(KDA_ERR_UNSUPPORTED, "%s: head_dim=%d chunk=%d (need 16|128, 16|64)", who,
                    head_dim, chunk);
    if (T < 0 || heads <= 0 || T_pad < T || T_pad % chunk)
        return fail(KDA_ERR_SHAPE, "%s: T=%d T_pad=%d heads=%d chunk=%d", who, T, T_pad, heads,
                    chunk);
    if (T == 0) return 1;   // no-op
    if (!q || !k || !gate || (!workspace && !own_ws) || (need_v && !v) || (need_beta && !beta) ||
        (need_out && (!state || !core)))
        return fail(KDA_ERR_NULL, "%s: null pointer argument", who);
    // own_ws: the library's own scratch array (never a caller region), so
    // there is no caller workspace to size or to check for overlap
    const size_t need = own_ws ? 0 : kda::prefill_workspace_bytes(T_pad, heads, head_dim, chunk);
    if (workspace_bytes < need)
        return fail(KDA_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu needed", who,
                    workspace_bytes, need);
    if (!aligned16(q) || !aligned16(k) || !aligned16(gate) || (need_v && !aligned16(v)) ||
        (need_out && (!aligned16(state) || !aligned16(core))) ||
        (reinterpret_cast<uintptr_t>(workspace) & 255u))
        return fail(KDA_ERR_SHAPE, "%s: misaligned pointer", who);
    const size_t rows_b = (size_t)T_pad * heads * head_dim * 4;
    const size_t st_b = (size_t)heads * head_dim * head_dim * 4;
    const void *ins[] = {q, k, v, gate};
    if (need_out) {
        for (const void *p : ins)
            if (overlap(core, rows_b, p, rows_b) || overlap(state, st_b, p, rows_b))
                return fail(KDA_ERR_ALIAS, "%s: core or state overlaps an input", who);
        if (overlap(core, rows_b, beta, (size_t)T_pad * heads * 4) ||
            overlap(core, rows_b, state, st_b) || overlap(workspace, need, core, rows_b) ||
            overlap(workspace, need, state, st_b))
            return fail(KDA_ERR_ALIAS, "%s: core, state, beta or workspace overlap", who);
    }
    for (const void *p : ins)
        if (overlap(workspace, need, p, rows_b))
            return fail(KDA_ERR_ALIAS, "%s: workspace overlaps an input", who);
    if (overlap(workspace, need, beta, (size_t)T_pad * heads * 4))
        return fail(KDA_ERR_ALIAS, "%s: workspace overlaps beta", who);
    return KDA_OK;
}

int kda_prefill(const float *q, const float *k, const float *v, const float *gate,
                const float *beta, float *state, float *core, int32_t T, int32_t T_pad,
                int32_t heads, int32_t head_dim, int32_t chunk, float scale, void *workspace,
                size_t workspace_bytes, hipStream_t stream)
{
    const int rc = check_prefill("kda_prefill", q, k, v, gate, beta, state, core, T, T_pad,
                                 heads, head_dim, chunk, workspace, workspace_bytes, true, true,
                                 true);
    if (rc == 1) return ok();
    if (rc) return rc;
    return hip_status(kda::launch_kda_prefill(q, k, v, gate, beta, state, core, T, heads,
                                              head_dim, chunk, scale, workspace, stream),
                      "kda_prefill launch");
}

int kda_prefill_noalloc(const float *q, const float *k, const float *v, const float *gate,
                        const float *beta, float *state, float *core, int32_t T, int32_t T_pad,
                        int32_t heads, int32_t head_dim, int32_t chunk, float scale,
                        hipStream_t stream)
{
    const int rc = check_prefill("kda_prefill_noalloc", q, k, v, gate, beta, state, core, T,
                                 T_pad, heads, head_dim, chunk, nullptr, 0, true, true, true,
                                 true);
    if (rc == 1) return ok();
    if (rc) return rc;
    const size_t per_chunk = kda::prefill_workspace_bytes(chunk, heads, head_dim, chunk);
    if (per_chunk > kda::kNoallocScratchBytes)
        return fail(KDA_ERR_WORKSPACE,
                    "kda_prefill_noalloc: one chunk of %d heads needs %zu bytes of operand blocks, "
                    "more than the %zu-byte scratch array", heads, per_chunk,
                    kda::kNoallocScratchBytes);
    return hip_status(kda::launch_kda_prefill_noalloc(q, k, v, gate, beta, state, core, T, heads,
                                                      head_dim, chunk, scale, stream),
                      "kda_prefill_noalloc launch");
}

int kda_prefill_bf16(const uint16_t *qkv, int64_t ldqkv, const float *gate, const float *beta,
                     float *state, float *core, int32_t T, int32_t T_pad, int32_t heads,
                     int32_t head_dim, int32_t chunk, float scale, void *workspace,
                     size_t workspace_bytes, hipStream_t stream)
{
    if (!head_dim_ok(head_dim) || !(chunk == 16 || chunk == 64))
        return fail(KDA_ERR_UNSUPPORTED, "kda_prefill_bf16: head_dim=%d chunk=%d", head_dim,
                    chunk);
    if (T < 0 || heads <= 0 || T_pad < T || T_pad % chunk)
        return fail(KDA_ERR_SHAPE, "kda_prefill_bf16: T=%d T_pad=%d heads=%d chunk=%d", T, T_pad,
                    heads, chunk);
    if (T == 0) return ok();
    if (!qkv || !gate || !beta || !state || !core || !workspace)
        return fail(KDA_ERR_NULL, "kda_prefill_bf16: null pointer argument");
    const int64_t qw = (int64_t)heads * head_dim;
    if (ldqkv < 3 * qw || ldqkv % 4)
        return fail(KDA_ERR_SHAPE, "kda_prefill_bf16: ldqkv=%lld", (long long)ldqkv);
    const size_t need = kda::prefill_workspace_bytes(T_pad, heads, head_dim, chunk);
    if (workspace_bytes < need)
        return fail(KDA_ERR_WORKSPACE, "kda_prefill_bf16: workspace %zu bytes < %zu needed",
                    workspace_bytes, need);
    if ((reinterpret_cast<uintptr_t>(qkv) & 7u) || !aligned16(gate) || !aligned16(state) ||
        !aligned16(core) || (reinterpret_cast<uintptr_t>(workspace) & 255u))
        return fail(KDA_ERR_SHAPE, "kda_prefill_bf16: misaligned pointer");
    const size_t rows_b = (size_t)T_pad * qw * 4, st_b = (size_t)heads * head_dim * head_dim * 4;
    const size_t qkv_b = (size_t)((T_pad - 1) * ldqkv + 3 * qw) * 2;
    const size_t beta_b = (size_t)T_pad * heads * 4;
    if (overlap(core, rows_b, qkv, qkv_b) || overlap(core, rows_b, gate, rows_b) ||
        overlap(core, rows_b, beta, beta_b) || overlap(core, rows_b, state, st_b) ||
        overlap(state, st_b, qkv, qkv_b) || overlap(state, st_b, gate, rows_b) ||
        overlap(state, st_b, beta, beta_b) || overlap(workspace, need, core, rows_b) ||
        overlap(workspace, need, state, st_b) || overlap(workspace, need, qkv, qkv_b) ||
        overlap(workspace, need, gate, rows_b) || overlap(workspace, need, beta, beta_b))
        return fail(KDA_ERR_ALIAS, "kda_prefill_bf16: core, state or workspace overlaps");
    return hip_status(kda::launch_kda_prefill_bf16(qkv, ldqkv, gate, beta, state, core, T, heads,
                                                   head_dim, chunk, scale, workspace, stream),
                      "kda_prefill_bf16 launch");
}

int kda_prefill_split(const float *q, const float *k, const float *v, const float *gate,
                      const float *beta, float *state, float *core, float *cap_state,
                      int32_t T, int32_t cap, int32_t T_pad, int32_t heads, int32_t head_dim,
                      int32_t chunk, float scale, void *workspace, size_t workspace_bytes,
                      hipStream_t stream)
{
    if (!(chunk == 16 || chunk == 64) || cap < 0 || T < 0 || cap > T)
        return fail(chunk == 16 || chunk == 64 ? KDA_ERR_SHAPE : KDA_ERR_UNSUPPORTED,
                    "kda_prefill_split: T=%d cap=%d chunk=%d", T, cap, chunk);
    // the tail's chunks start at cap, so its last chunk ends at
    // cap + round_up(T - cap, chunk): those rows must exist
    const int64_t need_rows = (int64_t)cap + ((int64_t)(T - cap) + chunk - 1) / chunk * chunk;
    if (T_pad < need_rows)
        return fail(KDA_ERR_SHAPE, "kda_prefill_split: T_pad=%d < cap + round_up(T - cap) = %lld",
                    T_pad, (long long)need_rows);
    const int rc = check_prefill("kda_prefill_split", q, k, v, gate, beta, state, core, T, T_pad,
                                 heads, head_dim, chunk, workspace, workspace_bytes, true, true,
                                 true);
    if (rc == 1) return ok();
    if (rc) return rc;
    if (!cap_state) return fail(KDA_ERR_NULL, "kda_prefill_split: cap_state is NULL");
    const size_t st_b = (size_t)heads * head_dim * head_dim * 4;
    const size_t rows_b = (size_t)T_pad * heads * head_dim * 4;
    if (!aligned16(cap_state))
        return fail(KDA_ERR_SHAPE, "kda_prefill_split: cap_state must be 16-byte aligned");
    if (overlap(cap_state, st_b, state, st_b) || overlap(cap_state, st_b, core, rows_b) ||
        overlap(cap_state, st_b, workspace, workspace_bytes) ||
        overlap(cap_state, st_b, q, rows_b) || overlap(cap_state, st_b, k, rows_b) ||
        overlap(cap_state, st_b, v, rows_b) || overlap(cap_state, st_b, gate, rows_b) ||
        overlap(cap_state, st_b, beta, (size_t)T_pad * heads * 4))
        return fail(KDA_ERR_ALIAS, "kda_prefill_split: cap_state overlaps an input, the state, "
                                   "core or the workspace");
    const int64_t HD = (int64_t)heads * head_dim;
    hipError_t e = hipSuccess;
    if (cap > 0)
        e = kda::launch_kda_prefill(q, k, v, gate, beta, state, core, cap, heads, head_dim, chunk,
                                    scale, workspace, stream);
    if (e == hipSuccess)
        e = hipMemcpyAsync(cap_state, state, st_b, hipMemcpyDeviceToDevice, stream);
    if (e == hipSuccess && T > cap)
        e = kda::launch_kda_prefill(q + cap * HD, k + cap * HD, v + cap * HD, gate + cap * HD,
                                    beta + (int64_t)cap * heads, state, core + cap * HD, T - cap,
                                    heads, head_dim, chunk, scale, workspace, stream);
    return hip_status(e, "kda_prefill_split launch");
}

int kda_prefill_prepare(const float *q, const float *k, const float *v, const float *gate,
                        const float *beta, int32_t T, int32_t T_pad, int32_t heads,
                        int32_t head_dim, int32_t chunk, void *workspace,
                        size_t workspace_bytes, hipStream_t stream)
{
    const int rc = check_prefill("kda_prefill_prepare", q, k, v, gate, beta, nullptr, nullptr, T,
                                 T_pad, heads, head_dim, chunk, workspace, workspace_bytes, true,
                                 true, false);
    if (rc == 1) return ok();
    if (rc) return rc;
    return hip_status(kda::launch_kda_prefill_prepare(q, k, v, gate, beta, T, heads, head_dim,
                                                      chunk, workspace, stream),
                      "kda_prefill_prepare launch");
}

int kda_prefill_forward(float *state, float *core, int32_t T, int32_t T_pad, int32_t heads,
                        int32_t head_dim, int32_t chunk, float scale, const void *workspace,
                        size_t workspace_bytes, hipStream_t stream)
{
    if (!head_dim_ok(head_dim) || !(chunk == 16 || chunk == 64))
        return fail(KDA_ERR_UNSUPPORTED, "kda_prefill_forward: head_dim=%d chunk=%d", head_dim,
                    chunk);
    if (T < 0 || heads <= 0 || T_pad < T || T_pad % chunk)
        return fail(KDA_ERR_SHAPE, "kda_prefill_forward: T=%d T_pad=%d heads=%d chunk=%d", T,
                    T_pad, heads, chunk);
    if (T == 0) return ok();
    if (!state || !core || !workspace)
        return fail(KDA_ERR_NULL, "kda_prefill_forward: null pointer argument");
    const size_t need = kda::prefill_workspace_bytes(T_pad, heads, head_dim, chunk);
    if (workspace_bytes < need)
        return fail(KDA_ERR_WORKSPACE, "kda_prefill_forward: workspace %zu bytes < %zu needed",
                    workspace_bytes, need);
    if (!aligned16(state) || !aligned16(core) || (reinterpret_cast<uintptr_t>(workspace) & 255u))
        return fail(KDA_ERR_SHAPE, "kda_prefill_forward: misaligned pointer");
    const size_t rows_b = (size_t)T_pad * heads * head_dim * 4;
    const size_t st_b = (size_t)heads * head_dim * head_dim * 4;
    if (overlap(core, rows_b, state, st_b) || overlap(workspace, need, core, rows_b) ||
        overlap(workspace, need, state, st_b))
        return fail(KDA_ERR_ALIAS, "kda_prefill_forward: core, state or workspace overlap");
    return hip_status(kda::launch_kda_prefill_forward(state, core, T, heads, head_dim, chunk,
                                                      scale, workspace, stream),
                      "kda_prefill_forward launch");
}

int kda_prefill_varlen(const float *q, const float *k, const float *v, const float *gate,
                       const float *beta, float *const *state, float *core,
                       const int32_t *cu_seqlens, int32_t B, int32_t rows, int32_t max_chunks,
                       int32_t total_chunks, int32_t heads, int32_t head_dim, int32_t chunk,
                       float scale, void *workspace, size_t workspace_bytes, int32_t *status,
                       hipStream_t stream)
{
    if (!head_dim_ok(head_dim) || !(chunk == 16 || chunk == 64))
        return fail(KDA_ERR_UNSUPPORTED, "kda_prefill_varlen: head_dim=%d chunk=%d", head_dim,
                    chunk);
    if (B < 0 || rows < 0 || max_chunks < 0 || total_chunks < 0 || heads <= 0 ||
        max_chunks > 65535 || B > 65535)
        return fail(KDA_ERR_SHAPE, "kda_prefill_varlen: B=%d rows=%d max_chunks=%d total_chunks=%d",
                    B, rows, max_chunks, total_chunks);
    if (B == 0 || rows == 0 || total_chunks == 0 || max_chunks == 0) return ok();
    if (!q || !k || !v || !gate || !beta || !state || !core || !cu_seqlens || !workspace)
        return fail(KDA_ERR_NULL, "kda_prefill_varlen: null pointer argument");
    if ((int64_t)total_chunks * chunk > (int64_t)1 << 30)
        return fail(KDA_ERR_SHAPE, "kda_prefill_varlen: total_chunks=%d too large", total_chunks);
    const size_t need = kda::prefill_varlen_workspace_bytes(B, total_chunks, heads, head_dim, chunk);
    if (workspace_bytes < need)
        return fail(KDA_ERR_WORKSPACE, "kda_prefill_varlen: workspace %zu bytes < %zu needed",
                    workspace_bytes, need);
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(gate) || !aligned16(core) ||
        (reinterpret_cast<uintptr_t>(workspace) & 255u) || (status && !aligned4(status)))
        return fail(KDA_ERR_SHAPE, "kda_prefill_varlen: misaligned pointer");
    const size_t rows_b = (size_t)rows * heads * head_dim * 4;
    const size_t beta_b = (size_t)rows * heads * 4;
    const void *ins[] = {q, k, v, gate};
    for (const void *p : ins)
        if (overlap(core, rows_b, p, rows_b) || overlap(workspace, need, p, rows_b))
            return fail(KDA_ERR_ALIAS, "kda_prefill_varlen: core or workspace overlaps an input");
    if (overlap(core, rows_b, beta, beta_b) || overlap(workspace, need, beta, beta_b) ||
        overlap(workspace, need, core, rows_b))
        return fail(KDA_ERR_ALIAS, "kda_prefill_varlen: core or workspace overlaps an input");
    return hip_status(kda::launch_kda_prefill_varlen(q, k, v, gate, beta, state, core, cu_seqlens,
                                                     B, rows, max_chunks, total_chunks, heads,
                                                     head_dim, chunk, scale, workspace, status,
                                                     stream),
                      "kda_prefill_varlen launch");
}

static int check_decode(const char *who, const uint16_t *qkv, int64_t ldqkv, const float *gate,
                        const float *beta, float *const *state, float *core, int32_t rows,
                        int32_t heads, int32_t head_dim)
{
    if (!qkv || !gate || !beta || !state || !core)
        return fail(KDA_ERR_NULL, "%s: null pointer argument", who);
    const int64_t qkvw = (int64_t)heads * head_dim;
    if (ldqkv < 3 * qkvw)
        return fail(KDA_ERR_SHAPE, "%s: ldqkv=%lld < 3*heads*head_dim", who, (long long)ldqkv);
    if (!aligned16(core))
        return fail(KDA_ERR_SHAPE, "%s: core must be 16-byte aligned", who);
    if (overlap(core, (size_t)rows * qkvw * 4, gate, (size_t)rows * qkvw * 4) ||
        overlap(core, (size_t)rows * qkvw * 4, qkv, (size_t)((rows - 1) * ldqkv + 3 * qkvw) * 2) ||
        overlap(core, (size_t)rows * qkvw * 4, beta, (size_t)rows * heads * 4))
        return fail(KDA_ERR_ALIAS, "%s: core overlaps an input", who);
    return KDA_OK;
}

int kda_decode(const uint16_t *qkv, int64_t ldqkv, const float *gate, const float *beta,
               float *const *state, float *core, int32_t B, int32_t heads, int32_t head_dim,
               float scale, hipStream_t stream)
{
    if (B < 0 || heads <= 0 || B > kMaxGridYZ)
        return fail(KDA_ERR_SHAPE, "kda_decode: B=%d heads=%d", B, heads);
    if (!head_dim_ok(head_dim))
        return fail(KDA_ERR_UNSUPPORTED, "kda_decode: head_dim=%d", head_dim);
    if (B == 0) return ok();
    if (int rc = check_decode("kda_decode", qkv, ldqkv, gate, beta, state, core, B, heads, head_dim))
        return rc;
    return hip_status(kda::launch_kda_recurrent(qkv, ldqkv, gate, beta, state, nullptr, core, B,
                                                1, heads, head_dim, scale, stream),
                      "kda_decode launch");
}

int kda_decode_k(const uint16_t *qkv, int64_t ldqkv, const float *gate, const float *beta,
                 float *const *state, float *const *snap, float *core, int32_t B, int32_t K,
                 int32_t heads, int32_t head_dim, float scale, hipStream_t stream)
{
    if (B < 0 || K < 0 || heads <= 0 || B > kMaxGridYZ)
        return fail(KDA_ERR_SHAPE, "kda_decode_k: B=%d K=%d heads=%d", B, K, heads);
    if (!head_dim_ok(head_dim))
        return fail(KDA_ERR_UNSUPPORTED, "kda_decode_k: head_dim=%d", head_dim);
    if (B == 0 || K == 0) return ok();
    if ((int64_t)B * K > (int64_t)1 << 30)
        return fail(KDA_ERR_SHAPE, "kda_decode_k: B*K too large");
    if (int rc = check_decode("kda_decode_k", qkv, ldqkv, gate, beta, state, core, B * K, heads,
                              head_dim))
        return rc;
    if (snap && (const void *)snap == (const void *)state)
        return fail(KDA_ERR_ALIAS, "kda_decode_k: snapshot table is the state table");
    return hip_status(kda::launch_kda_recurrent(qkv, ldqkv, gate, beta, state,
                                                K > 1 ? snap : nullptr, core, B, K, heads,
                                                head_dim, scale, stream),
                      "kda_decode_k launch");
}

int kda_verify_k(const uint16_t *qkv, int64_t ldqkv, const float *gate, const float *beta,
                 float *const *state, float *core, int32_t B, int32_t K, int32_t heads,
                 int32_t head_dim, float scale, hipStream_t stream)
{
    if (B < 0 || K < 0 || heads <= 0 || B > kMaxGridYZ)
        return fail(KDA_ERR_SHAPE, "kda_verify_k: B=%d K=%d heads=%d", B, K, heads);
    if (!head_dim_ok(head_dim))
        return fail(KDA_ERR_UNSUPPORTED, "kda_verify_k: head_dim=%d", head_dim);
    if (B == 0 || K == 0) return ok();
    if ((int64_t)B * K > (int64_t)1 << 30)
        return fail(KDA_ERR_SHAPE, "kda_verify_k: B*K too large");
    if (int rc = check_decode("kda_verify_k", qkv, ldqkv, gate, beta, state, core, B * K, heads,
                              head_dim))
        return rc;
    return hip_status(kda::launch_kda_verify(qkv, ldqkv, gate, beta, state, core, B, K, heads,
                                             head_dim, scale, stream),
                      "kda_verify_k launch");
}

int kda_verify_wy_k(const uint16_t *qkv, int64_t ldqkv, const float *gate, const float *beta,
                    float *const *state, float *const *wy, float *core, int32_t B, int32_t K,
                    int32_t heads, int32_t head_dim, float scale, hipStream_t stream)
{
    if (B < 0 || K < 0 || heads <= 0 || B > kMaxGridYZ)
        return fail(KDA_ERR_SHAPE, "kda_verify_wy_k: B=%d K=%d heads=%d", B, K, heads);
    if (!head_dim_ok(head_dim))
        return fail(KDA_ERR_UNSUPPORTED, "kda_verify_wy_k: head_dim=%d", head_dim);
    if (B == 0 || K == 0) return ok();
    if ((int64_t)B * K > (int64_t)1 << 30)
        return fail(KDA_ERR_SHAPE, "kda_verify_wy_k: B*K too large");
    if (!wy) return fail(KDA_ERR_NULL, "kda_verify_wy_k: null pointer argument");
    if (int rc = check_decode("kda_verify_wy_k", qkv, ldqkv, gate, beta, state, core, B * K,
                              heads, head_dim))
        return rc;
    if ((const void *)wy == (const void *)state)
        return fail(KDA_ERR_ALIAS, "kda_verify_wy_k: table of u rows is the state table");
    return hip_status(kda::launch_kda_verify_wy(qkv, ldqkv, gate, beta, state, wy, core, B, K,
                                                heads, head_dim, scale, stream),
                      "kda_verify_wy_k launch");
}

int kda_fold_wy(const uint16_t *qkv, int64_t ldqkv, const float *gate, float *const *state,
                float *const *wy, const int32_t *n_accept, int32_t B, int32_t K, int32_t heads,
                int32_t head_dim, int32_t *status, hipStream_t stream)
{
    if (B < 0 || K < 0 || heads <= 0 || B > kMaxGridYZ)
        return fail(KDA_ERR_SHAPE, "kda_fold_wy: B=%d K=%d heads=%d", B, K, heads);
    if (!head_dim_ok(head_dim))
        return fail(KDA_ERR_UNSUPPORTED, "kda_fold_wy: head_dim=%d", head_dim);
    if (B == 0 || K == 0) return ok();
    if ((int64_t)B * K > (int64_t)1 << 30)
        return fail(KDA_ERR_SHAPE, "kda_fold_wy: B*K too large");
    if (!qkv || !gate || !state || !wy || !n_accept)
        return fail(KDA_ERR_NULL, "kda_fold_wy: null pointer argument");
    if (ldqkv < 3LL * heads * head_dim)
        return fail(KDA_ERR_SHAPE, "kda_fold_wy: ldqkv=%lld < 3*heads*head_dim", (long long)ldqkv);
    if (status && !aligned4(status))
        return fail(KDA_ERR_SHAPE, "kda_fold_wy: status must be 4-byte aligned");
    if ((const void *)wy == (const void *)state)
        return fail(KDA_ERR_ALIAS, "kda_fold_wy: table of u rows is the state table");
    return hip_status(kda::launch_kda_fold_wy(qkv, ldqkv, gate, state, wy, n_accept, B, K, heads,
                                              head_dim, status, stream),
                      "kda_fold_wy launch");
}

int kda_fold_accepted(const uint16_t *qkv, int64_t ldqkv, const float *gate, const float *beta,
                      float *const *state, const int32_t *n_accept, int32_t B, int32_t K,
                      int32_t heads, int32_t head_dim, int32_t *status, hipStream_t stream)
{
    if (B < 0 || K < 0 || heads <= 0 || B > kMaxGridYZ)
        return fail(KDA_ERR_SHAPE, "kda_fold_accepted: B=%d K=%d heads=%d", B, K, heads);
    if (!head_dim_ok(head_dim))
        return fail(KDA_ERR_UNSUPPORTED, "kda_fold_accepted: head_dim=%d", head_dim);
    if (B == 0 || K == 0) return ok();
    if ((int64_t)B * K > (int64_t)1 << 30)
        return fail(KDA_ERR_SHAPE, "kda_fold_accepted: B*K too large");
    if (!qkv || !gate || !beta || !state || !n_accept)
        return fail(KDA_ERR_NULL, "kda_fold_accepted: null pointer argument");
    if (ldqkv < 3LL * heads * head_dim)
        return fail(KDA_ERR_SHAPE, "kda_fold_accepted: ldqkv=%lld < 3*heads*head_dim",
                    (long long)ldqkv);
    if (status && !aligned4(status))
        return fail(KDA_ERR_SHAPE, "kda_fold_accepted: status must be 4-byte aligned");
    return hip_status(kda::launch_kda_fold(qkv, ldqkv, gate, beta, state, n_accept, B, K, heads,
                                           head_dim, status, stream),
                      "kda_fold_accepted launch");
}

int gated_rmsnorm(const float *core, int64_t ldc, const uint16_t *out_gate, int64_t ldo,
                  const uint16_t *w, int32_t T, int32_t heads, int32_t head_dim, float eps,
                  uint16_t *out, int64_t ldy, hipStream_t stream)
{
    if (T < 0 || T > (1 << 24) || heads <= 0)
        return fail(KDA_ERR_SHAPE, "gated_rmsnorm: T=%d heads=%d", T, heads);
    if (!head_dim_ok(head_dim))
        return fail(KDA_ERR_UNSUPPORTED, "gated_rmsnorm: head_dim=%d", head_dim);
    if (T == 0) return ok();
    if (!core || !out_gate || !w || !out)
        return fail(KDA_ERR_NULL, "gated_rmsnorm: null pointer argument");
    const int64_t qkv = (int64_t)heads * head_dim;
    if (ldc < qkv || ldo < qkv || ldy < qkv || ldc % 4 || ldo % 8 || ldy % 8)
        return fail(KDA_ERR_SHAPE, "gated_rmsnorm: bad row stride");
    if (!aligned16(core) || !aligned16(out_gate) || !aligned16(w) || !aligned16(out))
        return fail(KDA_ERR_SHAPE, "gated_rmsnorm: pointers must be 16-byte aligned");
    const size_t ob = (size_t)((T - 1) * ldy + qkv) * 2;
    if (overlap(out, ob, out_gate, (size_t)((T - 1) * ldo + qkv) * 2) ||
        overlap(out, ob, core, (size_t)((T - 1) * ldc + qkv) * 4))
        return fail(KDA_ERR_ALIAS, "gated_rmsnorm: out overlaps an input");
    return hip_status(kda::launch_gated_rmsnorm(core, ldc, out_gate, ldo, w, T, heads, head_dim,
                                                eps, out, ldy, stream),
                      "gated_rmsnorm launch");
}

int kda_block_prefill(const uint16_t *hidden, const kda_block_weights *w, float *state,
                      uint16_t *const *conv_state, const kda_block_buffers *b, uint16_t *out,
                      int32_t T, int32_t T_pad, int32_t hidden_size, int32_t heads,
                      int32_t head_dim, int32_t rank, int32_t chunk, float scale, float eps_l2,
                      float eps_rms, hipStream_t stream)
{
    if (!head_dim_ok(head_dim) || !(chunk == 16 || chunk == 64))
        return fail(KDA_ERR_UNSUPPORTED, "kda_block_prefill: head_dim=%d chunk=%d", head_dim, chunk);
    const int64_t qkv = (int64_t)heads * head_dim, cd = 3 * qkv;
    if (T < 0 || T_pad < T || T_pad % chunk || heads <= 0 || hidden_size <= 0 || rank <= 0 ||
        hidden_size % 8 || rank % 8 || qkv % 8 || T_pad > (1 << 24) ||
        ((int64_t)T + kda::kConvRowsPerTile - 1) / kda::kConvRowsPerTile > kMaxGridYZ)
        return fail(KDA_ERR_SHAPE, "kda_block_prefill: T=%d T_pad=%d hidden=%d heads=%d rank=%d",
                    T, T_pad, hidden_size, heads, rank);
    if (T == 0) return ok();
    if (!hidden || !w || !state || !conv_state || !b || !out)
        return fail(KDA_ERR_NULL, "kda_block_prefill: null pointer argument");
    const void *wp[] = {w->q_proj, w->k_proj, w->v_proj, w->conv, w->f_a, w->f_b, w->dt_bias,
                        w->a_log, w->b_proj, w->g_a, w->g_b, w->o_norm, w->o_proj};
    const void *bp[] = {b->qkv_proj, b->conv_out, b->fa, b->g_raw, b->b_raw, b->gate, b->beta,
                        b->core, b->ga, b->out_gate, b->o_norm_out, b->prefill_ws};
    for (const void *p : wp)
        if (!p) return fail(KDA_ERR_NULL, "kda_block_prefill: a weight pointer is NULL");
    for (const void *p : bp)
        if (!p) return fail(KDA_ERR_NULL, "kda_block_prefill: a buffer pointer is NULL");
    // the fp32 copies of q, k, v are optional outputs: all three or none
    const bool copies = b->q32 || b->k32 || b->v32;
    if (copies && !(b->q32 && b->k32 && b->v32))
        return fail(KDA_ERR_NULL, "kda_block_prefill: q32, k32, v32 must all be given or all NULL");
    if (copies && (!aligned16(b->q32) || !aligned16(b->k32) || !aligned16(b->v32)))
        return fail(KDA_ERR_SHAPE, "kda_block_prefill: misaligned fp32 copy");
    if (!b->gemm_ws && b->gemm_ws_bytes)
        return fail(KDA_ERR_NULL, "kda_block_prefill: gemm_ws is NULL with gemm_ws_bytes > 0");
    const size_t need = kda::prefill_workspace_bytes(T_pad, heads, head_dim, chunk);
    if (b->prefill_ws_bytes < need)
        return fail(KDA_ERR_WORKSPACE, "kda_block_prefill: prefill workspace %zu bytes < %zu needed",
                    b->prefill_ws_bytes, need);
    for (const void *p : wp)
        if (!aligned16(p)) return fail(KDA_ERR_SHAPE, "kda_block_prefill: misaligned weight");
    for (const void *p : bp)
        if (!aligned16(p)) return fail(KDA_ERR_SHAPE, "kda_block_prefill: misaligned buffer");
    if (!aligned16(hidden) || !aligned16(out) || !aligned16(state) ||
        (reinterpret_cast<uintptr_t>(b->prefill_ws) & 255u))
        return fail(KDA_ERR_SHAPE, "kda_block_prefill: misaligned pointer");

    // every region the call reads or writes; outputs must not touch any other
    const size_t Tp = (size_t)T_pad, H2 = 2, F4 = 4;
    struct Region { const void *p; size_t n; bool written; };
    const Region rg[] = {
        {hidden, (size_t)T * hidden_size * H2, false},
        {w->q_proj, (size_t)qkv * hidden_size * H2, false},
        {w->k_proj, (size_t)qkv * hidden_size * H2, false},
        {w->v_proj, (size_t)qkv * hidden_size * H2, false},
        {w->conv, (size_t)cd * 4 * H2, false},
        {w->f_a, (size_t)rank * hidden_size * H2, false},
        {w->f_b, (size_t)qkv * rank * H2, false},
        {w->dt_bias, (size_t)qkv * F4, false},
        {w->a_log, (size_t)heads * F4, false},
        {w->b_proj, (size_t)heads * hidden_size * H2, false},
        {w->g_a, (size_t)rank * hidden_size * H2, false},
        {w->g_b, (size_t)qkv * rank * H2, false},
        {w->o_norm, (size_t)head_dim * H2, false},
        {w->o_proj, (size_t)hidden_size * qkv * H2, false},
        {b->qkv_proj, Tp * cd * H2, true},
        {b->conv_out, Tp * cd * H2, true},
        {b->q32, Tp * qkv * F4, true},
        {b->k32, Tp * qkv * F4, true},
        {b->v32, Tp * qkv * F4, true},
        {b->fa, Tp * rank * H2, true},
        {b->g_raw, Tp * qkv * H2, true},
        {b->b_raw, Tp * heads * H2, true},
        {b->gate, Tp * qkv * F4, true},
        {b->beta, Tp * heads * F4, true},
        {b->core, Tp * qkv * F4, true},
        {b->ga, Tp * rank * H2, true},
        {b->out_gate, Tp * qkv * H2, true},
        {b->o_norm_out, Tp * qkv * H2, true},
        {b->prefill_ws, need, true},
        {b->gemm_ws, b->gemm_ws_bytes, true},
        {state, (size_t)heads * head_dim * head_dim * F4, true},
        {out, (size_t)T * hidden_size * H2, true},
    };
    const int nr = sizeof(rg) / sizeof(rg[0]);
    for (int i = 0; i < nr; ++i)
        for (int j = i + 1; j < nr; ++j)
            if ((rg[i].written || rg[j].written) && overlap(rg[i].p, rg[i].n, rg[j].p, rg[j].n))
                return fail(KDA_ERR_ALIAS, "kda_block_prefill: regions %d and %d overlap", i, j);

    const char *what = "";
    auto gemm = [&](const char *name, const uint16_t *x, int64_t ldx, const uint16_t *wt,
                    uint16_t *y, int64_t ldy, int n_out, int n_in) {
        if (kda::gemm_bf16_xwT(x, ldx, wt, n_in, y, ldy, T, n_out, n_in, b->gemm_ws,
                               b->gemm_ws_bytes, stream, &what))
            return fail(KDA_ERR_HIP, "kda_block_prefill: %s projection: hipBLASLt %s", name, what);
        return (int)KDA_OK;
    };
    int rc;
    // q|k|v projections straight into the packed pre-conv rows; weights that
    // lie back to back ([q_proj; k_proj; v_proj] as one [3*qkv, hidden]
    // matrix, as a serving engine packs them) run as one wider GEMM
    const size_t wsz = (size_t)qkv * hidden_size;
    if (w->k_proj == w->q_proj + wsz && w->v_proj == w->k_proj + wsz) {
        if ((rc = gemm("qkv", hidden, hidden_size, w->q_proj, b->qkv_proj, cd, (int)cd,
                       hidden_size)))
            return rc;
    } else if ((rc = gemm("q", hidden, hidden_size, w->q_proj, b->qkv_proj, cd, (int)qkv,
                          hidden_size)) ||
               (rc = gemm("k", hidden, hidden_size, w->k_proj, b->qkv_proj + qkv, cd, (int)qkv,
                          hidden_size)) ||
               (rc = gemm("v", hidden, hidden_size, w->v_proj, b->qkv_proj + 2 * qkv, cd,
                          (int)qkv, hidden_size))) {
        return rc;
    }
    if ((rc = hip_status(kda::launch_conv_silu_l2(b->qkv_proj, cd, w->conv, conv_state, nullptr, 1,
                                                  T, heads, head_dim, eps_l2, b->conv_out, cd,
                                                  b->q32, b->k32, b->v32, stream),
                         "kda_block_prefill: conv_silu_l2 launch")))
        return rc;
    // f_a, g_a and b_proj read the same hidden rows: weights that lie back to
    // back ([f_a; g_a; b_proj], one [2*rank + heads, hidden] matrix) run as
    // one GEMM into the start of the GEMM workspace, when it has room for the
    // [T, 2*rank + heads] result beside 4 MiB for the library, and the three
    // column ranges are copied out (the hidden rows are read once, not three
    // times)
    const size_t lr_w = (size_t)rank * hidden_size;
    const int n_lr = 2 * rank + heads;
    const size_t lr_bytes = ((size_t)T * n_lr * 2 + 255) & ~size_t(255);
    const bool lr_packed = w->g_a == w->f_a + lr_w && w->b_proj == w->g_a + lr_w &&
                           heads % 8 == 0 && b->gemm_ws_bytes >= lr_bytes + (size_t(4) << 20);
    if (lr_packed) {
        uint16_t *tmp = static_cast<uint16_t *>(b->gemm_ws);
        if (kda::gemm_bf16_xwT(hidden, hidden_size, w->f_a, hidden_size, tmp, n_lr, T, n_lr,
                               hidden_size, static_cast<char *>(b->gemm_ws) + lr_bytes,
                               b->gemm_ws_bytes - lr_bytes, stream, &what))
            return fail(KDA_ERR_HIP, "kda_block_prefill: f_a|g_a|b_proj projection: hipBLASLt %s",
                        what);
        uint16_t *const ys[3] = {b->fa, b->ga, b->b_raw};
        const int cs[3] = {0, rank, 2 * rank}, ns[3] = {rank, rank, heads};
        if ((rc = hip_status(kda::launch_split_cols(tmp, n_lr, T, 3, ys, cs, ns, stream),
                             "kda_block_prefill: fa|ga|b_raw split launch")))
            return rc;
    } else if ((rc = gemm("f_a", hidden, hidden_size, w->f_a, b->fa, rank, rank, hidden_size)) ||
               (rc = gemm("b_proj", hidden, hidden_size, w->b_proj, b->b_raw, heads, heads,
                          hidden_size))) {
        return rc;
    }
    if ((rc = gemm("f_b", b->fa, rank, w->f_b, b->g_raw, qkv, (int)qkv, rank)))
        return rc;
    if ((rc = hip_status(kda::launch_kda_gate(b->g_raw, qkv, b->b_raw, heads, w->a_log, w->dt_bias,
                                              T, heads, head_dim, b->gate, b->beta, stream),
                         "kda_block_prefill: kda_gate launch")))
        return rc;
    // the core reads q | k | v straight from the bf16 conv output (the fp32
    // copies, when asked for, are its exact widening)
    if ((rc = hip_status(kda::launch_kda_prefill_bf16(b->conv_out, cd, b->gate, b->beta, state,
                                                      b->core, T, heads, head_dim, chunk, scale,
                                                      b->prefill_ws, stream),
                         "kda_block_prefill: kda_prefill launch")))
        return rc;
    if ((!lr_packed && (rc = gemm("g_a", hidden, hidden_size, w->g_a, b->ga, rank, rank,
                                  hidden_size))) ||
        (rc = gemm("g_b", b->ga, rank, w->g_b, b->out_gate, qkv, (int)qkv, rank)))
        return rc;
    if ((rc = hip_status(kda::launch_gated_rmsnorm(b->core, qkv, b->out_gate, qkv, w->o_norm, T,
                                                   heads, head_dim, eps_rms, b->o_norm_out, qkv,
                                                   stream),
                         "kda_block_prefill: gated_rmsnorm launch")))
        return rc;
    if ((rc = gemm("o", b->o_norm_out, qkv, w->o_proj, out, hidden_size, hidden_size, (int)qkv)))
        return rc;
    return ok();
}

int dense_gemv_bf16_batchm(const uint16_t *x, int64_t ldx, const uint16_t *w, int32_t M,
                           int32_t N, int32_t Kd, uint16_t *y, int64_t ldy, hipStream_t stream)
{
    if (M < 0 || N <= 0 || Kd <= 0 || Kd % 32 || M > kMaxGridYZ * 64)
        return fail(KDA_ERR_SHAPE, "dense_gemv_bf16_batchm: M=%d N=%d Kd=%d (Kd %% 32 == 0)", M,
                    N, Kd);
    if (M == 0) return ok();
    if (!x || !w || !y) return fail(KDA_ERR_NULL, "dense_gemv_bf16_batchm: null pointer argument");
    if (ldx < Kd || ldy < N || ldx % 8 || ldx > (1 << 22))
        return fail(KDA_ERR_SHAPE, "dense_gemv_bf16_batchm: ldx=%lld ldy=%lld", (long long)ldx,
                    (long long)ldy);
    if (!aligned16(x) || !aligned16(w) || !aligned16(y))
        return fail(KDA_ERR_SHAPE, "dense_gemv_bf16_batchm: pointers must be 16-byte aligned");
    const size_t yb = (size_t)((M - 1) * ldy + N) * 2;
    if (overlap(y, yb, x, (size_t)((M - 1) * ldx + Kd) * 2) ||
        overlap(y, yb, w, (size_t)N * Kd * 2))
        return fail(KDA_ERR_ALIAS, "dense_gemv_bf16_batchm: y overlaps x or w");
    const kda::GemvSeg seg{x, w, y, ldx, ldy, N, Kd};
    return hip_status(kda::launch_gemv_bf16_batchm(&seg, 1, M, stream),
                      "dense_gemv_bf16_batchm launch");
}

// K rows of B sequences through the block: decode_k (states written, optional
// snapshots) or, with `verify`, the write-on-accept verify (no state, conv
// state or snapshot written).
static int block_decode_run(const uint16_t *hidden, const kda_block_weights *w,
                            float *const *state, uint16_t *const *conv_state, float *const *snap,
                            uint16_t *const *conv_snap, const kda_block_decode_buffers *b,
                            uint16_t *out, int32_t B, int32_t K, int32_t hidden_size,
                            int32_t heads, int32_t head_dim, int32_t rank, float scale,
                            float eps_l2, float eps_rms, bool verify, hipStream_t stream,
                            float *const *wy = nullptr)
{
    if (!head_dim_ok(head_dim))
        return fail(KDA_ERR_UNSUPPORTED, "kda_block_decode_k: head_dim=%d", head_dim);
    const int64_t qkv = (int64_t)heads * head_dim, cd = 3 * qkv;
    if (B < 0 || K < 0 || heads <= 0 || hidden_size <= 0 || rank <= 0 || hidden_size % 32 ||
        rank % 32 || qkv % 32 || (int64_t)B * K > kMaxGridYZ * 64 || B > kMaxGridYZ ||
        hidden_size > (1 << 22) ||
        rank > (1 << 22) || qkv > (1 << 22))
        return fail(KDA_ERR_SHAPE, "kda_block_decode_k: B=%d K=%d hidden=%d heads=%d rank=%d", B,
                    K, hidden_size, heads, rank);
    if (B == 0 || K == 0) return ok();
    if (!hidden || !w || !state || !conv_state || !b || !out)
        return fail(KDA_ERR_NULL, "kda_block_decode_k: null pointer argument");
    const void *wp[] = {w->q_proj, w->k_proj, w->v_proj, w->conv, w->f_a, w->f_b, w->dt_bias,
                        w->a_log, w->b_proj, w->g_a, w->g_b, w->o_norm, w->o_proj};
    const void *bp[] = {b->qkv_proj, b->conv_out, b->fa, b->g_raw, b->b_raw, b->gate,
                        b->beta, b->core, b->ga, b->out_gate, b->o_norm_out};
    for (const void *p : wp)
        if (!p) return fail(KDA_ERR_NULL, "kda_block_decode_k: a weight pointer is NULL");
    for (const void *p : bp)
        if (!p) return fail(KDA_ERR_NULL, "kda_block_decode_k: a buffer pointer is NULL");
    for (const void *p : wp)
        if (!aligned16(p)) return fail(KDA_ERR_SHAPE, "kda_block_decode_k: misaligned weight");
    for (const void *p : bp)
        if (!aligned16(p)) return fail(KDA_ERR_SHAPE, "kda_block_decode_k: misaligned buffer");
    if (!aligned16(hidden) || !aligned16(out))
        return fail(KDA_ERR_SHAPE, "kda_block_decode_k: misaligned pointer");
    if (snap && (const void *)snap == (const void *)state)
        return fail(KDA_ERR_ALIAS, "kda_block_decode_k: snapshot table is the state table");
    if (conv_snap && (const void *)conv_snap == (const void *)conv_state)
        return fail(KDA_ERR_ALIAS, "kda_block_decode_k: conv snapshot table is the conv state table");

    const size_t M = (size_t)B * K, H2 = 2, F4 = 4;
    struct Region { const void *p; size_t n; bool written; };
    const Region rg[] = {
        {hidden, M * hidden_size * H2, false},
        {w->q_proj, (size_t)qkv * hidden_size * H2, false},
        {w->k_proj, (size_t)qkv * hidden_size * H2, false},
        {w->v_proj, (size_t)qkv * hidden_size * H2, false},
        {w->conv, (size_t)cd * 4 * H2, false},
        {w->f_a, (size_t)rank * hidden_size * H2, false},
        {w->f_b, (size_t)qkv * rank * H2, false},
        {w->dt_bias, (size_t)qkv * F4, false},
        {w->a_log, (size_t)heads * F4, false},
        {w->b_proj, (size_t)heads * hidden_size * H2, false},
        {w->g_a, (size_t)rank * hidden_size * H2, false},
        {w->g_b, (size_t)qkv * rank * H2, false},
        {w->o_norm, (size_t)head_dim * H2, false},
        {w->o_proj, (size_t)hidden_size * qkv * H2, false},
        {b->qkv_proj, M * cd * H2, true},
        {b->conv_out, M * cd * H2, true},
        {b->fa, M * rank * H2, true},
        {b->g_raw, M * qkv * H2, true},
        {b->b_raw, M * heads * H2, true},
        {b->gate, M * qkv * F4, true},
        {b->beta, M * heads * F4, true},
        {b->core, M * qkv * F4, true},
        {b->ga, M * rank * H2, true},
        {b->out_gate, M * qkv * H2, true},
        {b->o_norm_out, M * qkv * H2, true},
        {out, M * hidden_size * H2, true},
    };
    const int nr = sizeof(rg) / sizeof(rg[0]);
    for (int i = 0; i < nr; ++i)
        for (int j = i + 1; j < nr; ++j)
            if ((rg[i].written || rg[j].written) && overlap(rg[i].p, rg[i].n, rg[j].p, rg[j].n))
                return fail(KDA_ERR_ALIAS, "kda_block_decode_k: regions %d and %d overlap", i, j);

    const int Mi = (int)M, hs = hidden_size, rk = rank, qk = (int)qkv;
    // front: every projection of the hidden rows, one launch.  Where the
    // output buffer can hold them (it is written only by the last launch),
    // the f_a, g_a and b_proj products are split into kLowRankSplit chunks
    // of the contraction, left there as chunk sums and finished by their
    // consumer: their few column tiles then spread over the CUs next to the
    // q|k|v tiles instead of giving some CUs a fourth whole tile.  The split
    // depends on the shapes alone, so every path gives the same bits.
    const int ks = kda::kLowRankSplit;
    const bool split = hidden_size % (32 * ks) == 0 &&
                       (int64_t)2 * ks * (2 * rank + heads) <= hidden_size;
    float *const part = split ? reinterpret_cast<float *>(out) : nullptr;
    const size_t lr_chunk = (size_t)ks * M * rank;   // floats of one split product
    const kda::GemvSeg front[] = {
        {hidden, w->q_proj, b->qkv_proj, hs, cd, qk, hs},
        {hidden, w->k_proj, b->qkv_proj + qkv, hs, cd, qk, hs},
        {hidden, w->v_proj, b->qkv_proj + 2 * qkv, hs, cd, qk, hs},
        {hidden, w->f_a, b->fa, hs, rk, rk, hs, kda::kEpiNone, nullptr, nullptr, nullptr, 0,
         split ? ks : 1, part},
        {hidden, w->g_a, b->ga, hs, rk, rk, hs, kda::kEpiNone, nullptr, nullptr, nullptr, 0,
         split ? ks : 1, split ? part + lr_chunk : nullptr},
        // b_proj, beta = sigmoid(b_raw) in its epilogue when unsplit (else the
        // consumer forms both from the chunk sums)
        {hidden, w->b_proj, b->b_raw, hs, heads, heads, hs, kda::kEpiBeta, b->beta, nullptr,
         nullptr, 0, split ? ks : 1, split ? part + 2 * lr_chunk : nullptr},
    };
    const kda::GemvSeg mid[] = {
        // f_b with the log-decay gate fused into its epilogue
        {b->fa, w->f_b, b->g_raw, rk, qkv, qk, rk, kda::kEpiGate, b->gate, w->a_log, w->dt_bias,
         head_dim},
        {b->ga, w->g_b, b->out_gate, rk, qkv, qk, rk},
    };
    const kda::GemvSeg back[] = {{b->o_norm_out, w->o_proj, out, qkv, hs, hs, qk}};
    // The rank-R gate products, conv + SiLU + L2, the recurrence and the
    // gated RMSNorm: for up to 16 rows at rank <= 128 in one kernel per
    // (head, sequence) (measured faster than the four launches below at every
    // batch from 1 to 256 sequences), the same bits as the four launches
    // otherwise taken.  A verify writes neither state nor snapshots.
    const bool fuse_mixer = K <= kda::kMixerMaxRows && rank <= kda::kMixerMaxRank;
    kda::MixerArgs mixer{};
    mixer.x = b->qkv_proj;
    mixer.ldx = cd;
    mixer.conv_w = w->conv;
    mixer.conv_state = conv_state;
    mixer.conv_snap = K > 1 && !verify ? conv_snap : nullptr;
    mixer.y = b->conv_out;
    mixer.ldy = cd;
    mixer.fa = b->fa;
    mixer.ga = b->ga;
    mixer.lr_part = part;
    mixer.ks = split ? ks : 1;
    mixer.b_raw = b->b_raw;
    mixer.f_b = w->f_b;
    mixer.g_b = w->g_b;
    mixer.a_log = w->a_log;
    mixer.dt_bias = w->dt_bias;
    mixer.g_raw = b->g_raw;
    mixer.gate = b->gate;
    mixer.beta = b->beta;
    mixer.state = state;
    mixer.snap = K > 1 && !verify ? snap : nullptr;
    mixer.wy = wy;
    mixer.core = b->core;
    mixer.out_gate = b->out_gate;
    mixer.norm_w = w->o_norm;
    mixer.out = b->o_norm_out;
    mixer.K = K;
    mixer.H = heads;
    mixer.R = rank;
    mixer.scale = scale;
    mixer.eps_l2 = eps_l2;
    mixer.eps_rms = eps_rms;
    mixer.write_state = !verify;
    // o_proj's weight, [hidden, H*D], read while the mixer runs
    mixer.warm_w = w->o_proj;
    mixer.warm_bytes = (int64_t)hidden_size * qkv * 2;
    mixer.warm_tile_bytes = (int64_t)16 * qkv * 2;
    mixer.warm_sleeps = 4;
    int rc;
    if ((rc = hip_status(kda::launch_gemv_bf16_batchm(front, 6, Mi, stream),
                         "kda_block_decode_k: front projections launch")) ||
        (rc = hip_status(fuse_mixer || !split
                             ? hipSuccess
                             : kda::launch_lowrank_finish(part, ks, Mi, rk, heads, b->fa, b->ga,
                                                          b->b_raw, b->beta, stream),
                         "kda_block_decode_k: low-rank finish launch")) ||
        (rc = hip_status(fuse_mixer ? hipSuccess : kda::launch_gemv_bf16_batchm(mid, 2, Mi, stream),
                         "kda_block_decode_k: low-rank projections launch")) ||
        (rc = hip_status(
             fuse_mixer ? kda::launch_kda_mixer(mixer, B, head_dim, stream)
                        : kda::launch_conv_silu_l2(b->qkv_proj, cd, w->conv, conv_state,
                                                   mixer.conv_snap, B, K, heads, head_dim, eps_l2,
                                                   b->conv_out, cd, nullptr, nullptr, nullptr,
                                                   stream, !verify),
             "kda_block_decode_k: conv launch")) ||
        (rc = hip_status(fuse_mixer ? hipSuccess
                         : verify ? (wy ? kda::launch_kda_verify_wy(b->conv_out, cd, b->gate,
                                                                    b->beta, state, wy, b->core, B,
                                                                    K, heads, head_dim, scale,
                                                                    stream)
                                        : kda::launch_kda_verify(b->conv_out, cd, b->gate, b->beta,
                                                                 state, b->core, B, K, heads,
                                                                 head_dim, scale, stream))
                                  : kda::launch_kda_recurrent(b->conv_out, cd, b->gate, b->beta,
                                                              state, mixer.snap, b->core, B, K,
                                                              heads, head_dim, scale, stream),
                         "kda_block_decode_k: recurrent launch")) ||
        (rc = hip_status(fuse_mixer ? hipSuccess
                                    : kda::launch_gated_rmsnorm(b->core, qkv, b->out_gate, qkv,
                                                                w->o_norm, Mi, heads, head_dim,
                                                                eps_rms, b->o_norm_out, qkv, stream),
                         "kda_block_decode_k: gated_rmsnorm launch")) ||
        (rc = hip_status(kda::launch_gemv_bf16_batchm(back, 1, Mi, stream),
                         "kda_block_decode_k: o_proj launch")))
        return rc;
    return ok();
}

int kda_block_decode_k(const uint16_t *hidden, const kda_block_weights *w, float *const *state,
                       uint16_t *const *conv_state, float *const *snap,
                       uint16_t *const *conv_snap, const kda_block_decode_buffers *b,
                       uint16_t *out, int32_t B, int32_t K, int32_t hidden_size, int32_t heads,
                       int32_t head_dim, int32_t rank, float scale, float eps_l2, float eps_rms,
                       hipStream_t stream)
{
    return block_decode_run(hidden, w, state, conv_state, snap, conv_snap, b, out, B, K,
                            hidden_size, heads, head_dim, rank, scale, eps_l2, eps_rms, false,
                            stream);
}

int kda_block_verify_k(const uint16_t *hidden, const kda_block_weights *w, float *const *state,
                       uint16_t *const *conv_state, const kda_block_decode_buffers *b,
                       uint16_t *out, int32_t B, int32_t K, int32_t hidden_size, int32_t heads,
                       int32_t head_dim, int32_t rank, float scale, float eps_l2, float eps_rms,
                       hipStream_t stream)
{
    return block_decode_run(hidden, w, state, conv_state, nullptr, nullptr, b, out, B, K,
                            hidden_size, heads, head_dim, rank, scale, eps_l2, eps_rms, true,
                            stream);
}

int kda_block_verify_wy_k(const uint16_t *hidden, const kda_block_weights *w, float *const *state,
                          uint16_t *const *conv_state, float *const *wy,
                          const kda_block_decode_buffers *b, uint16_t *out, int32_t B, int32_t K,
                          int32_t hidden_size, int32_t heads, int32_t head_dim, int32_t rank,
                          float scale, float eps_l2, float eps_rms, hipStream_t stream)
{
    if (B > 0 && K > 0 && !wy)
        return fail(KDA_ERR_NULL, "kda_block_verify_wy_k: null pointer argument");
    if (wy && ((const void *)wy == (const void *)state || (const void *)wy == (const void *)conv_state))
        return fail(KDA_ERR_ALIAS, "kda_block_verify_wy_k: table of u rows is a state table");
    return block_decode_run(hidden, w, state, conv_state, nullptr, nullptr, b, out, B, K,
                            hidden_size, heads, head_dim, rank, scale, eps_l2, eps_rms, true,
                            stream, wy);
}

int kda_block_fold_wy(const kda_block_decode_buffers *b, float *const *state,
                      uint16_t *const *conv_state, float *const *wy, const int32_t *n_accept,
                      int32_t B, int32_t K, int32_t heads, int32_t head_dim, int32_t *status,
                      hipStream_t stream)
{
    if (B < 0 || K < 0 || heads <= 0 || (int64_t)B * K > (1 << 24) || B > kMaxGridYZ)
        return fail(KDA_ERR_SHAPE, "kda_block_fold_wy: B=%d K=%d heads=%d", B, K, heads);
    if (!head_dim_ok(head_dim))
        return fail(KDA_ERR_UNSUPPORTED, "kda_block_fold_wy: head_dim=%d", head_dim);
    if (B == 0 || K == 0) return ok();
    if (!b || !state || !conv_state || !wy || !n_accept || !b->qkv_proj || !b->conv_out ||
        !b->gate)
        return fail(KDA_ERR_NULL, "kda_block_fold_wy: null pointer argument");
    if (!aligned16(b->qkv_proj) || !aligned16(b->conv_out) || !aligned16(b->gate) ||
        (status && !aligned4(status)))
        return fail(KDA_ERR_SHAPE, "kda_block_fold_wy: misaligned buffer");
    if ((const void *)wy == (const void *)state || (const void *)wy == (const void *)conv_state)
        return fail(KDA_ERR_ALIAS, "kda_block_fold_wy: table of u rows is a state table");
    const int64_t cd = 3LL * heads * head_dim;
    int rc;
    if ((rc = hip_status(kda::launch_kda_fold_wy(b->conv_out, cd, b->gate, state, wy, n_accept, B,
                                                 K, heads, head_dim, status, stream),
                         "kda_block_fold_wy: state fold launch")) ||
        (rc = hip_status(kda::launch_conv_fold(b->qkv_proj, cd, conv_state, n_accept, B, K, heads,
                                               head_dim, stream),
                         "kda_block_fold_wy: conv fold launch")))
        return rc;
    return ok();
}

int kda_block_fold_accepted(const kda_block_decode_buffers *b, float *const *state,
                            uint16_t *const *conv_state, const int32_t *n_accept, int32_t B,
                            int32_t K, int32_t heads, int32_t head_dim, int32_t *status,
                            hipStream_t stream)
{
    if (B < 0 || K < 0 || heads <= 0 || (int64_t)B * K > (1 << 24) || B > kMaxGridYZ)
        return fail(KDA_ERR_SHAPE, "kda_block_fold_accepted: B=%d K=%d heads=%d", B, K, heads);
    if (!head_dim_ok(head_dim))
        return fail(KDA_ERR_UNSUPPORTED, "kda_block_fold_accepted: head_dim=%d", head_dim);
    if (B == 0 || K == 0) return ok();
    if (!b || !state || !conv_state || !n_accept || !b->qkv_proj || !b->conv_out || !b->gate ||
        !b->beta)
        return fail(KDA_ERR_NULL, "kda_block_fold_accepted: null pointer argument");
    if (!aligned16(b->qkv_proj) || !aligned16(b->conv_out) || !aligned16(b->gate) ||
        (status && !aligned4(status)))
        return fail(KDA_ERR_SHAPE, "kda_block_fold_accepted: misaligned buffer");
    const int64_t cd = 3LL * heads * head_dim;
    int rc;
    if ((rc = hip_status(kda::launch_kda_fold(b->conv_out, cd, b->gate, b->beta, state, n_accept,
                                              B, K, heads, head_dim, status, stream),
                         "kda_block_fold_accepted: state fold launch")) ||
        (rc = hip_status(kda::launch_conv_fold(b->qkv_proj, cd, conv_state, n_accept, B, K, heads,
                                               head_dim, stream),
                         "kda_block_fold_accepted: conv fold launch")))
        return rc;
    return ok();
}

int kda_block_decode(const uint16_t *hidden, const kda_block_weights *w, float *const *state,
                     uint16_t *const *conv_state, const kda_block_decode_buffers *b,
                     uint16_t *out, int32_t B, int32_t hidden_size, int32_t heads,
                     int32_t head_dim, int32_t rank, float scale, float eps_l2, float eps_rms,
                     hipStream_t stream)
{
    return kda_block_decode_k(hidden, w, state, conv_state, nullptr, nullptr, b, out, B, 1,
                              hidden_size, heads, head_dim, rank, scale, eps_l2, eps_rms, stream);
}

}  // extern "C"
