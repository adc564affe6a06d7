// Host-side launchers, one per kernel family.  Arguments are validated by the
// C entry points (api.cpp) before any launcher runs; launchers only pick the
// template instance and grid, enqueue on `stream`, and return the launch
// status.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

// Run-time report bits (the KDA_REPORT_* values of kda.h) that kernels OR
// into a caller's status word with a vector atomic.
constexpr int32_t kReportSeqSkipped = 1, kReportRowsClamped = 2, kReportAcceptClamped = 4;

// Rows per conv_silu_l2 workgroup tile: a launch's row tiles form grid y,
// so a sequence holds at most 65535 tiles of this many rows.
constexpr int kConvRowsPerTile = 8;

hipError_t launch_conv_silu_l2(const uint16_t *x, int64_t ldx, const uint16_t *w,
                               uint16_t *const *conv_state, uint16_t *const *conv_snap,
                               int n_seq, int rows, int heads, int head_dim, float eps_l2,
                               uint16_t *y, int64_t ldy, float *q32, float *k32, float *v32,
                               hipStream_t stream, bool write_state = true);

// Move each conv window past the first n_accept[b] of its K pre-conv rows x
// (sequence-major [B*K] rows): the write-on-accept fold of the conv state.
hipError_t launch_conv_fold(const uint16_t *x, int64_t ldx, uint16_t *const *conv_state,
                            const int32_t *n_accept, int B, int K, int heads, int head_dim,
                            hipStream_t stream);

hipError_t launch_kda_gate(const uint16_t *g_raw, int64_t ldg, const uint16_t *b_raw,
                           int64_t ldb, const float *a_log, const float *dt_bias, int T,
                           int heads, int head_dim, float *gate, float *beta,
                           hipStream_t stream);

hipError_t launch_gated_rmsnorm(const float *core, int64_t ldc, const uint16_t *out_gate,
                                int64_t ldo, const uint16_t *w, int T, int heads,
                                int head_dim, float eps, uint16_t *out, int64_t ldy,
                                hipStream_t stream);

// K = 1 is single-token decode; the same kernel serves both entry points so
// that K-row decode is bit-identical to K single-row calls.
hipError_t launch_kda_recurrent(const uint16_t *qkv, int64_t ldqkv, const float *gate,
                                const float *beta, float *const *state, float *const *snap,
                                float *core, int B, int K, int heads, int head_dim,
                                float scale, hipStream_t stream);

// Write-on-accept: outputs of K rows with the state left as it is, then the
// first n_accept[b] rows folded into the state (same per-row code as above).
hipError_t launch_kda_verify(const uint16_t *qkv, int64_t ldqkv, const float *gate,
                             const float *beta, float *const *state, float *core, int B, int K,
                             int heads, int head_dim, float scale, hipStream_t stream);
hipError_t launch_kda_fold(const uint16_t *qkv, int64_t ldqkv, const float *gate,
                           const float *beta, float *const *state, const int32_t *n_accept,
                           int B, int K, int heads, int head_dim, int32_t *status,
                           hipStream_t stream);
// Table form: the verify also writes each row's u (the value the row adds to
// the state with its key) to wy[b] fp32 [heads, K, head_dim]; the fold then
// applies the first n_accept[b] rows in one closed-form pass from those rows.
hipError_t launch_kda_verify_wy(const uint16_t *qkv, int64_t ldqkv, const float *gate,
                                const float *beta, float *const *state, float *const *wy,
                                float *core, int B, int K, int heads, int head_dim, float scale,
                                hipStream_t stream);
hipError_t launch_kda_fold_wy(const uint16_t *qkv, int64_t ldqkv, const float *gate,
                              float *const *state, float *const *wy, const int32_t *n_accept,
                              int B, int K, int heads, int head_dim, int32_t *status,
                              hipStream_t stream);

// The block decode's per-head stages in one kernel, one workgroup per
// (head, sequence): the head's columns of the two rank-R products (f_b from fa
// with the log-decay gate in its epilogue, g_b from ga), then for each of the
// K rows conv + SiLU + L2 of the head's q | k | v channels, the recurrence,
// and the gated RMSNorm of its output — the accumulation order of
// dense_gemv_bf16_batchm and the per-row code of conv_silu_l2, kda_recurrent
// and gated_rmsnorm, so every buffer gets the bits those launches would
// write.  write_state false (a verify): neither state is written and no
// snapshots are taken.
constexpr int kMixerMaxRows = 16;    // K of a fused call (its gates are held in LDS)
constexpr int kMixerMaxRank = 128;   // R of a fused call (one contraction step per quarter)
struct MixerArgs {
    const uint16_t *x;              // pre-conv rows [B*K, ldx] (q | k | v)
    int64_t ldx;
    const uint16_t *conv_w;         // [3*H*D, 4]
    uint16_t *const *conv_state;    // per sequence [4, 3*H*D]
    uint16_t *const *conv_snap;     // per (sequence, row < K-1), or nullptr
    uint16_t *y;                    // conv_out rows [B*K, ldy]
    int64_t ldy;
    uint16_t *fa, *ga;              // low-rank inputs [B*K, R] (ks == 1), else written here
    const float *lr_part;           // with ks > 1: the chunk sums of f_a, g_a, b_proj
    int ks;                         // (launch_lowrank_finish's layout)
    uint16_t *b_raw;                // [B*K, H], written when ks > 1
    const uint16_t *f_b, *g_b;      // [H*D, R]
    const float *a_log, *dt_bias;   // [H], [H*D]
    uint16_t *g_raw;                // [B*K, H*D] (f_b product, bf16)
    float *gate;                    // [B*K, H, D] (log-decay gate of g_raw)
    float *beta;                    // [B*K, H] (read; written when ks > 1)
    float *const *state;            // per sequence [H, D, D]
    float *const *snap;             // per (sequence, row < K-1), or nullptr
    float *const *wy;               // per sequence [H, K, D] rows u, or nullptr
    float *core;                    // [B*K, H*D]
    uint16_t *out_gate;             // [B*K, H*D] (g_b product, bf16)
    const uint16_t *norm_w;         // [D]
    uint16_t *out;                  // o_norm_out [B*K, H*D]
    int K, H, R;
    int B;                      // sequences (set by launch_kda_mixer)
    float scale, eps_l2, eps_rms;
    bool write_state;
    // Optional warm-up of the weight that the next launch on the stream
    // streams (a dense_gemv_bf16_batchm operand read in 16-row column tiles,
    // tile t by that launch's workgroup t): the CUs the mixer leaves idle run
    // workgroups of this launch that read one word of every 128-byte line of
    // it, each tile from the XCD (t mod 8 in dispatch order) whose L2 the
    // reading workgroup will use (measured: the lines are then served from
    // the last-level cache, not that L2).  Only reads; no result changes.
    const uint16_t *warm_w;
    int64_t warm_bytes;         // the whole weight
    int64_t warm_tile_bytes;    // one 16-row tile
    int32_t warm_sleeps;        // delay before the reads, in units of 2048 cycles
};
hipError_t launch_kda_mixer(const MixerArgs &a, int B, int head_dim, hipStream_t stream);

size_t prefill_workspace_bytes(int T_pad, int heads, int head_dim, int chunk);
int prefill_segment_chunks(int T, int heads, int head_dim, int chunk);

// phase 1 (per chunk, state-free) and phase 2 (serial over chunks)
hipError_t launch_kda_prefill_prepare(const float *q, const float *k, const float *v,
                                      const float *gate, const float *beta, int T, int heads,
                                      int head_dim, int chunk, void *workspace,
                                      hipStream_t stream);
hipError_t launch_kda_prefill_forward(float *state, float *core, int T, int heads, int head_dim,
                                      int chunk, float scale, const void *workspace,
                                      hipStream_t stream);

hipError_t launch_kda_prefill(const float *q, const float *k, const float *v,
                              const float *gate, const float *beta, float *state,
                              float *core, int T, int heads, int head_dim, int chunk,
                              float scale, void *workspace, hipStream_t stream);

// kda_prefill with a given segment length (seg >= 1 chunks per segment; the
// workspace holds seg chunks' operand blocks): the same bits for every seg.
hipError_t launch_kda_prefill_segments(const float *q, const float *k, const float *v,
                                       const float *gate, const float *beta, float *state,
                                       float *core, int T, int heads, int head_dim, int chunk,
                                       float scale, void *workspace, int seg, hipStream_t stream);

// kda_prefill on the library-held scratch array (kda_noalloc.hip): the
// segment length fitted to the array; returns hipErrorInvalidValue when one
// chunk of all heads does not fit, or the error of the symbol lookup.
constexpr size_t kNoallocScratchBytes = size_t(64) << 20;
hipError_t launch_kda_prefill_noalloc(const float *q, const float *k, const float *v,
                                      const float *gate, const float *beta, float *state,
                                      float *core, int T, int heads, int head_dim, int chunk,
                                      float scale, hipStream_t stream);

// kda_prefill reading q | k | v directly from bf16 rows [T_pad, ldqkv] (the
// conv output; q at column 0, k at heads*head_dim, v at 2*heads*head_dim):
// bitwise the result of kda_prefill on their exact fp32 widening.
hipError_t launch_kda_prefill_bf16(const uint16_t *qkv, int64_t ldqkv, const float *gate,
                                   const float *beta, float *state, float *core, int T,
                                   int heads, int head_dim, int chunk, float scale,
                                   void *workspace, hipStream_t stream);

// Several sequences back to back (rows [cu[s], cu[s+1]) of sequence s), one
// state pointer each; one prepare and one walk for all of them.  total_chunks
// = sum over sequences of ceil(len / chunk) operand blocks in the workspace;
// max_chunks = the longest sequence's chunk count.  Sequences that would not
// fit either are left untouched.  The workspace holds the operand blocks and
// then the call's sequence tables: prefill_varlen_workspace_bytes.
size_t prefill_varlen_workspace_bytes(int B, int total_chunks, int heads, int head_dim, int chunk);
hipError_t launch_kda_prefill_varlen(const float *q, const float *k, const float *v,
                                     const float *gate, const float *beta, float *const *state,
                                     float *core, const int32_t *cu_seqlens, int B, int64_t rows,
                                     int max_chunks, int total_chunks, int heads, int head_dim,
                                     int chunk, float scale, void *workspace, int32_t *status,
                                     hipStream_t stream);

// Row-order-exact bf16 products y = bf16(x w^T) for a few rows (kda_gemv.hip).
// Each segment has its own x [M][Kd] (stride ldx), w [N][Kd] (contiguous
// rows) and y [M][N] (stride ldy); all segments share M.  Kd % 32 == 0, rows
// 16-byte aligned.  Each output element's accumulation order depends on
// neither M nor the row's position.
constexpr int kGemvMaxSegs = 6;
// Epilogue of a segment: the bf16 result only, or also the fp32 activation
// the KDA stages take from it — the log-decay gate (from g_raw, with a_log
// per head of head_dim channels and dt_bias per channel) or beta =
// sigmoid(b_raw) — written to act[m * N + n], exactly as kda_gate forms
// them from the same bf16 values.
enum GemvEpi : int32_t { kEpiNone = 0, kEpiGate = 1, kEpiBeta = 2 };
// A segment may also be split along the contraction into ksplit equal
// chunks (Kd % (32 ksplit) == 0), each a workgroup of its own: chunk c then
// writes its fp32 sum (the chunk's quarters added as usual) to part[(c M + m)
// N + n] instead of y, and the element is split_sum's sum of the chunks in
// order, rounded to bf16 by whoever consumes it.  Small products then spread
// over more workgroups next to large ones in the same launch.
struct GemvSeg {
    const uint16_t *x;
    const uint16_t *w;
    uint16_t *y;
    int64_t ldx, ldy;
    int32_t N, Kd;
    int32_t epi = kEpiNone;
    float *act = nullptr;
    const float *a_log = nullptr, *dt_bias = nullptr;
    int32_t head_dim = 0;
    int32_t ksplit = 1;
    float *part = nullptr;
};
hipError_t launch_gemv_bf16_batchm(const GemvSeg *segs, int nseg, int M, hipStream_t stream);
// A block's f_a, g_a and b_proj products split ks ways (chunk sums in part:
// f_a [ks][M][rank], then g_a alike, then b_proj [ks][M][heads]) finished
// into fa, ga, b_raw and beta.
constexpr int kLowRankSplit = 4;   // contraction chunks of a block's low-rank products
hipError_t launch_lowrank_finish(const float *part, int ks, int M, int rank, int heads,
                                 uint16_t *fa, uint16_t *ga, uint16_t *b_raw, float *beta,
                                 hipStream_t stream);

// y[rows][n_out] (row stride ldy) = bf16(x[rows][n_in] (stride ldx) w^T), w in
// torch Linear layout [n_out][n_in] (stride ldw), fp32 accumulation, on the
// vendor GEMM (kda_gemm.cpp).  Returns 0, or 1 with *what naming the failure.
// y_r[t][0 .. n[r]) = x[t][c[r] .. c[r] + n[r]) for nr <= 3 column ranges of a bf16
// matrix (n[r] multiples of 8; x, y 16-byte aligned, ldx a multiple of 8).
hipError_t launch_split_cols(const uint16_t *x, int64_t ldx, int64_t rows, int nr,
                             uint16_t *const *y, const int *c, const int *n, hipStream_t stream);

int gemm_bf16_xwT(const uint16_t *x, int64_t ldx, const uint16_t *w, int64_t ldw, uint16_t *y,
                  int64_t ldy, int rows, int n_out, int n_in, void *ws, size_t ws_bytes,
                  hipStream_t stream, const char **what);

}  // namespace kda
