/*
 * libkda — Kimi-Delta-Attention (KDA) core for AMD MI355X (gfx950).
 *
 * C ABI.  Every entry point:
 *   - takes DEVICE pointers owned by the caller (the library allocates
 *     nothing and keeps no pointer after returning);
 *   - enqueues its kernels on `stream` and returns without synchronising
 *     (stream-ordered, like any HIP launch);
 *   - returns KDA_OK (0) or a negative kda_status; on error nothing has been
 *     enqueued and kda_last_error() gives a message (thread-local);
 *   - never writes outside the rows and buffers it documents.
 *
 * Types: bf16 values travel as uint16_t bit patterns; fp32 as float.  Row
 * strides (`ld*`) are in ELEMENTS and must be multiples of 8 for bf16 rows and
 * of 4 for fp32 rows; base pointers must be 16-byte aligned.  Channel
 * c = h*head_dim + d everywhere.  Supported: head_dim in {16, 128}, prefill
 * chunk in {16, 64}, conv kernel width 4.
 *
 * Cited passages are from the four API pages of the documented engine:
 * "Glm5NextKdaWorkspace" (the buffer contract), "Glm5NextKdaLayer" (decode,
 * decode_k, prefill, prefill_with_pad_fill), "Glm5NextLayer" (engine traits)
 * and "Glm5NextKdaWeights" (the weights).
 */
#ifndef KDA_H
#define KDA_H
/* Launch-grid limits, reported as KDA_ERR_SHAPE: a batch B of sequences
 * (decode paths, conv n_seq, block decode) at most 65535, and at most
 * 65535 x 16 rows per sequence in conv_silu_l2. */

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kda_status {
    KDA_OK = 0,
    KDA_ERR_NULL = -1,        /* a required pointer is NULL                      */
    KDA_ERR_SHAPE = -2,       /* negative size, T_pad < T, T_pad % chunk != 0,
                                 bad stride or misaligned pointer                */
    KDA_ERR_UNSUPPORTED = -3, /* head_dim, chunk or conv width not built         */
    KDA_ERR_ALIAS = -4,       /* an output aliases an input it must not          */
    KDA_ERR_WORKSPACE = -5,   /* workspace smaller than kda_prefill_workspace_bytes */
    KDA_ERR_HIP = -6          /* the HIP runtime rejected a launch               */
} kda_status;

/* Message for the last non-zero status returned on this thread ("" if none). */
const char *kda_last_error(void);

/* Run-time report bits.  A few calls take their sizes from device memory
 * (cu_seqlens, n_accept), which the host cannot check before the launch.
 * Such a call takes an optional `status` argument: a device int32 word that
 * the kernels OR these bits into when they meet a value they had to clamp or
 * a sequence they had to skip.  The library never clears the word (the
 * caller zeroes it and reads it when it likes), so one word can collect the
 * reports of many calls; NULL turns the report off.  The results of a call
 * whose report is 0 are exactly as documented. */
#define KDA_REPORT_SEQ_SKIPPED 1     /* a sequence's chunks exceed max_chunks or
                                        total_chunks: it was left untouched      */
#define KDA_REPORT_ROWS_CLAMPED 2    /* cu_seqlens decreasing, negative or past
                                        rows: the offsets were clamped           */
#define KDA_REPORT_ACCEPT_CLAMPED 4  /* an n_accept outside [0, K] was clamped   */

/* ------------------------------------------------------------------------
 * conv_silu_l2 — short causal depthwise conv + SiLU + per-head L2 of q and k.
 * "Glm5NextKdaWorkspace" page, fields qkv_proj and conv_out (conv + SiLU with
 * q|k L2-normalised, fused on decode); "Glm5NextKdaWeights" page, field conv
 * ([conv_dim, conv_kernel] depthwise weight); "Glm5NextKdaLayer" page, decode
 * and decode_k (the conv state is carried, snapshots after each row).
 *
 * n_seq sequences of `rows` rows each, sequence-major:
 *   x          bf16 [n_seq*rows, conv_dim] (row stride ldx), conv_dim =
 *              3*heads*head_dim, channels q|k|v.
 *   w          bf16 [conv_dim, kc]; tap kc-1 multiplies the current row.
 *   conv_state device array [n_seq] of pointers to bf16 [kc, conv_dim]: the
 *              last kc pre-conv rows, newest last.  In/out: on return it holds
 *              the window after the sequence's last row.
 *   conv_snap  NULL, or a device array [n_seq*(rows-1)] of pointers to bf16
 *              [kc, conv_dim]; entry s*(rows-1)+t receives the window after
 *              row t of sequence s (t < rows-1).
 *   y          bf16 [n_seq*rows, conv_dim] (row stride ldy): SiLU(conv), with
 *              each head of the q and k sections divided by
 *              sqrt(sum of squares + eps_l2), rounded once to bf16.
 *   q32,k32,v32 NULL (all three) or fp32 [n_seq*rows, heads*head_dim] each:
 *              the q, k, v sections of y widened exactly ("Glm5NextKdaWorkspace"
 *              page, field q_f32).  Rows past n_seq*rows are not touched.
 * y must not alias x (KDA_ERR_ALIAS).  rows == 0 or n_seq == 0 is a no-op.
 * ------------------------------------------------------------------------ */
int conv_silu_l2(const uint16_t *x, int64_t ldx, const uint16_t *w,
                 uint16_t *const *conv_state, uint16_t *const *conv_snap,
                 int32_t n_seq, int32_t rows, int32_t heads, int32_t head_dim,
                 int32_t kc, float eps_l2, uint16_t *y, int64_t ldy,
                 float *q32, float *k32, float *v32, hipStream_t stream);

/* ------------------------------------------------------------------------
 * kda_gate — bounded per-channel log-decay and beta.
 * "Glm5NextKdaWorkspace" page, fields g_raw, gate and beta; "Glm5NextKdaWeights"
 * page, fields a_log ([heads], per head) and dt_bias ([heads*head_dim], per
 * channel).
 *   g_raw   bf16 [T, heads*head_dim] (row stride ldg)
 *   b_raw   bf16 [T, heads] (row stride ldb, b_proj output) or NULL
 *   gate    fp32 [T_pad, heads, head_dim]: for t < T,
 *           gate[t,h,d] = -exp(a_log[h]) * softplus(g_raw[t,h*D+d] + dt_bias[h*D+d]),
 *           softplus(z) = log(1+e^z), z for z > 20.  exp(gate) is in (0, 1].
 *   beta    fp32 [T_pad, heads]: beta[t,h] = 1/(1+exp(-b_raw[t,h])); not touched
 *           when b_raw is NULL (then beta may be NULL).
 * Rows t >= T of gate/beta are not touched.  T == 0 is a no-op; T above 2^24
 * returns KDA_ERR_SHAPE.
 * ------------------------------------------------------------------------ */
int kda_gate(const uint16_t *g_raw, int64_t ldg, const uint16_t *b_raw,
             int64_t ldb, const float *a_log, const float *dt_bias, int32_t T,
             int32_t heads, int32_t head_dim, float *gate, float *beta,
             hipStream_t stream);

/* ------------------------------------------------------------------------
 * kda_prefill — chunked prefill of the KDA recurrence from a carried state.
 * "Glm5NextKdaLayer" page, prefill (chunked prefill over t tokens from the
 * carried state) and prefill_with_pad_fill (the chunk kernels guard past T:
 * the padded tail may hold anything); "Glm5NextKdaWorkspace" page, fields
 * q_f32/k_f32/v_f32, gate, beta, core (shapes; buffers padded to whole chunks).
 *
 * Per head, with S[i][j] (i = key channel, j = value channel), each token t:
 *   S <- diag(exp(gate_t)) S;  u = beta_t (v_t - S^T k_t);  S <- S + k_t u^T;
 *   core_t = scale * S^T q_t.
 * q and k are used as given (pre-normalised contract, no re-normalisation).
 *   q,k,v,gate fp32 [T_pad, heads, head_dim]; beta fp32 [T_pad, heads].
 *   state      fp32 [heads, head_dim, head_dim], in/out (updated in place).
 *   core       fp32 [T_pad, heads, head_dim]; rows t < T written, rows >= T
 *              not touched.
 *   Rows t >= T of every input are never used: any bits (0, 1e30, NaN) give
 *   bitwise the same core rows < T and state.  T_pad % chunk == 0, T_pad >= T.
 *   workspace  device scratch of at least kda_prefill_workspace_bytes(...)
 *              bytes, 256-byte aligned; contents on return are unspecified.
 * core must not alias an input or state (KDA_ERR_ALIAS).  T == 0 is a no-op.
 *
 * kda_prefill runs the two phases below over consecutive segments of
 * kda_prefill_segment_chunks(...) chunks (prepare, then forward, per segment,
 * each segment reusing the start of the workspace), so the operand blocks of
 * a segment are still in the last-level cache when the forward phase reads
 * them.  The result is bitwise that of one prepare + forward over all rows.
 * ------------------------------------------------------------------------ */
size_t kda_prefill_workspace_bytes(int32_t T_pad, int32_t heads,
                                   int32_t head_dim, int32_t chunk);

/* Chunks per segment of kda_prefill for T tokens (at least 1; 0 on invalid
 * heads/head_dim/chunk): the number of segments is the workspace of all
 * ceil(T/chunk) chunks divided by a 160 MiB cache budget, rounded up, and
 * the chunks are spread evenly over them. */
int32_t kda_prefill_segment_chunks(int32_t T, int32_t heads, int32_t head_dim,
                                   int32_t chunk);

/* Workspace bytes of kda_prefill_varlen over B sequences of total_chunks
 * chunks: the operand blocks of kda_prefill_workspace_bytes(total_chunks *
 * chunk, ...) followed by the call's sequence tables, (total_chunks + 3B + 1)
 * int32 rounded up to 256 bytes, which a one-workgroup kernel fills from
 * cu_seqlens at the start of the call so that every later launch of the call
 * is sized by its segment and finds a workgroup's sequence in a few table
 * reads.  0 on invalid arguments (B outside [0, 65535], total_chunks < 0,
 * total_chunks * chunk above 2^30, heads <= 0, chunk not 16 or 64). */
size_t kda_prefill_varlen_workspace_bytes(int32_t B, int32_t total_chunks,
                                          int32_t heads, int32_t head_dim,
                                          int32_t chunk);

int kda_prefill(const float *q, const float *k, const float *v,
                const float *gate, const float *beta, float *state, float *core,
                int32_t T, int32_t T_pad, int32_t heads, int32_t head_dim,
                int32_t chunk, float scale, void *workspace,
                size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * kda_prefill_noalloc — kda_prefill for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments as kda_prefill without the workspace;
 * the result is bitwise that of kda_prefill.
 *   The operand blocks go to a library-held device array of
 *   KDA_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU, which each GPU the library
 *   runs on holds until the process ends; the call itself allocates nothing
 *   (no hipMalloc, no hipFree, no allocating library routine) and walks the
 *   sequence in segments of as many chunks as the array holds.
 *   Every call on one GPU shares that GPU's array: calls whose work overlaps
 *   in time (different streams, or host threads with no ordering between
 *   them) race on it and give undefined results; order them (one stream, or
 *   events).  The array keeps the last call's contents; nothing in it needs
 *   to start at zero.
 *   Errors as kda_prefill; KDA_ERR_WORKSPACE when one chunk of all heads,
 *   heads * (4*chunk*head_dim + chunk*chunk + head_dim) * 4 bytes, exceeds
 *   the array; KDA_ERR_HIP when the array's address cannot be looked up.
 * ------------------------------------------------------------------------ */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int kda_prefill_noalloc(const float *q, const float *k, const float *v,
                        const float *gate, const float *beta, float *state, float *core,
                        int32_t T, int32_t T_pad, int32_t heads, int32_t head_dim,
                        int32_t chunk, float scale, hipStream_t stream);

/* ------------------------------------------------------------------------
 * kda_prefill_prepare / kda_prefill_forward — the two phases of kda_prefill,
 * callable separately ("Glm5NextLayer" page, split-prefill section: a batched
 * linear-attention prefill runs its phases as separate steps).  Calling
 * prepare then forward on one stream with the same T, T_pad, heads,
 * head_dim, chunk and workspace gives bitwise the same result as kda_prefill.
 *   prepare: reads q, k, v, gate, beta (rows < T) and writes, per chunk and
 *            head, every operand of the chunk-state walk into the workspace
 *            (the UT-transformed keys and values, decayed queries and keys,
 *            the decayed query-key scores, the chunk decay).  It reads no
 *            state: it may run before the carried state is known.
 *   forward: reads only the workspace and the carried state; walks the
 *            chunks in order; writes core rows < T and the final state.
 * Arguments, layouts and errors are those of kda_prefill.
 * ------------------------------------------------------------------------ */
int kda_prefill_prepare(const float *q, const float *k, const float *v,
                        const float *gate, const float *beta, int32_t T,
                        int32_t T_pad, int32_t heads, int32_t head_dim,
                        int32_t chunk, void *workspace, size_t workspace_bytes,
                        hipStream_t stream);

int kda_prefill_forward(float *state, float *core, int32_t T, int32_t T_pad,
                        int32_t heads, int32_t head_dim, int32_t chunk,
                        float scale, const void *workspace,
                        size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * kda_prefill_bf16 — kda_prefill reading q, k and v straight from the bf16
 * conv output rows.  "Glm5NextKdaWorkspace" page: conv_out holds q | k | v
 * in bf16 and the prefill's q_f32 copies are its exact widening, so reading
 * conv_out directly gives bitwise the result of kda_prefill on those copies
 * without writing or reading them.
 *   qkv    bf16 [T_pad, ldqkv] rows: q at column 0, k at heads*head_dim, v at
 *          2*heads*head_dim (ldqkv >= 3*heads*head_dim, ldqkv % 4 == 0,
 *          8-byte aligned); rows >= T may hold anything.
 *   gate, beta, state, core, workspace and every other argument: as
 *   kda_prefill.
 * ------------------------------------------------------------------------ */
int kda_prefill_bf16(const uint16_t *qkv, int64_t ldqkv, const float *gate,
                     const float *beta, float *state, float *core, int32_t T,
                     int32_t T_pad, int32_t heads, int32_t head_dim, int32_t chunk,
                     float scale, void *workspace, size_t workspace_bytes,
                     hipStream_t stream);

/* ------------------------------------------------------------------------
 * kda_prefill_split — one prefill pass split at row cap, with the state at
 * the split captured.  "Glm5NextLayer" page, supports_replay_tail_split: the
 * rows from cap on get exactly the bits a prefill starting at cap gives them
 * (the linear-attention layer splits its recurrence there and copies its
 * state into the plan's slot).
 *   Rows [0, cap) are prefilled from *state on chunks starting at row 0; the
 *   state after row cap-1 is copied to cap_state (fp32 [heads, head_dim,
 *   head_dim], caller-owned); rows [cap, T) are prefilled from that state on
 *   chunks starting at row cap.  Bitwise the same as kda_prefill over
 *   [0, cap) followed by kda_prefill over [cap, T).
 * Arguments and errors as kda_prefill, plus: 0 <= cap <= T; T_pad at least
 * cap + round_up(T - cap, chunk) (the tail's last chunk must exist; rows
 * past T may hold anything); cap_state 16-byte aligned and disjoint from
 * the inputs, state, core and workspace (KDA_ERR_ALIAS).  T == 0 is a no-op.
 * ------------------------------------------------------------------------ */
int kda_prefill_split(const float *q, const float *k, const float *v,
                      const float *gate, const float *beta, float *state, float *core,
                      float *cap_state, int32_t T, int32_t cap, int32_t T_pad,
                      int32_t heads, int32_t head_dim, int32_t chunk, float scale,
                      void *workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * kda_prefill_varlen — chunked prefill of B sequences in one call, each from
 * its own carried state.  "Glm5NextLayer" page, batched linear-attention
 * prefill (prefill_gdn_full_batched / ..._varlen): one state pointer per
 * sequence in a device table, the sequences' tokens back to back in the
 * stage buffers, row offsets in a device cu_seqlens array, the longest
 * sequence's chunk count and the total chunk count passed alongside.
 *   q, k, v, gate fp32 [rows, heads, head_dim]; beta fp32 [rows, heads]:
 *          sequence s owns rows [cu_seqlens[s], cu_seqlens[s+1]); rows past
 *          the last sequence may hold anything.
 *   state  device array [B] of pointers to fp32 [heads, head_dim, head_dim],
 *          in/out; entries must be distinct.
 *   core   fp32 [rows, heads, head_dim]: rows of each sequence written,
 *          other rows untouched.
 *   cu_seqlens  device int32 [B+1], non-decreasing, cu_seqlens[B] <= rows.
 *   max_chunks  max over s of ceil(len_s / chunk);
 *   total_chunks sum over s of ceil(len_s / chunk);
 *   workspace   at least kda_prefill_varlen_workspace_bytes(B, total_chunks,
 *               heads, head_dim, chunk) bytes, 256-byte aligned.
 * Each sequence's core rows and final state are bitwise those of a
 * kda_prefill call on that sequence alone (the chunk arithmetic is the same;
 * a chunk's rows past its sequence's end are pad rows to it).  The lengths
 * live in device memory, so the host checks only the sizes it is given; a
 * sequence whose chunks would fall outside max_chunks or total_chunks is
 * skipped (its state and core rows are left as they are), never written
 * past the workspace.  Rows are clamped to [0, rows).  B == 0 or
 * total_chunks == 0 is a no-op.  Errors as kda_prefill; B and max_chunks at
 * most 65535.
 *   status      optional device int32 word (NULL: no report): gets
 *               KDA_REPORT_SEQ_SKIPPED when a sequence was skipped as above
 *               and KDA_REPORT_ROWS_CLAMPED when an offset was clamped; both
 *               are the "default returns an error" of the page's batched
 *               prefill turned into a report, since the lengths are only
 *               known on the device.
 * ------------------------------------------------------------------------ */
int kda_prefill_varlen(const float *q, const float *k, const float *v,
                       const float *gate, const float *beta, float *const *state,
                       float *core, const int32_t *cu_seqlens, int32_t B,
                       int32_t rows, int32_t max_chunks, int32_t total_chunks,
                       int32_t heads, int32_t head_dim, int32_t chunk, float scale,
                       void *workspace, size_t workspace_bytes, int32_t *status,
                       hipStream_t stream);

/* ------------------------------------------------------------------------
 * kda_decode — one token for each of B independent sequences.
 * "Glm5NextKdaLayer" page, decode (single-token decode; q/k arrive already
 * normalised from the fused conv and must not be re-normalised; the state is
 * updated in place).  Same step as kda_prefill, one row.
 *   qkv    bf16 [B, 3*heads*head_dim] (row stride ldqkv): the conv_out rows,
 *          q | k | v sections.
 *   gate   fp32 [B, heads, head_dim]; beta fp32 [B, heads].
 *   state  device array [B] of pointers to fp32 [heads, head_dim, head_dim],
 *          in/out.  Entries must be distinct.
 *   core   fp32 [B, heads, head_dim].
 * B == 0 is a no-op.
 * ------------------------------------------------------------------------ */
int kda_decode(const uint16_t *qkv, int64_t ldqkv, const float *gate,
               const float *beta, float *const *state, float *core, int32_t B,
               int32_t heads, int32_t head_dim, float scale, hipStream_t stream);

/* ------------------------------------------------------------------------
 * kda_decode_k — K consecutive tokens of each of B sequences (speculative
 * verify), with the state after every row but the last copied out.
 * "Glm5NextKdaLayer" page, decode_k: the recurrence walks one token at a
 * time exactly as decode does and the result is bit-identical to K serial
 * kda_decode calls; snapshots[t] receives the state AFTER row t, K-1 of them
 * or none.
 *   qkv    bf16 [B*K, 3*heads*head_dim], sequence-major (row b*K + t).
 *   gate   fp32 [B*K, heads, head_dim]; beta fp32 [B*K, heads].
 *   state  device array [B] of pointers to fp32 [heads, head_dim, head_dim],
 *          in/out: on return the state after row K-1.
 *   snap   NULL or device array [B*(K-1)] of pointers to fp32
 *          [heads, head_dim, head_dim]; entry b*(K-1)+t = state after row t.
 *          Snapshot buffers must not overlap any state.
 *   core   fp32 [B*K, heads, head_dim].
 * B == 0 or K == 0 is a no-op.
 * ------------------------------------------------------------------------ */
int kda_decode_k(const uint16_t *qkv, int64_t ldqkv, const float *gate,
                 const float *beta, float *const *state, float *const *snap,
                 float *core, int32_t B, int32_t K, int32_t heads,
                 int32_t head_dim, float scale, hipStream_t stream);

/* ------------------------------------------------------------------------
 * kda_verify_k / kda_fold_accepted — write-on-accept form of decode_k.
 * "Glm5NextLayer" page, LayerWriteOnAccept: the verify produces the K rows'
 * outputs without writing the state, and once the number of accepted rows of
 * each sequence is known, gdn_fold_accepted folds those rows into the state
 * (na_tab: a device array of accepted row counts in batch order).  Against
 * kda_decode_k with K-1 snapshots this moves each sequence's state 3 times
 * (read, then read and write) instead of K+1 times.
 *
 * kda_verify_k: arguments as kda_decode_k without snapshots; core rows are
 *   bitwise those of kda_decode_k; every state is left unchanged.
 * kda_fold_accepted: qkv, gate, beta must hold the same rows the verify read
 *   ([B*K, ...], sequence-major); n_accept device int32 [B], each clamped to
 *   [0, K].  Afterwards *state[b] is bitwise the state kda_decode_k would
 *   have left after row n_accept[b]-1 (its snapshot, or its final state for
 *   n_accept[b] == K); n_accept[b] == 0 leaves it untouched.  Writes no output.
 *   status: optional device int32 word (NULL: no report) that gets
 *   KDA_REPORT_ACCEPT_CLAMPED when some n_accept[b] lay outside [0, K].
 * Errors as kda_decode_k (n_accept required).  B == 0 or K == 0 is a no-op.
 * ------------------------------------------------------------------------ */
int kda_verify_k(const uint16_t *qkv, int64_t ldqkv, const float *gate,
                 const float *beta, float *const *state, float *core, int32_t B,
                 int32_t K, int32_t heads, int32_t head_dim, float scale,
                 hipStream_t stream);

int kda_fold_accepted(const uint16_t *qkv, int64_t ldqkv, const float *gate,
                      const float *beta, float *const *state, const int32_t *n_accept,
                      int32_t B, int32_t K, int32_t heads, int32_t head_dim,
                      int32_t *status, hipStream_t stream);

/* ------------------------------------------------------------------------
 * kda_verify_wy_k / kda_fold_wy — table form of write-on-accept.
 * "Glm5NextLayer" page, LayerWriteOnAccept: gdn_verify_run_batched takes the
 * layer's staged WY tables (wy_tables), and gdn_fold_accepted folds the
 * accepted rows through the layer's WY pointer table (h_table) and the
 * accepted counts (na_tab).
 * The pages do not spell the tables out; here a sequence's table holds, per
 * head and row, the row's delta-rule value u_t = beta_t (v_t - S'^T k_t)
 * (S' the decayed state before row t: the U rows of the rows' WY form), so
 * the fold is one pass of the unrolled recurrence instead of a row-by-row
 * walk:
 *   S_n = diag(e^{g_0 + .. + g_{n-1}}) S_0
 *         + sum_{s<n} diag(e^{g_{s+1} + .. + g_{n-1}}) k_s u_s^T.
 * kda_verify_wy_k: kda_verify_k (core rows bitwise those of kda_decode_k,
 *   states unchanged) that also writes the u rows: wy is a device array [B]
 *   of pointers to fp32 [heads, K, head_dim] (16-byte aligned), row t of
 *   head h at wy[b] + (h*K + t)*head_dim.  wy must not be the state table
 *   (KDA_ERR_ALIAS).
 * kda_fold_wy: qkv and gate hold the rows the verify read (k and the decay
 *   are read again; v, q and beta are not); wy the verify's tables, n_accept
 *   device int32 [B], each clamped to [0, K] and reported as in
 *   kda_fold_accepted.  Afterwards *state[b] is the state after row
 *   n_accept[b]-1 — equal to kda_decode_k's snapshot up to rounding (the
 *   decays are summed from the last accepted row down, each channel's
 *   e^{sum} S_0 first, then one fma per accepted row from the last down),
 *   not bitwise like kda_fold_accepted.
 * Errors as kda_verify_k / kda_fold_accepted.  B == 0 or K == 0 is a no-op.
 * ------------------------------------------------------------------------ */
int kda_verify_wy_k(const uint16_t *qkv, int64_t ldqkv, const float *gate,
                    const float *beta, float *const *state, float *const *wy,
                    float *core, int32_t B, int32_t K, int32_t heads,
                    int32_t head_dim, float scale, hipStream_t stream);

int kda_fold_wy(const uint16_t *qkv, int64_t ldqkv, const float *gate,
                float *const *state, float *const *wy, const int32_t *n_accept,
                int32_t B, int32_t K, int32_t heads, int32_t head_dim,
                int32_t *status, hipStream_t stream);

/* ------------------------------------------------------------------------
 * gated_rmsnorm — sigmoid-gated RMSNorm of the core output, per (token, head).
 * "Glm5NextKdaWorkspace" page, fields core, out_gate and o_norm_out;
 * "Glm5NextKdaWeights" page, field o_norm ([head_dim] bf16).
 *   core     fp32 [T, heads*head_dim] (row stride ldc)
 *   out_gate bf16 [T, heads*head_dim] (row stride ldo)
 *   w        bf16 [head_dim]
 *   out      bf16 [T, heads*head_dim] (row stride ldy):
 *            out = bf16(x / sqrt(mean_d x^2 + eps) * w[d] * sigmoid(out_gate)).
 * out must not alias out_gate or core (KDA_ERR_ALIAS).  T == 0 is a no-op;
 * T above 2^24 returns KDA_ERR_SHAPE.
 * ------------------------------------------------------------------------ */
int gated_rmsnorm(const float *core, int64_t ldc, const uint16_t *out_gate,
                  int64_t ldo, const uint16_t *w, int32_t T, int32_t heads,
                  int32_t head_dim, float eps, uint16_t *out, int64_t ldy,
                  hipStream_t stream);

/* ------------------------------------------------------------------------
 * kda_block_prefill — one whole KDA block over one sequence of T tokens from
 * the carried state ("Glm5NextKdaLayer" page, prefill; stage buffers of the
 * "Glm5NextKdaWorkspace" page; weights of the "Glm5NextKdaWeights" page):
 *
 *   qkv_proj   = [h q_proj^T | h k_proj^T | h v_proj^T]     bf16 projections
 *   conv_out   = conv_silu_l2(qkv_proj) from *conv_state[0] (updated), plus
 *                its fp32 widening q32/k32/v32 when those buffers are given
 *   fa = h f_a^T, g_raw = fa f_b^T, b_raw = h b_proj^T      bf16 projections
 *   gate, beta = kda_gate(g_raw, b_raw, a_log, dt_bias)
 *   core       = kda_prefill_bf16(conv_out, gate, beta) from state (updated),
 *                bitwise kda_prefill on the fp32 widening of conv_out
 *   ga = h g_a^T, out_gate = ga g_b^T                       bf16 projections
 *   o_norm_out = gated_rmsnorm(core, out_gate, o_norm)
 *   out        = o_norm_out o_proj^T                        bf16 [T, hidden]
 *
 * The projections are plain GEMMs (bf16 operands, fp32 accumulation, bf16
 * result) run by the vendor library (hipBLASLt); everything between them is
 * this library's own kernels.  The library keeps one hipBLASLt handle and
 * one algorithm choice per GEMM shape for each device, made on first use;
 * it allocates no device memory of its own per call (the GEMM workspace is
 * gemm_ws, which may be NULL with gemm_ws_bytes 0).
 *
 * Weights (device, caller-owned) are bf16 in torch Linear layout [out, in]:
 *   q_proj, k_proj, v_proj [heads*head_dim, hidden]; conv [3*heads*head_dim, 4];
 *   f_a, g_a [rank, hidden]; f_b, g_b [heads*head_dim, rank];
 *   b_proj [heads, hidden]; o_norm [head_dim]; o_proj [hidden, heads*head_dim];
 *   a_log fp32 [heads]; dt_bias fp32 [heads*head_dim].
 * Buffers (device, caller-owned, rows beyond T left as they are):
 *   qkv_proj, conv_out bf16 [T_pad, 3*heads*head_dim]; core, gate fp32
 *   [T_pad, heads*head_dim]; q32, k32, v32 fp32 [T_pad, heads*head_dim] or
 *   all three NULL (optional copies); beta fp32 [T_pad, heads];
 *   fa, ga bf16 [T_pad, rank]; g_raw, out_gate, o_norm_out bf16
 *   [T_pad, heads*head_dim]; b_raw bf16 [T_pad, heads];
 *   prefill_ws of at least kda_prefill_workspace_bytes(T_pad, ...) bytes.
 * hidden bf16 [T, hidden]; out bf16 [T, hidden]; state fp32 [heads, head_dim,
 * head_dim] in/out; conv_state a device table of one pointer to bf16
 * [4, 3*heads*head_dim] in/out.
 * Every buffer, out, state and the conv state must be pairwise disjoint and
 * disjoint from hidden and the weights (KDA_ERR_ALIAS).  hidden, rank and
 * heads*head_dim must be multiples of 8; chunk 16 or 64 with T_pad % chunk
 * == 0 (KDA_ERR_SHAPE / KDA_ERR_UNSUPPORTED).  A vendor GEMM failure returns
 * KDA_ERR_HIP with its reason in kda_last_error().  T == 0 is a no-op.
 * ------------------------------------------------------------------------ */
typedef struct kda_block_weights {
    const uint16_t *q_proj, *k_proj, *v_proj, *conv;
    const uint16_t *f_a, *f_b;
    const float *dt_bias, *a_log;
    const uint16_t *b_proj, *g_a, *g_b, *o_norm, *o_proj;
} kda_block_weights;

typedef struct kda_block_buffers {
    uint16_t *qkv_proj, *conv_out;
    float *q32, *k32, *v32;
    uint16_t *fa, *g_raw, *b_raw;
    float *gate, *beta, *core;
    uint16_t *ga, *out_gate, *o_norm_out;
    void *prefill_ws;
    size_t prefill_ws_bytes;
    void *gemm_ws;
    size_t gemm_ws_bytes;
} kda_block_buffers;

int kda_block_prefill(const uint16_t *hidden, const kda_block_weights *w, float *state,
                      uint16_t *const *conv_state, const kda_block_buffers *buf,
                      uint16_t *out, int32_t T, int32_t T_pad, int32_t hidden_size,
                      int32_t heads, int32_t head_dim, int32_t rank, int32_t chunk,
                      float scale, float eps_l2, float eps_rms, hipStream_t stream);

/* ------------------------------------------------------------------------
 * dense_gemv_bf16_batchm — y = bf16(x w^T) for a few rows, row-order exact.
 * "Glm5NextKdaLayer" page, decode_k: the weight-heavy projections of K rows
 * run once over all rows (weights read once), and each row's result must be
 * bit-identical to the same row's product computed alone, because an
 * accepted draft token must equal what single-token decode would emit.
 *   x  bf16 [M, Kd] (row stride ldx)
 *   w  bf16 [N, Kd] in torch Linear layout [out, in], contiguous rows
 *   y  bf16 [M, N] (row stride ldy): y[m][n] = bf16(sum_k x[m][k] w[n][k]),
 *      fp32 accumulation in an order fixed by (n, k) alone — not by M, not by
 *      the row's position among the M rows.  Rounding to nearest, ties to even.
 * Kd % 32 == 0, ldx % 8 == 0, ldx <= 2^22, N >= 1, M <= 65535 * 64; x, w, y
 * 16-byte aligned (KDA_ERR_SHAPE).  y must not overlap x or w (KDA_ERR_ALIAS).  M == 0 is a
 * no-op.  Meant for small M (up to a few hundred rows); each 64 rows re-read
 * the weights.
 * ------------------------------------------------------------------------ */
int dense_gemv_bf16_batchm(const uint16_t *x, int64_t ldx, const uint16_t *w,
                           int32_t M, int32_t N, int32_t Kd, uint16_t *y,
                           int64_t ldy, hipStream_t stream);

/* ------------------------------------------------------------------------
 * kda_block_decode_k — K consecutive tokens of each of B sequences through a
 * whole KDA block ("Glm5NextKdaLayer" page, decode_k: the projections run
 * once over all B*K rows, the recurrence walks one token at a time; result
 * bit-identical to K serial kda_block_decode calls, snapshots[t] = the
 * recurrent state and the conv state AFTER row t, K-1 of them or none).
 * Per row, the stages of kda_block_prefill:
 *
 *   qkv_proj   = [h q_proj^T | h k_proj^T | h v_proj^T]   dense_gemv_bf16_batchm
 *   fa = h f_a^T, ga = h g_a^T, b_raw = h b_proj^T        (same launch;
 *                beta = sigmoid(b_raw) formed as b_raw is stored)
 *   g_raw = fa f_b^T, out_gate = ga g_b^T                  dense_gemv_bf16_batchm
 *                (gate = kda_gate's log-decay of g_raw formed as it is stored)
 *   conv_out   = conv_silu_l2 row by row from *conv_state[b] (updated)
 *   core       = kda_decode_k(conv_out, gate, beta) from *state[b] (updated)
 *   o_norm_out = gated_rmsnorm(core, out_gate, o_norm)
 *   out        = o_norm_out o_proj^T                       dense_gemv_bf16_batchm
 *
 * hidden bf16 [B*K, hidden], sequence-major (row b*K + t); out bf16
 * [B*K, hidden].  Weights as kda_block_prefill.  state: device array [B] of
 * pointers to fp32 [heads, head_dim, head_dim]; conv_state: device array [B]
 * of pointers to bf16 [4, 3*heads*head_dim]; snap / conv_snap: NULL or device
 * arrays [B*(K-1)] (entry b*(K-1)+t = after row t).  Buffers (caller-owned,
 * B*K rows each): qkv_proj, conv_out bf16 [., 3*heads*head_dim]; fa, ga bf16
 * [., rank]; g_raw, out_gate, o_norm_out bf16 [., heads*head_dim]; b_raw bf16
 * [., heads]; gate, core fp32 [., heads*head_dim]; beta fp32 [., heads].
 * hidden, rank and heads*head_dim must be multiples of 32 and at most 2^22
 * (KDA_ERR_SHAPE);
 * head_dim 16 or 128 (KDA_ERR_UNSUPPORTED).  Buffers, out, hidden and the
 * weights must be pairwise disjoint where one of them is written
 * (KDA_ERR_ALIAS); the per-sequence states are reached through the tables
 * and must be distinct, with snapshots disjoint from them.  B == 0 or K == 0
 * is a no-op.  Allocates nothing; three launches on `stream` when K <= 16
 * and rank <= 128 (the gate products, conv, recurrence and norm of each
 * (head, sequence) in one kernel), six or seven otherwise; the same bits
 * either way.
 * ------------------------------------------------------------------------ */
typedef struct kda_block_decode_buffers {
    uint16_t *qkv_proj, *conv_out;
    uint16_t *fa, *g_raw, *b_raw;
    float *gate, *beta, *core;
    uint16_t *ga, *out_gate, *o_norm_out;
} kda_block_decode_buffers;

int kda_block_decode_k(const uint16_t *hidden, const kda_block_weights *w,
                       float *const *state, uint16_t *const *conv_state,
                       float *const *snap, uint16_t *const *conv_snap,
                       const kda_block_decode_buffers *buf, uint16_t *out, int32_t B,
                       int32_t K, int32_t hidden_size, int32_t heads, int32_t head_dim,
                       int32_t rank, float scale, float eps_l2, float eps_rms,
                       hipStream_t stream);

/* ------------------------------------------------------------------------
 * kda_block_verify_k / kda_block_fold_accepted — write-on-accept form of
 * kda_block_decode_k ("Glm5NextLayer" page, LayerWriteOnAccept: verify
 * without writing the layer's states, then gdn_fold_accepted folds the
 * accepted rows of each sequence into them).
 * kda_block_verify_k: arguments as kda_block_decode_k without snapshots;
 *   every stage buffer and out are bitwise those of kda_block_decode_k; the
 *   recurrent states and conv states are read, never written.
 * kda_block_fold_accepted: buf must hold the verify's stage buffers (its
 *   qkv_proj, conv_out, gate and beta rows are what the fold reads);
 *   n_accept device int32 [B], each clamped to [0, K].  Afterwards *state[b]
 *   and *conv_state[b] are bitwise the recurrent and conv snapshots
 *   kda_block_decode_k would have written after row n_accept[b]-1 (its final
 *   states for n_accept[b] == K); n_accept[b] == 0 leaves both untouched.
 *   Two launches; no output; `status` as kda_fold_accepted.  Errors as
 *   kda_block_decode_k.
 * ------------------------------------------------------------------------ */
int kda_block_verify_k(const uint16_t *hidden, const kda_block_weights *w,
                       float *const *state, uint16_t *const *conv_state,
                       const kda_block_decode_buffers *buf, uint16_t *out, int32_t B,
                       int32_t K, int32_t hidden_size, int32_t heads, int32_t head_dim,
                       int32_t rank, float scale, float eps_l2, float eps_rms,
                       hipStream_t stream);

int kda_block_fold_accepted(const kda_block_decode_buffers *buf, float *const *state,
                            uint16_t *const *conv_state, const int32_t *n_accept, int32_t B,
                            int32_t K, int32_t heads, int32_t head_dim, int32_t *status,
                            hipStream_t stream);

/* ------------------------------------------------------------------------
 * kda_block_verify_wy_k / kda_block_fold_wy — the block's write-on-accept
 * in table form ("Glm5NextLayer" page, LayerWriteOnAccept: the verify with
 * the layer's WY tables, gdn_fold_accepted through the WY pointer table and
 * the accepted counts; the tables as in kda_verify_wy_k).
 * kda_block_verify_wy_k: kda_block_verify_k that also writes the recurrent
 *   rows' u values to wy (a device array [B] of pointers to fp32 [heads, K,
 *   head_dim], 16-byte aligned); out and every stage buffer bitwise those of
 *   kda_block_verify_k; wy must not be a state table (KDA_ERR_ALIAS).
 * kda_block_fold_wy: buf the verify's stage buffers, wy its tables; the
 *   recurrent state as kda_fold_wy (equal to kda_block_decode_k's snapshot
 *   up to rounding), the conv state bitwise as kda_block_fold_accepted.
 *   Two launches; no output; `status` as kda_fold_accepted.
 * Errors as kda_block_verify_k / kda_block_fold_accepted.
 * ------------------------------------------------------------------------ */
int kda_block_verify_wy_k(const uint16_t *hidden, const kda_block_weights *w,
                          float *const *state, uint16_t *const *conv_state,
                          float *const *wy, const kda_block_decode_buffers *buf,
                          uint16_t *out, int32_t B, int32_t K, int32_t hidden_size,
                          int32_t heads, int32_t head_dim, int32_t rank, float scale,
                          float eps_l2, float eps_rms, hipStream_t stream);

int kda_block_fold_wy(const kda_block_decode_buffers *buf, float *const *state,
                      uint16_t *const *conv_state, float *const *wy,
                      const int32_t *n_accept, int32_t B, int32_t K, int32_t heads,
                      int32_t head_dim, int32_t *status, hipStream_t stream);

/* ------------------------------------------------------------------------
 * kda_block_decode — one token for each of B sequences through the whole
 * block ("Glm5NextKdaLayer" page, decode: single-token decode carrying both
 * states, result in out, states updated in place).  Exactly
 * kda_block_decode_k with K = 1 (same kernels, no snapshots).
 * ------------------------------------------------------------------------ */
int kda_block_decode(const uint16_t *hidden, const kda_block_weights *w,
                     float *const *state, uint16_t *const *conv_state,
                     const kda_block_decode_buffers *buf, uint16_t *out, int32_t B,
                     int32_t hidden_size, int32_t heads, int32_t head_dim, int32_t rank,
                     float scale, float eps_l2, float eps_rms, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* KDA_H */
