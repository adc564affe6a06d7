#!/usr/bin/env python3
"""Benchmark of the KDA core on one MI355X.

Step (the timed unit): one chunked prefill of the KDA core over the workload
T=4096 tokens, 32 heads, head_dim 128, chunk 64, from an fp32 carried state
~ N(0, 0.05), on inputs already resident in HBM: one kda_prefill call (per
segment of kda_prefill_segment_chunks chunks, prepare then forward).
value = T / step time.  Kernel durations for the roofline come from the same
number of steps right after, in the same schedule spelled out phase by phase
with HIP events between the kernels.

Also reported on the same JSON line (measured after the timed steps):
  decode    B=256 sequences x 64 steps, state [256,32,128,128] fp32: state
            read+write bytes / median step time (the metric's second half),
            with the counted HBM traffic of a step;
  decode_k  B=64, K=4 with 3 snapshots per sequence (conv decode-K +
            kda_decode_k), and the write-on-accept pair kda_verify_k +
            kda_fold_accepted on the same rows;
  stages    conv_silu_l2 / kda_gate / gated_rmsnorm at T=8192 (block shapes);
  block     the full KDA block (kda_block_prefill) at T=8192, hidden 4096:
            tokens/s, each stage kernel alone, and the projections' share;
  prefill_bf16_rows  the same prefill with q|k|v as bf16 rows
            (kda_prefill_bf16), checked bitwise against the fp32-input run;
  prefill_varlen  the 4096 tokens as 8 x 512 and 64 x 64 prompts in one
            kda_prefill_varlen call;
  block_decode  the block for one sequence: K=4 verify vs one token (each
            call marshalled once with kda.bind; per call, and per call over
            40 calls back to back), the write-on-accept pair, HIP-graph
            replays, 16 sequences x 4 rows, and the projection kernel's
            weight-read rate;
  roofline  for the dominant prefill kernel, from HIP events on the stream
            the kernels run on, with its counted HBM traffic;
  cpu_baseline  the fp64 oracle on the same prefill workload, and on samples
            of the decode and decode_k workloads, on host cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
       (--prefill-only, --decode-only, --block-only, --block-decode-only,
       --varlen-only and --calibrate-copy serve profiler runs)
"""
import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads  # noqa: E402

METRIC = "KDA prefill tokens/s (H=32,D=128) + decode state HBM GB/s, 1 MI355X"
PEAK_BF16_MFMA = 2.5e15       # MI355X dense bf16 matrix peak, FLOP/s
PEAK_HBM = 8.0e12             # MI355X HBM3E peak, B/s
# HBM bytes per launch (FETCH_SIZE and WRITE_SIZE scaled by the copy
# calibration) from rocprofv3 counter runs of the kernels as they are built
# now; a kernel is left out once it changes after its counters were taken.
TRAFFIC_BYTES = {"kda_chunk_prep": (66872.2 * 2.0 + 143872.0 * 1.0) * 1024,
                 "kda_chunk_fwd": (73053.5 * 2.0 + 34816.0 * 1.0) * 1024}
# Counted HBM traffic of one decode step at 256 sequences (FETCH_SIZE x 2 +
# WRITE_SIZE, KiB per dispatch) for the recurrent kernel as built now.
DECODE_TRAFFIC_BYTES = (267441.6 * 2.0 + 528933.7 * 1.0) * 1024
# Both prefill kernels run each fp32 product as three bf16 products (hi*hi,
# hi*lo, lo*hi, fp32 accumulation), so their matrix-unit ceiling in
# fp32-equivalent flops is a third of the bf16 peak.
MATRIX_PEAK = {"kda_chunk_fwd": (PEAK_BF16_MFMA / 3, "bf16x3 MFMA (v_mfma_f32_16x16x32_bf16)"),
               "kda_chunk_prep": (PEAK_BF16_MFMA / 3, "bf16x3 MFMA (v_mfma_f32_16x16x32_bf16)")}

T, H, D, C = 4096, 32, 128, 64


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def cpu_threads():
    """Threads the oracle baseline uses: the host cores this process may run
    on, capped at 16 (the GPU machine's per-GPU share of host cores)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


# Algorithmic HBM bytes of the whole prefill call (the survey's measurement
# plan): per token, q, k, v and the gate read as fp32 [H, D] rows, beta
# [H] and the core written [H, D]; plus the carried state read and written
# once.  Each byte is attributed to the kernel that has to move it: the
# prepare kernel reads every input row, the walk writes core and carries the
# state.
def alg_bytes_in_per_token(H, D):
    return H * (4 * D * 4 + 4)


def alg_bytes_out_per_token(H, D):
    return H * D * 4


def alg_state_bytes(H, D):
    return 2 * H * D * D * 4


def alg_call_bytes(T, H, D):
    return T * (alg_bytes_in_per_token(H, D) + alg_bytes_out_per_token(H, D)) + alg_state_bytes(H, D)


def alg_call_flops(T, H, D, C):
    # the survey's triangular chunk-form count per token and head:
    # 5CD + 6D^2 + C^2/3
    return T * H * (5 * C * D + 6 * D * D + C * C / 3.0)


# Algorithmic work per token and head of the two prefill kernels (chunk C,
# head_dim D).  Matrix products count 2 flops per multiply-add; products over
# a lower triangle count its (C+1)/2 average row length.
def fwd_flops_per_token_head(D, C):
    # W S, Qg S, KdT U: 2*D*D each;  P U over the lower triangle: (C+1)*D
    return 6 * D * D + (C + 1) * D


def prep_flops_per_token_head(D, C):
    # A strictly lower (C-1)*D and P with diagonal (C+1)*D; the unit-lower
    # triangular inverse C^2/3; W = Tb Kg and U' = Tb V: (C+1)*D each
    return 2 * C * D + C * C / 3.0 + 2 * (C + 1) * D


def block_floats(D, C):
    # per (chunk, head) operand block as moved: W, U', Qg, KdT, Ec and the
    # 16 x 32 pair fragments of P that reach the diagonal (a fragment wholly
    # above it, 32 kb > 16 w + 15, is neither written nor read)
    p_frags = sum(w // 2 + 1 for w in range(C // 16))
    return 4 * C * D + p_frags * 16 * 32 + D


def fwd_impl_bytes(T, H, D, C):
    # implementation traffic: read every operand block once, write core,
    # read + write the state
    return (T // C) * H * block_floats(D, C) * 4 + T * H * D * 4 + 2 * H * D * D * 4


def prep_impl_bytes(T, H, D, C):
    # implementation traffic: read q, k, v, gate, beta; write the operand blocks
    return T * H * (4 * D * 4 + 4) + (T // C) * H * block_floats(D, C) * 4


def ev():
    return torch.cuda.Event(enable_timing=True)


def setup_prefill(kda, dev):
    raw = workloads.core_raw(T, H, D, workloads.SEED_INPUT + 1, qkv_bf16=True)
    q, k, v = (torch.from_numpy(raw[n]).to(dev) for n in ("q", "k", "v"))
    gate = torch.empty(T, H, D, device=dev)
    beta = torch.empty(T, H, device=dev)
    kda.kda_gate(workloads.to_bf16(raw["g_raw"]).to(dev), torch.from_numpy(raw["a_log"]).to(dev),
                 torch.from_numpy(raw["dt_bias"]).to(dev), gate, T=T, heads=H, head_dim=D,
                 b_raw=workloads.to_bf16(raw["b_raw"]).to(dev), beta=beta)
    state = torch.from_numpy(workloads.state(H, D, 0.05, workloads.SEED_STATE + 1)).to(dev)
    core = torch.empty(T, H, D, device=dev)
    # kda_prefill's schedule: segments of `seg` chunks, each prepared into the
    # start of the workspace and walked at once
    seg = kda.kda_prefill_segment_chunks(T, H, D, C)
    ws = torch.empty(kda.kda_prefill_workspace_bytes(T, H, D, C), dtype=torch.uint8, device=dev)
    # the segments' row views, built once so the phase pass launches back to back
    rows = seg * C
    segs = []
    for r0 in range(0, T, rows):
        sl = slice(r0, min(T, r0 + rows))
        segs.append((q[sl], k[sl], v[sl], gate[sl], beta[sl], core[sl], sl.stop - sl.start))
    return dict(q=q, k=k, v=v, gate=gate, beta=beta, state=state, core=core, ws=ws, raw=raw,
                seg=seg, segs=segs)


def prefill_step(kda, P):
    """One whole prefill of T tokens: one kda_prefill call."""
    kda.kda_prefill(P["q"], P["k"], P["v"], P["gate"], P["beta"], P["state"], P["core"], P["ws"],
                    T=T, T_pad=T, heads=H, head_dim=D, chunk=C, scale=D ** -0.5)


def prefill_step_phases(kda, P, evs=None):
    """The same prefill as kda_prefill's own schedule spelled out (per segment
    of P["seg"] chunks: prepare into the start of the workspace, then
    forward; bitwise kda_prefill), with events (e0, e1, e2) per segment
    around the two kernels when evs is given."""
    for i, (q, k, v, g, b, core, Ts) in enumerate(P["segs"]):
        kw = dict(T=Ts, T_pad=Ts, heads=H, head_dim=D, chunk=C)
        if evs is not None:
            evs[i][0].record()
        kda.kda_prefill_prepare(q, k, v, g, b, P["ws"], **kw)
        if evs is not None:
            evs[i][1].record()
        kda.kda_prefill_forward(P["state"], core, P["ws"], scale=D ** -0.5, **kw)
        if evs is not None:
            evs[i][2].record()


def bench_prefill_bf16(kda, dev, P, reps=200):
    """The same prefill workload with q | k | v held as one bf16 [T, 3*H*D]
    row buffer (the conv output's form; the workload's values are bf16, so
    the fp32 arrays are their exact widening), run by kda_prefill_bf16.
    Checked bitwise against kda_prefill from the same state first."""
    qw = H * D
    qkv16 = torch.cat([P[n].reshape(T, qw) for n in ("q", "k", "v")], 1).to(torch.bfloat16)
    assert torch.equal(qkv16[:, :qw].float(), P["q"].reshape(T, qw))
    S0 = torch.from_numpy(workloads.state(H, D, 0.05, workloads.SEED_STATE + 1)).to(dev)
    st_a, st_b = S0.clone(), S0.clone()
    core_a, core_b = torch.empty_like(P["core"]), torch.empty_like(P["core"])
    kda.kda_prefill(P["q"], P["k"], P["v"], P["gate"], P["beta"], st_a, core_a, P["ws"], T=T,
                    T_pad=T, heads=H, head_dim=D, chunk=C, scale=D ** -0.5)

    def call(st, core):
        kda.kda_prefill_bf16(qkv16, P["gate"], P["beta"], st, core, P["ws"], T=T, T_pad=T,
                             heads=H, head_dim=D, chunk=C, scale=D ** -0.5)

    call(st_b, core_b)
    torch.cuda.synchronize()
    bitwise = bool(torch.equal(core_a, core_b) and torch.equal(st_a, st_b))
    for _ in range(20):
        call(st_b, core_b)
    a, b = ev(), ev()
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        call(st_b, core_b)
    b.record()
    torch.cuda.synchronize()
    t = a.elapsed_time(b) * 1e-3 / reps
    return dict(config=f"prefill T={T}, heads={H}, head_dim={D}, chunk={C}, q|k|v as bf16 rows "
                       "(kda_prefill_bf16)",
                ms=t * 1e3, tokens_per_s=T / t, bitwise_equal_to_fp32_inputs=bitwise)


def bench_decode(kda, dev, n_steps=64, n_inputs=8):
    B = 256
    a_log, dt = workloads.gate_params(H, D, workloads.SEED_INPUT + 2)
    a_log, dt = torch.from_numpy(a_log).to(dev), torch.from_numpy(dt).to(dev)
    steps = []
    for s in range(n_inputs):
        r = workloads.decode_step_raw(B, H, D, workloads.SEED_INPUT + 20 + s)
        g = torch.empty(B, H, D, device=dev)
        b = torch.empty(B, H, device=dev)
        kda.kda_gate(workloads.to_bf16(r["g_raw"]).to(dev), a_log, dt, g, T=B, heads=H,
                     head_dim=D, b_raw=workloads.to_bf16(r["b_raw"]).to(dev), beta=b)
        steps.append((r["qkv"].to(dev), g, b))
    state = torch.from_numpy(workloads.state(H, D, 0.05, workloads.SEED_STATE + 2, B=B)).to(dev)
    table = kda.ptr_table(state)
    core = torch.empty(B, H, D, device=dev)

    def one(i):
        qkv, g, b = steps[i % n_inputs]
        kda.kda_decode(qkv, g, b, table, core, B=B, heads=H, head_dim=D, scale=D ** -0.5)

    for i in range(4):
        one(i)
    evs = [(ev(), ev()) for _ in range(n_steps)]
    torch.cuda.synchronize()
    for i in range(n_steps):
        evs[i][0].record()
        one(i)
        evs[i][1].record()
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in evs])
    t = float(np.median(ms)) * 1e-3
    state_bytes = 2 * B * H * D * D * 4
    io_bytes = B * (3 * H * D * 2 + H * D * 4 + H * 4 + H * D * 4)
    return dict(config="decode B=256 H=32 D=128, 64 steps, fp32 state 537 MB",
                state_GBps=state_bytes / t / 1e9, total_GBps=(state_bytes + io_bytes) / t / 1e9,
                ms_per_step_median=t * 1e3, tokens_per_s=B / t,
                hbm_frac=(state_bytes + io_bytes) / t / PEAK_HBM,
                state_bytes_per_step=state_bytes, traffic=DECODE_TRAFFIC_BYTES)


def bench_decode_k(kda, dev, n_calls=32, n_sets=4):
    B, K = 64, 4
    cd = 3 * H * D
    a_log, dt = workloads.gate_params(H, D, workloads.SEED_INPUT + 3)
    a_log, dt = torch.from_numpy(a_log).to(dev), torch.from_numpy(dt).to(dev)
    conv = workloads.conv_raw(B * K, H, D, 4, workloads.SEED_INPUT + 3, n_seq=B)
    x = conv["x"].to(dev)
    w = conv["w"].to(dev)
    g_raw = workloads.to_bf16(np.random.default_rng(31).standard_normal((B * K, H * D))).to(dev)
    b_raw = workloads.to_bf16(np.random.default_rng(32).standard_normal((B * K, H))).to(dev)
    gate = torch.empty(B * K, H, D, device=dev)
    beta = torch.empty(B * K, H, device=dev)
    kda.kda_gate(g_raw, a_log, dt, gate, T=B * K, heads=H, head_dim=D, b_raw=b_raw, beta=beta)
    # rotate state sets so the 134 MB working set does not sit in the 256 MB cache
    sets = []
    for s in range(n_sets):
        st = torch.from_numpy(workloads.state(H, D, 0.05, workloads.SEED_STATE + 30 + s, B=B)).to(dev)
        cs = conv["state"].to(dev).clone()
        sets.append((st, kda.ptr_table(st), cs, kda.ptr_table(cs)))
    snaps = torch.empty(B * (K - 1), H, D, D, device=dev)
    snap_tab = kda.ptr_table(snaps)
    csnaps = torch.empty(B * (K - 1), 4, cd, dtype=torch.bfloat16, device=dev)
    csnap_tab = kda.ptr_table(csnaps)
    y = torch.empty(B * K, cd, dtype=torch.bfloat16, device=dev)
    core = torch.empty(B * K, H, D, device=dev)

    def one(i, e=None):
        st, tab, cs, ctab = sets[i % n_sets]
        if e:
            e[0].record()
        kda.conv_silu_l2(x, w, y, n_seq=B, rows=K, heads=H, head_dim=D, conv_state=ctab,
                         conv_snap=csnap_tab)
        if e:
            e[1].record()
        kda.kda_decode_k(y, gate, beta, tab, core, B=B, K=K, heads=H, head_dim=D,
                         scale=D ** -0.5, snap=snap_tab)
        if e:
            e[2].record()

    for i in range(n_sets):
        one(i)
    evs = [(ev(), ev(), ev()) for _ in range(n_calls)]
    torch.cuda.synchronize()
    for i in range(n_calls):
        one(i, evs[i])
    torch.cuda.synchronize()
    t_conv = float(np.median([a.elapsed_time(b) for a, b, _ in evs])) * 1e-3
    t_dk = float(np.median([b.elapsed_time(c) for _, b, c in evs])) * 1e-3

    # write-on-accept on the same rows: verify (state read only), then fold
    # K-1 accepted rows of every sequence (state read and written once)
    na = torch.full((B,), K - 1, dtype=torch.int32, device=dev)

    def woa(i, e=None):
        st, tab, _, _ = sets[i % n_sets]
        if e:
            e[0].record()
        kda.kda_verify_k(y, gate, beta, tab, core, B=B, K=K, heads=H, head_dim=D,
                         scale=D ** -0.5)
        if e:
            e[1].record()
        kda.kda_fold_accepted(y, gate, beta, tab, na, B=B, K=K, heads=H, head_dim=D)
        if e:
            e[2].record()

    for i in range(n_sets):
        woa(i)
    evw = [(ev(), ev(), ev()) for _ in range(n_calls)]
    torch.cuda.synchronize()
    for i in range(n_calls):
        woa(i, evw[i])
    torch.cuda.synchronize()
    t_ver = float(np.median([a.elapsed_time(b) for a, b, _ in evw])) * 1e-3
    t_fold = float(np.median([b.elapsed_time(c) for _, b, c in evw])) * 1e-3

    # the table form: the verify also writes each row's u, the fold applies
    # the K-1 accepted rows in one pass from them
    wy = torch.empty(B, H, K, D, device=dev)
    wy_tab = kda.ptr_table(wy)

    def woa_wy(i, e=None):
        st, tab, _, _ = sets[i % n_sets]
        if e:
            e[0].record()
        kda.kda_verify_wy_k(y, gate, beta, tab, wy_tab, core, B=B, K=K, heads=H, head_dim=D,
                            scale=D ** -0.5)
        if e:
            e[1].record()
        kda.kda_fold_wy(y, gate, tab, wy_tab, na, B=B, K=K, heads=H, head_dim=D)
        if e:
            e[2].record()

    for i in range(n_sets):
        woa_wy(i)
    evt = [(ev(), ev(), ev()) for _ in range(n_calls)]
    torch.cuda.synchronize()
    for i in range(n_calls):
        woa_wy(i, evt[i])
    torch.cuda.synchronize()
    t_ver_wy = float(np.median([a.elapsed_time(b) for a, b, _ in evt])) * 1e-3
    t_fold_wy = float(np.median([b.elapsed_time(c) for _, b, c in evt])) * 1e-3
    st1 = B * H * D * D * 4
    ver_b = st1 + B * K * (cd * 2 + H * D * 4 + H * 4 + H * D * 4)
    fold_b = 2 * st1 + B * (K - 1) * (2 * H * D * 2 + H * D * 4 + H * 4)
    state_b = B * H * D * D * 4 * (2 + (K - 1))                 # read, final write, K-1 snapshots
    io_b = B * K * (cd * 2 + H * D * 4 + H * 4 + H * D * 4)     # qkv, gate, beta, core
    conv_b = B * (4 * cd * 2) * (2 + (K - 1)) + B * K * cd * 2 * 2 + cd * 4 * 2
    return dict(config="decode_k B=64 K=4 H=32 D=128, 3 snapshots/seq, conv decode-K with snapshots",
                decode_k_ms=t_dk * 1e3, decode_k_GBps=(state_b + io_b) / t_dk / 1e9,
                decode_k_hbm_frac=(state_b + io_b) / t_dk / PEAK_HBM,
                conv_ms=t_conv * 1e3, conv_GBps=conv_b / t_conv / 1e9,
                verify_tokens_per_s=B * K / (t_dk + t_conv),
                write_on_accept=dict(verify_ms=t_ver * 1e3, fold_ms=t_fold * 1e3,
                                     verify_GBps=ver_b / t_ver / 1e9,
                                     fold_GBps=fold_b / t_fold / 1e9,
                                     state_bytes=3 * st1, decode_k_state_bytes=state_b,
                                     speedup_vs_snapshots=t_dk / (t_ver + t_fold),
                                     n_accept=K - 1,
                                     table_form=dict(verify_ms=t_ver_wy * 1e3,
                                                     fold_ms=t_fold_wy * 1e3,
                                                     fold_GBps=(2 * st1 + B * (K - 1) * (H * D * 2 + H * D * 4 + H * D * 4)) / t_fold_wy / 1e9)))


def bench_stages(kda, dev, reps=10):
    Tb = 8192
    cd = 3 * H * D
    conv = workloads.conv_raw(Tb, H, D, 4, workloads.SEED_INPUT + 4, n_seq=1)
    x, w = conv["x"].to(dev), conv["w"].to(dev)
    cs = torch.zeros(1, 4, cd, dtype=torch.bfloat16, device=dev)
    ctab = kda.ptr_table(cs)
    y = torch.empty(Tb, cd, dtype=torch.bfloat16, device=dev)
    q32, k32, v32 = (torch.empty(Tb, H * D, device=dev) for _ in range(3))
    r = np.random.default_rng(41)
    g_raw = workloads.to_bf16(r.standard_normal((Tb, H * D))).to(dev)
    b_raw = workloads.to_bf16(r.standard_normal((Tb, H))).to(dev)
    a_log, dt = workloads.gate_params(H, D, 42)
    a_log, dt = torch.from_numpy(a_log).to(dev), torch.from_numpy(dt).to(dev)
    gate = torch.empty(Tb, H, D, device=dev)
    beta = torch.empty(Tb, H, device=dev)
    nr = workloads.norm_raw(Tb, H, D, 43)
    core = torch.from_numpy(nr["core"]).to(dev).view(Tb, H * D)
    og, ow = nr["out_gate"].to(dev), nr["w"].to(dev)
    out = torch.empty(Tb, H * D, dtype=torch.bfloat16, device=dev)
    calls = {
        "conv_silu_l2": (lambda: kda.conv_silu_l2(x, w, y, n_seq=1, rows=Tb, heads=H, head_dim=D,
                                                  conv_state=ctab, q32=q32, k32=k32, v32=v32),
                         Tb * cd * 2 * 2 + Tb * H * D * 4 * 3),
        "kda_gate": (lambda: kda.kda_gate(g_raw, a_log, dt, gate, T=Tb, heads=H, head_dim=D,
                                          b_raw=b_raw, beta=beta),
                     Tb * H * D * (2 + 4) + Tb * H * (2 + 4)),
        "gated_rmsnorm": (lambda: kda.gated_rmsnorm(core, og, ow, out, T=Tb, heads=H, head_dim=D),
                          Tb * H * D * (4 + 2 + 2)),
    }
    res = {}
    for name, (fn, nbytes) in calls.items():
        fn()
        es = [(ev(), ev()) for _ in range(reps)]
        torch.cuda.synchronize()
        for a, b in es:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        t = float(np.median([a.elapsed_time(b) for a, b in es])) * 1e-3
        res[name] = dict(ms=t * 1e3, GBps=nbytes / t / 1e9, hbm_frac=nbytes / t / PEAK_HBM,
                         bytes=nbytes)
    res["config"] = "T=8192 rows, H=32, D=128 (conv_dim 12288), conv with fp32 q/k/v copies"
    return res


def bench_block(kda, dev, reps=10, pack_low_rank=True):
    """The full KDA block at T = 8192 (hidden 4096, 32 heads x 128, rank-128
    gates, weights ~ N(0, 0.02)): one kda_block_prefill call per repetition,
    from a zero state.  The projections' share is the block time less the
    stage kernels timed alone on the same buffers."""
    Tb, hidden, rank = 8192, 4096, 128
    qkv = H * D
    x, w = workloads.block_raw(Tb, hidden, H, D, rank, 4, workloads.SEED_INPUT + 4)
    x = x.to(dev)
    wd = {n: t.to(dev).contiguous() for n, t in w.items()}
    # q, k, v projection weights packed back to back, as a serving engine
    # stores them (the block then runs them as one GEMM), and likewise f_a,
    # g_a and b_proj
    wqkv = torch.cat([wd["q_proj"], wd["k_proj"], wd["v_proj"]]).contiguous()
    wd["q_proj"], wd["k_proj"], wd["v_proj"] = wqkv[:qkv], wqkv[qkv:2 * qkv], wqkv[2 * qkv:]
    if pack_low_rank:
        wlr = torch.cat([wd["f_a"], wd["g_a"], wd["b_proj"]]).contiguous()
        wd["f_a"], wd["g_a"], wd["b_proj"] = wlr[:rank], wlr[rank:2 * rank], wlr[2 * rank:]
    st = torch.zeros(H, D, D, device=dev)
    cs = torch.zeros(1, 4, 3 * qkv, dtype=torch.bfloat16, device=dev)
    ctab = kda.ptr_table(cs)
    buf = kda.block_buffers(Tb, heads=H, head_dim=D, rank=rank, chunk=C, device=dev)
    out = torch.empty(Tb, hidden, dtype=torch.bfloat16, device=dev)

    def block():
        kda.kda_block_prefill(x, wd, st, ctab, buf, out, T=Tb, T_pad=Tb, hidden_size=hidden,
                              heads=H, head_dim=D, rank=rank, chunk=C, scale=D ** -0.5)

    stages = {
        "conv_silu_l2": lambda: kda.conv_silu_l2(buf["qkv_proj"], wd["conv"], buf["conv_out"],
                                                 n_seq=1, rows=Tb, heads=H, head_dim=D,
                                                 conv_state=ctab),
        "kda_gate": lambda: kda.kda_gate(buf["g_raw"], wd["a_log"], wd["dt_bias"], buf["gate"],
                                         T=Tb, heads=H, head_dim=D, b_raw=buf["b_raw"],
                                         beta=buf["beta"]),
        "kda_prefill": lambda: kda.kda_prefill_bf16(buf["conv_out"], buf["gate"], buf["beta"],
                                                    st, buf["core"], buf["prefill_ws"], T=Tb,
                                                    T_pad=Tb, heads=H, head_dim=D, chunk=C,
                                                    scale=D ** -0.5),
        "gated_rmsnorm": lambda: kda.gated_rmsnorm(buf["core"].view(Tb, qkv), buf["out_gate"],
                                                   wd["o_norm"], buf["o_norm_out"], T=Tb, heads=H,
                                                   head_dim=D),
    }

    def timed(fn):
        for _ in range(3):
            fn()
        es = [(ev(), ev()) for _ in range(reps)]
        torch.cuda.synchronize()
        for a, b in es:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in es])) * 1e-3

    t_block = timed(block)
    t_st = {n: timed(f) for n, f in stages.items()}
    gemm_flops = 2.0 * Tb * (3 * qkv * hidden + 2 * rank * hidden + 2 * qkv * rank
                             + H * hidden + hidden * qkv)
    t_gemm = t_block - sum(t_st.values())
    return dict(config=f"block prefill T={Tb}, hidden={hidden}, heads={H}, head_dim={D}, "
                       f"rank={rank}, bf16 weights ~N(0,0.02), zero initial state",
                tokens_per_s=Tb / t_block, ms=t_block * 1e3,
                stage_ms={n: t * 1e3 for n, t in t_st.items()},
                projections_ms=t_gemm * 1e3, projection_gflop=gemm_flops / 1e9,
                projection_TFLOPs=gemm_flops / t_gemm / 1e12,
                projection_mfma_frac=gemm_flops / t_gemm / PEAK_BF16_MFMA)


def bench_prefill_varlen(kda, dev, reps=50):
    """The prefill workload's 4096 tokens (32 heads x 128, chunk 64, fp32
    states ~ N(0, 0.05)) as many prompts in one kda_prefill_varlen call:
    8 x 512 and 64 x 64 tokens, each prompt from its own state; and 16 times
    the workload's tokens (its rows repeated) as 256 prompts of 256."""
    out = {}
    raw = workloads.core_raw(T, H, D, workloads.SEED_INPUT + 6, qkv_bf16=True)
    a_log, dt = torch.from_numpy(raw["a_log"]).to(dev), torch.from_numpy(raw["dt_bias"]).to(dev)
    gate1 = torch.empty(T, H, D, device=dev)
    beta1 = torch.empty(T, H, device=dev)
    kda.kda_gate(workloads.to_bf16(raw["g_raw"]).to(dev), a_log, dt, gate1, T=T, heads=H,
                 head_dim=D, b_raw=workloads.to_bf16(raw["b_raw"]).to(dev), beta=beta1)
    q1, k1, v1 = (torch.from_numpy(raw[n]).to(dev) for n in ("q", "k", "v"))
    for n_seq, rep_rows in ((8, 1), (64, 1), (256, 16)):
        rows = T * rep_rows
        L = rows // n_seq
        q, k, v, gate = (x.repeat(rep_rows, 1, 1) for x in (q1, k1, v1, gate1))
        beta = beta1.repeat(rep_rows, 1)
        gen = torch.Generator(device=dev).manual_seed(workloads.SEED_STATE + 6)
        st = torch.randn(n_seq, H, D, D, device=dev, generator=gen) * 0.05
        tab = kda.ptr_table(st)
        cu = torch.arange(0, rows + 1, L, dtype=torch.int32, device=dev)
        mx, tot = kda.varlen_chunks([L] * n_seq, C)
        ws = torch.empty(kda.kda_prefill_varlen_workspace_bytes(n_seq, tot, H, D, C), dtype=torch.uint8,
                         device=dev)
        core = torch.empty(rows, H, D, device=dev)

        def call():
            kda.kda_prefill_varlen(q, k, v, gate, beta, tab, core, cu, ws, B=n_seq, rows=rows,
                                   max_chunks=mx, total_chunks=tot, heads=H, head_dim=D,
                                   chunk=C, scale=D ** -0.5)

        for _ in range(5):
            call()
        es = [(ev(), ev()) for _ in range(reps)]
        torch.cuda.synchronize()
        for a, b in es:
            a.record()
            call()
            b.record()
        torch.cuda.synchronize()
        t = float(np.median([a.elapsed_time(b) for a, b in es])) * 1e-3
        out[f"{n_seq}x{L}"] = dict(ms=t * 1e3, tokens_per_s=rows / t)
        del q, k, v, gate, beta, st, ws, core
    out["config"] = (f"{T} tokens as equal prompts (and {16 * T} as 256 x 256), heads={H}, "
                     f"head_dim={D}, chunk={C}, one kda_prefill_varlen call, per-prompt fp32 "
                     "states ~ N(0, 0.05)")
    return out


def bench_block_decode(kda, dev, reps=40, n_sets=4):
    """Block-level decode at the layer's full size (hidden 4096, 32 heads x
    128, rank-128 gates, weights ~ N(0, 0.02)): one sequence verifying K = 4
    draft tokens in one kda_block_decode_k call (3 state and conv snapshots)
    against one single-token kda_block_decode.  Calls rotate over n_sets
    independent layers (weights, state, conv state) whose weights together
    exceed the 256 MB last-level cache, as consecutive layers of a model
    would, so the weights stream from HBM.  The projection kernel alone
    (dense_gemv_bf16_batchm, q|k|v as one [12288, 4096] weight, 4 rows) gives
    the weight-read roofline."""
    hidden, rank, K = 4096, 128, 4
    qkv = H * D
    sets = []
    for s in range(n_sets):
        x, w = workloads.block_raw(K, hidden, H, D, rank, 4, workloads.SEED_INPUT + 5 + s)
        wd = {n: t.to(dev).contiguous() for n, t in w.items()}
        st = torch.from_numpy(workloads.state(H, D, 0.05, workloads.SEED_STATE + 5 + s)).to(dev)
        cs = workloads.conv_raw(1, H, D, 4, workloads.SEED_INPUT + 5 + s)["state"].to(dev)
        wqkv = torch.cat([wd["q_proj"], wd["k_proj"], wd["v_proj"]]).contiguous()
        sets.append(dict(x=x.to(dev).contiguous(), w=wd, st=st, tab=kda.ptr_table(st),
                         cs=cs, ctab=kda.ptr_table(cs), wqkv=wqkv))
    snaps = torch.empty(K - 1, H, D, D, device=dev)
    csnaps = torch.empty(K - 1, 4, 3 * qkv, dtype=torch.bfloat16, device=dev)
    snap_tab, csnap_tab = kda.ptr_table(snaps), kda.ptr_table(csnaps)
    buf_k = kda.block_decode_buffers(K, heads=H, head_dim=D, rank=rank, device=dev)
    buf_1 = kda.block_decode_buffers(1, heads=H, head_dim=D, rank=rank, device=dev)
    out = torch.empty(K, hidden, dtype=torch.bfloat16, device=dev)
    y = torch.empty(K, 3 * qkv, dtype=torch.bfloat16, device=dev)

    def verify(i):
        S = sets[i % n_sets]
        kda.kda_block_decode_k(S["x"], S["w"], S["tab"], S["ctab"], buf_k, out, B=1, K=K,
                               hidden_size=hidden, heads=H, head_dim=D, rank=rank,
                               scale=D ** -0.5, snap=snap_tab, conv_snap=csnap_tab)

    def decode(i):
        S = sets[i % n_sets]
        kda.kda_block_decode(S["x"][:1], S["w"], S["tab"], S["ctab"], buf_1, out[:1], B=1,
                             hidden_size=hidden, heads=H, head_dim=D, rank=rank,
                             scale=D ** -0.5)

    def gemv(i):
        S = sets[i % n_sets]
        kda.dense_gemv_bf16_batchm(S["x"], S["wqkv"], y, M=K, N=3 * qkv, Kd=hidden)

    na = torch.full((1,), K - 1, dtype=torch.int32, device=dev)

    def woa(i):   # write-on-accept: verify (no state writes), then fold K-1 rows
        S = sets[i % n_sets]
        kda.kda_block_verify_k(S["x"], S["w"], S["tab"], S["ctab"], buf_k, out, B=1, K=K,
                               hidden_size=hidden, heads=H, head_dim=D, rank=rank,
                               scale=D ** -0.5)
        kda.kda_block_fold_accepted(buf_k, S["tab"], S["ctab"], na, B=1, K=K, heads=H, head_dim=D)

    def timed(fn):
        for i in range(2 * n_sets):
            fn(i)
        es = [(ev(), ev()) for _ in range(reps)]
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(es):
            a.record()
            fn(i)
            b.record()
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in es])) * 1e-3

    def back_to_back(fn):   # reps calls between two events: per call, as layers follow layers
        a, b = ev(), ev()
        torch.cuda.synchronize()
        a.record()
        for i in range(reps):
            fn(i)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e-3 / reps

    wy = torch.empty(1, H, K, D, device=dev)
    wy_tab = kda.ptr_table(wy)

    def woa_wy(i):   # the same in table form: the fold from the verify's u rows
        S = sets[i % n_sets]
        kda.kda_block_verify_wy_k(S["x"], S["w"], S["tab"], S["ctab"], wy_tab, buf_k, out, B=1,
                                  K=K, hidden_size=hidden, heads=H, head_dim=D, rank=rank,
                                  scale=D ** -0.5)
        kda.kda_block_fold_wy(buf_k, S["tab"], S["ctab"], wy_tab, na, B=1, K=K, heads=H,
                              head_dim=D)

    # Each layer's call is checked and marshalled once (kda.bind) and then
    # re-issued, so the timing is the GPU's: the binding's per-call checks
    # cost tens of microseconds of host time, as much as the GPU work of one
    # call, and a loop of direct calls times the host as often as the GPU.
    def bound(fn):
        calls = [kda.bind(fn, i) for i in range(n_sets)]
        return lambda i: calls[i % n_sets]()

    t_v, t_d, t_g, t_w = timed(bound(verify)), timed(bound(decode)), timed(bound(gemv)), \
        timed(bound(woa))
    t_wt = timed(bound(woa_wy))
    t_v_py, t_d_py = timed(verify), timed(decode)
    t_v_bb, t_d_bb = back_to_back(bound(verify)), back_to_back(bound(decode))

    # the same calls captured once per layer in a HIP graph and replayed (the
    # launches of a call are enqueued back to back without host gaps)
    def graphs_of(fn):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(n_sets):
                fn(i)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        gs = []
        for i in range(n_sets):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                fn(i)
            gs.append(g)
        return gs

    # a batch: 16 sequences verifying K rows each (64 projection rows)
    Bb = 16
    for S in sets:
        S["stb"] = torch.from_numpy(workloads.state(H, D, 0.05, workloads.SEED_STATE + 7,
                                                    B=Bb)).to(dev)
        S["tabb"] = kda.ptr_table(S["stb"])
        S["csb"] = workloads.conv_raw(1, H, D, 4, workloads.SEED_INPUT + 7, n_seq=Bb)["state"].to(dev)
        S["ctabb"] = kda.ptr_table(S["csb"])
        S["xb"] = workloads.to_bf16(np.random.default_rng(77).standard_normal(
            (Bb * K, hidden))).to(dev)
    buf_b = kda.block_decode_buffers(Bb * K, heads=H, head_dim=D, rank=rank, device=dev)
    out_b = torch.empty(Bb * K, hidden, dtype=torch.bfloat16, device=dev)

    def verify_batch(i):
        S = sets[i % n_sets]
        kda.kda_block_decode_k(S["xb"], S["w"], S["tabb"], S["ctabb"], buf_b, out_b, B=Bb, K=K,
                               hidden_size=hidden, heads=H, head_dim=D, rank=rank,
                               scale=D ** -0.5)

    t_vb = timed(bound(verify_batch))
    gv, gd = graphs_of(verify), graphs_of(decode)
    t_gv = timed(lambda i: gv[i % n_sets].replay())
    t_gd = timed(lambda i: gd[i % n_sets].replay())
    w_bytes = 2 * (3 * qkv * hidden + 2 * rank * hidden + H * hidden + 2 * qkv * rank
                   + hidden * qkv)
    g_bytes = 2 * (3 * qkv * hidden + K * hidden + K * 3 * qkv)
    return dict(config=f"block decode, 1 sequence, K={K} verify rows, hidden={hidden}, "
                       f"heads={H}, head_dim={D}, rank={rank}, bf16 weights ~N(0,0.02), "
                       f"{n_sets} layers rotated (weights from HBM)",
                verify_ms=t_v * 1e3, decode_ms=t_d * 1e3,
                back_to_back_ms=dict(verify=t_v_bb * 1e3, decode=t_d_bb * 1e3,
                                     note=f"{reps} calls between two events, per call"),
                python_call_ms=dict(verify=t_v_py * 1e3, decode=t_d_py * 1e3,
                                    note="the same calls through the checking wrappers, "
                                         "each call marshalled anew"),
                write_on_accept_ms=t_w * 1e3,
                write_on_accept_table_ms=t_wt * 1e3,
                graph_verify_ms=t_gv * 1e3, graph_decode_ms=t_gd * 1e3,
                batch_verify=dict(sequences=Bb, rows=Bb * K, ms=t_vb * 1e3,
                                  tokens_per_s=Bb * K / t_vb),
                graph_speedup_vs_serial=K * t_gd / t_gv,
                verify_tokens_per_s=K / t_v, decode_tokens_per_s=1.0 / t_d,
                speedup_vs_serial=K * t_d / t_v, weight_bytes=w_bytes,
                verify_weight_GBps=w_bytes / t_v / 1e9,
                gemv=dict(shape=f"M={K} N={3 * qkv} Kd={hidden}", us=t_g * 1e6, bytes=g_bytes,
                          GBps=g_bytes / t_g / 1e9, hbm_frac=g_bytes / t_g / PEAK_HBM))


def measured_copy_bw(dev, nbytes=1 << 30, reps=20):
    """HBM bandwidth torch's device copy reaches on this GPU (read + write
    bytes per second, median of reps)."""
    src = torch.empty(nbytes // 4, device=dev)
    src.fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    es = [(ev(), ev()) for _ in range(reps)]
    torch.cuda.synchronize()
    for a, b in es:
        a.record()
        dst.copy_(src)
        b.record()
    torch.cuda.synchronize()
    t = float(np.median([a.elapsed_time(b) for a, b in es])) * 1e-3
    del src, dst
    return 2 * nbytes / t


def _timed_loop(fn, min_seconds):
    n, t0 = 0, time.perf_counter()
    while True:
        fn()
        n += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            return n, dt


def cpu_baseline(raw, threads, seconds=(8.0, 4.0, 4.0)):
    """The fp64 oracle, as it stands, timed on the host cores beside the GPU
    workloads: the whole prefill workload repeated for about seconds[0];
    decode (one step of a sample of the 256 sequences, state N(0, 0.05))
    and decode_k (K = 4 rows with the 3 state snapshots, a sample of the 64
    sequences) for about seconds[1] and seconds[2].  Decode and decode_k are
    also given as GB/s-equivalent over the same algorithmic bytes the GPU
    figures count (state read + written, snapshots, rows)."""
    import oracle
    scale = D ** -0.5
    g, b = oracle.kda_gate(raw["g_raw"], raw["a_log"], raw["dt_bias"], H, D, b_raw=raw["b_raw"])
    S0 = workloads.state(H, D, 0.05, workloads.SEED_STATE + 1)
    n, dt = _timed_loop(lambda: oracle.kda_recurrence(raw["q"], raw["k"], raw["v"], g, b, S0,
                                                      scale, threads=threads), seconds[0])
    res = dict(value=n * T / dt, unit="tokens/s", cores=threads,
               host_cpu_count=os.cpu_count(), affinity_cores=len(os.sched_getaffinity(0)),
               kind="oracle",
               sample=f"the whole prefill workload (T={T}, H={H}, D={D}) {n} times, "
                      f"token-serial fp64, heads split over {threads} threads; {dt:.1f} s")

    # decode: sequences of the decode workload, one step each (T = 1)
    a_log, dt_b = workloads.gate_params(H, D, workloads.SEED_INPUT + 2)
    Bs = 16
    r = workloads.decode_step_raw(Bs, H, D, workloads.SEED_INPUT + 20)
    qkv = r["qkv"].float().numpy().reshape(Bs, 3, H, D)
    gd, bd = oracle.kda_gate(r["g_raw"], a_log, dt_b, H, D, b_raw=r["b_raw"])
    gd, bd = gd.reshape(Bs, 1, H, D), bd.reshape(Bs, 1, H)
    Sd = workloads.state(H, D, 0.05, workloads.SEED_STATE + 2, B=Bs)

    from concurrent.futures import ThreadPoolExecutor
    pool = ThreadPoolExecutor(threads)   # independent sequences side by side (the C call
                                         # releases the GIL), one thread per sequence

    def dec():
        list(pool.map(lambda i: oracle.kda_recurrence(qkv[i, 0][None], qkv[i, 1][None],
                                                      qkv[i, 2][None], gd[i], bd[i], Sd[i],
                                                      scale), range(Bs)))

    n, dt = _timed_loop(dec, seconds[1])
    steps = n * Bs
    step_bytes = 2 * H * D * D * 4 + (3 * H * D * 2 + H * D * 4 + H * 4 + H * D * 4)
    res["decode"] = dict(tokens_per_s=steps / dt, GBps_equivalent=steps * step_bytes / dt / 1e9,
                         sample=f"{Bs} sequences x 1 step of the decode workload, {n} times, "
                                f"sequences over {threads} threads; {dt:.1f} s")

    # decode_k: K = 4 rows per sequence with the state after rows 0..2 kept
    K, Bk = 4, 16
    rk = workloads.decode_step_raw(Bk * K, H, D, workloads.SEED_INPUT + 3)
    qk = rk["qkv"].float().numpy().reshape(Bk, K, 3, H, D)
    gk, bk = oracle.kda_gate(rk["g_raw"], a_log, dt_b, H, D, b_raw=rk["b_raw"])
    gk, bk = gk.reshape(Bk, K, H, D), bk.reshape(Bk, K, H)
    Sk = workloads.state(H, D, 0.05, workloads.SEED_STATE + 30, B=Bk)

    def deck():
        list(pool.map(lambda i: oracle.kda_recurrence(qk[i, :, 0], qk[i, :, 1], qk[i, :, 2], gk[i],
                                                      bk[i], Sk[i], scale, snapshots=True),
                      range(Bk)))

    n, dt = _timed_loop(deck, seconds[2])
    seqs = n * Bk
    seq_bytes = H * D * D * 4 * (2 + (K - 1)) + K * (3 * H * D * 2 + H * D * 4 + H * 4 + H * D * 4)
    res["decode_k"] = dict(tokens_per_s=seqs * K / dt, GBps_equivalent=seqs * seq_bytes / dt / 1e9,
                           sample=f"{Bk} sequences x K={K} rows with 3 state snapshots, {n} "
                                  f"times, sequences over {threads} threads; {dt:.1f} s")
    pool.shutdown()
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    # defaults: ~20 ms of warm-up steps bring the GPU to its sustained clocks
    # (with 5 warm-up steps, 20 timed steps read ~20 % slower than steady state)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--prefill-only", action="store_true",
                    help="time the prefill steps only (profiler runs)")
    ap.add_argument("--block-only", action="store_true",
                    help="time the full-block call only and print its JSON object (profiler runs)")
    ap.add_argument("--decode-only", action="store_true",
                    help="time decode and decode_k only and print their JSON objects (profiler runs)")
    ap.add_argument("--block-decode-only", action="store_true",
                    help="time the block decode / K-row verify only (profiler runs)")
    ap.add_argument("--varlen-only", action="store_true",
                    help="time the several-prompt prefill only (profiler runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one plain 1 GiB device copy (scales HBM counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: measures one GPU only (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE {world}); the KDA core is measured per GPU and sharding is by "
              "sequence or head with no exchange inside the core.", file=sys.stderr)
        sys.exit(2)

    import gated_delta_rule_bounded_amd as kda
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.block_only:
        print(json.dumps({"block": bench_block(kda, dev)}), flush=True)
        return
    if args.decode_only:
        if args.calibrate_copy:
            src = torch.ones(1 << 28, device=dev)
            dst = torch.empty_like(src)
            torch.neg(src, out=dst)
            torch.cuda.synchronize()
            del src, dst
        print(json.dumps({"decode": bench_decode(kda, dev), "decode_k": bench_decode_k(kda, dev)}),
              flush=True)
        return
    if args.block_decode_only:
        print(json.dumps({"block_decode": bench_block_decode(kda, dev)}), flush=True)
        return
    if args.varlen_only:
        print(json.dumps({"prefill_varlen": bench_prefill_varlen(kda, dev)}), flush=True)
        return

    if args.calibrate_copy:
        # one elementwise kernel that reads 1 GiB and writes 1 GiB: the scale
        # of the FETCH_SIZE / WRITE_SIZE counters
        src = torch.ones(1 << 28, device=dev)           # 1 GiB fp32
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        log("copy calibration: 1 GiB read + 1 GiB write done")
        del src, dst

    P = setup_prefill(kda, dev)
    nseg = -(-T // (P["seg"] * C))
    log(f"prefill inputs ready ({nseg} segments of {P['seg']} chunks)")
    # Bring the GPU to its sustained clocks before anything is timed: about
    # half a second of the same step (a freshly started box runs the first
    # few hundred steps ~20 % slower).  Then the W warm-up and the K timed
    # steps of the contract.
    t_end = time.perf_counter() + 0.5
    while time.perf_counter() < t_end:
        for _ in range(20):
            prefill_step(kda, P)
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        prefill_step(kda, P)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        prefill_step(kda, P)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall / args.steps * 1e3
    # kernel durations: the same steps again in the spelled-out schedule, with
    # HIP events on the stream between the kernels
    evs = [[(ev(), ev(), ev()) for _ in range(nseg)] for _ in range(args.steps)]
    for _ in range(2):
        prefill_step_phases(kda, P)
    for i in range(args.steps):
        prefill_step_phases(kda, P, evs[i])
    torch.cuda.synchronize()
    # per kernel: the whole prefill's time in that kernel (sum over segments)
    t_prep = float(np.mean([sum(a.elapsed_time(b) for a, b, _ in e) for e in evs])) * 1e-3
    t_fwd = float(np.mean([sum(b.elapsed_time(c) for _, b, c in e) for e in evs])) * 1e-3
    log(f"prefill: {ms_step:.4f} ms/step, prepare {t_prep*1e6:.1f} us, forward {t_fwd*1e6:.1f} us "
        f"(per step, over {nseg} segments)")

    # Per launch (each kernel runs once per segment; the segments here are
    # equal): its share of the call's algorithmic bytes and flops, its
    # implementation traffic, and its average event duration.
    tok = T / nseg
    f_fwd = fwd_flops_per_token_head(D, C) * T * H / nseg
    f_prep = prep_flops_per_token_head(D, C) * T * H / nseg
    t_fwd, t_prep = t_fwd / nseg, t_prep / nseg
    kernels = {
        "kda_chunk_fwd": dict(avg_us=t_fwd * 1e6, launches_per_step=nseg, flops=f_fwd,
                              alg_bytes=tok * alg_bytes_out_per_token(H, D)
                              + alg_state_bytes(H, D) / nseg,
                              impl_bytes=fwd_impl_bytes(T, H, D, C) / nseg),
        "kda_chunk_prep": dict(avg_us=t_prep * 1e6, launches_per_step=nseg, flops=f_prep,
                               alg_bytes=tok * alg_bytes_in_per_token(H, D),
                               impl_bytes=prep_impl_bytes(T, H, D, C) / nseg),
    }
    for k, kv in kernels.items():
        t_k = kv["avg_us"] * 1e-6
        kv["TFLOPs"] = kv["flops"] / t_k / 1e12
        kv["alg_GBps"] = kv["alg_bytes"] / t_k / 1e9
        kv["impl_GBps"] = kv["impl_bytes"] / t_k / 1e9
        kv["matrix_peak_TFLOPs"] = MATRIX_PEAK[k][0] / 1e12
        kv["matrix_frac"] = kv["TFLOPs"] / kv["matrix_peak_TFLOPs"]
        kv["hbm_frac"] = kv["alg_GBps"] / (PEAK_HBM / 1e9)
        kv["traffic"] = TRAFFIC_BYTES.get(k)
    copy_Bps = measured_copy_bw(dev)
    # The dominant kernel is the slower one; its bound is the ceiling its
    # algorithmic work would reach first: bytes at 8 TB/s or products at the
    # matrix peak of the form it runs them in.
    dom = max(kernels, key=lambda k: kernels[k]["avg_us"])
    kd = kernels[dom]
    t_dom = kd["avg_us"] * 1e-6
    mat_peak, mat_dtype = MATRIX_PEAK[dom]
    if kd["alg_bytes"] / PEAK_HBM >= kd["flops"] / mat_peak:
        achieved = kd["alg_bytes"] / t_dom / 1e9
        roofline = dict(kernel=dom, bound="hbm", achieved=achieved, peak=PEAK_HBM / 1e9,
                        unit="GB/s", frac=achieved / (PEAK_HBM / 1e9), traffic=kd["traffic"],
                        alg_bytes_per_launch=kd["alg_bytes"],
                        frac_of_measured_copy=achieved / (copy_Bps / 1e9))
    else:
        achieved = kd["flops"] / t_dom / 1e12
        roofline = dict(kernel=dom, bound="mfma", achieved=achieved, peak=mat_peak / 1e12,
                        unit="TFLOP/s", frac=achieved / (mat_peak / 1e12), traffic=kd["traffic"],
                        dtype=mat_dtype, flops_per_launch=kd["flops"])
    # The whole call against its roofline: t_roof = max(F_alg / matrix peak,
    # B_alg / HBM peak) over the measured step, against the datasheet HBM
    # peak and against what a device copy reaches on this GPU.
    B_alg, F_alg = alg_call_bytes(T, H, D), alg_call_flops(T, H, D, C)
    t_meas = ms_step * 1e-3
    t_f = F_alg / MATRIX_PEAK["kda_chunk_fwd"][0]
    roofline["whole_call"] = dict(
        alg_bytes=B_alg, alg_flops=F_alg, ms=ms_step,
        t_roof_us=max(t_f, B_alg / PEAK_HBM) * 1e6,
        frac=max(t_f, B_alg / PEAK_HBM) / t_meas,
        measured_copy_GBps=copy_Bps / 1e9,
        t_roof_measured_us=max(t_f, B_alg / copy_Bps) * 1e6,
        frac_of_measured=max(t_f, B_alg / copy_Bps) / t_meas)

    out = {
        "metric": METRIC, "value": T / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32",
        "matrix_products": "f32 storage and accumulation; each fp32 product as 3 bf16 MFMA "
                           "(hi*hi + hi*lo + lo*hi)",
        "data": "synthetic",
        "config": {"workload": "chunked prefill core, 1 sequence, T=4096, heads=32, head_dim=128, "
                               "chunk=64, fp32 carried state ~N(0,0.05), q/k/v bf16-widened",
                   "T": T, "heads": H, "head_dim": D, "chunk": C},
        "roofline": roofline,
        "kernels": kernels,
    }
    log("prefill, bf16 q|k|v rows ...")
    out["prefill_bf16_rows"] = bench_prefill_bf16(kda, dev, P)
    log(f"prefill bf16 rows: {out['prefill_bf16_rows']['ms']:.4f} ms, bitwise "
        f"{out['prefill_bf16_rows']['bitwise_equal_to_fp32_inputs']}")
    if not args.prefill_only:
        log("decode ...")
        out["decode"] = bench_decode(kda, dev)
        log(f"decode: {out['decode']['state_GBps']:.1f} GB/s state")
        log("decode_k ...")
        out["decode_k"] = bench_decode_k(kda, dev)
        log("stages ...")
        out["stages"] = bench_stages(kda, dev)
        log("block ...")
        out["block"] = bench_block(kda, dev)
        log(f"block: {out['block']['tokens_per_s'] / 1e6:.2f} M tokens/s")
        log("prefill varlen ...")
        out["prefill_varlen"] = bench_prefill_varlen(kda, dev)
        log("block decode ...")
        out["block_decode"] = bench_block_decode(kda, dev)
        log(f"block decode: verify {out['block_decode']['verify_ms'] * 1e3:.1f} us, "
            f"decode {out['block_decode']['decode_ms'] * 1e3:.1f} us")
    if not args.no_cpu_baseline and not args.prefill_only:
        log("cpu baseline (oracle) ...")
        out["cpu_baseline"] = cpu_baseline(P["raw"], cpu_threads())
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
