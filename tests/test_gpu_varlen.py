"""kda_prefill_varlen: several sequences back to back in one call, each from
its own carried state ("Glm5NextLayer" page, batched / varlen linear-attention
prefill), against the oracle per sequence (2e-3, max relative error) and
bitwise against kda_prefill on each sequence alone."""
import numpy as np
import pytest
import torch

import gated_delta_rule_bounded_amd as kda
from conftest import relerr
from kda_cases import THREADS, core_case, cuda, gpu_prefill, say
import oracle

pytestmark = pytest.mark.gpu
TOL = 2e-3
SENTINEL = 7.0


def run_varlen(cases, H, D, C, scale, tail=3, tail_fill=np.nan, total_chunks=None, report=0,
               cu_first=0, max_chunks=None):
    """One kda_prefill_varlen call over the cases; its run-time report word
    must come out as ``report``.  ``cu_first`` replaces cu_seqlens[0] (a
    negative value is clamped to row 0 and reported); ``max_chunks`` and
    ``total_chunks`` replace the counts the lengths give."""
    lengths = [c["q"].shape[0] for c in cases]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    rows = int(cu[-1]) + tail      # rows past the last sequence hold poison

    def stack(name, shape):
        out = np.full((rows,) + shape, tail_fill, np.float32)
        for s, c in enumerate(cases):
            out[cu[s]:cu[s + 1]] = c[name]
        return cuda(out)

    q, k, v, g = (stack(n, (H, D)) for n in ("q", "k", "v", "gate"))
    b = stack("beta", (H,))
    states = [cuda(c["S0"]).contiguous() for c in cases]
    core = torch.full((rows, H, D), SENTINEL, dtype=torch.float32, device="cuda")
    mx, tot = kda.varlen_chunks(lengths, C)
    tot = tot if total_chunks is None else total_chunks
    mx = mx if max_chunks is None else max_chunks
    ws = torch.empty(max(1, kda.kda_prefill_varlen_workspace_bytes(len(cases), tot, H, D, C)),
                     dtype=torch.uint8, device="cuda")
    say("varlen", lengths, H, D, C, tot)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    cu_dev = cu.copy()
    cu_dev[0] = cu_first
    kda.kda_prefill_varlen(q, k, v, g, b, kda.ptr_table(states), core,
                           torch.from_numpy(cu_dev).cuda(), ws, B=len(cases), rows=rows,
                           max_chunks=mx, total_chunks=tot, heads=H, head_dim=D, chunk=C,
                           scale=scale, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == report, f"report word {int(status.item())}, expected {report}"
    return cu, core.cpu().numpy(), [s.cpu().numpy() for s in states]


@pytest.mark.parametrize("lengths,H,D,C", [
    ([57, 0, 64, 130, 1], 2, 16, 16),
    ([57, 16, 33], 2, 16, 64),
    ([200, 64, 0, 31, 129], 2, 128, 64),
    ([40, 17], 2, 128, 16),
])
def test_varlen_matches_oracle_and_single_calls(lengths, H, D, C):
    scale = D ** -0.5
    cases = [core_case(T, H, D, 1400 + 7 * s + T, 0.05) for s, T in enumerate(lengths)]
    cu, core, states = run_varlen(cases, H, D, C, scale)
    covered = np.zeros(core.shape[0], bool)
    for s, (c, T) in enumerate(zip(cases, lengths)):
        rows = core[cu[s]:cu[s + 1]]
        covered[cu[s]:cu[s + 1]] = True
        if T == 0:
            np.testing.assert_array_equal(states[s], c["S0"])
            continue
        ref_core, ref_S, _ = oracle.kda_recurrence(c["q"], c["k"], c["v"], c["gate"], c["beta"],
                                                   c["S0"], scale)
        assert relerr(rows, ref_core) < TOL, f"seq {s} core"
        assert relerr(states[s], ref_S) < TOL, f"seq {s} state"
        T_pad = -(-T // C) * C
        one_core, one_S = gpu_prefill(c, T, T_pad, C, scale, fill=0.0)
        np.testing.assert_array_equal(rows, one_core[:T], err_msg=f"seq {s} core bitwise")
        np.testing.assert_array_equal(states[s], one_S, err_msg=f"seq {s} state bitwise")
    assert np.all(core[~covered] == SENTINEL)


def test_varlen_full_size_many_prompts():
    # the prefill workload's 4096 tokens as 8 prompts of mixed length at the
    # full head shape (32 heads x 128, chunk 64), each from its own state
    H, D, C = 32, 128, 64
    lengths = [512, 1000, 64, 7, 777, 1024, 300, 412]
    assert sum(lengths) == 4096
    scale = D ** -0.5
    cases = [core_case(T, H, D, 1500 + s, 0.05, qkv_bf16=True) for s, T in enumerate(lengths)]
    cu, core, states = run_varlen(cases, H, D, C, scale)
    for s, (c, T) in enumerate(zip(cases, lengths)):
        rows = core[cu[s]:cu[s + 1]]
        T_pad = -(-T // C) * C
        one_core, one_S = gpu_prefill(c, T, T_pad, C, scale, fill=0.0)
        np.testing.assert_array_equal(rows, one_core[:T], err_msg=f"seq {s} core bitwise")
        np.testing.assert_array_equal(states[s], one_S, err_msg=f"seq {s} state bitwise")
        if s in (1, 3, 6):
            ref_core, ref_S, _ = oracle.kda_recurrence(c["q"], c["k"], c["v"], c["gate"],
                                                       c["beta"], c["S0"], scale, threads=THREADS)
            assert relerr(rows, ref_core) < TOL, f"seq {s} core"
            assert relerr(states[s], ref_S) < TOL, f"seq {s} state"
    assert np.all(core[cu[-1]:] == SENTINEL)


# Calls of more than a wave (64) of sequences find them through the tables of
# a plan kernel, smaller ones from cu directly: ``lead`` empty prompts ahead
# of the cases take a test through the tables.
LEADS = [0, 100]


def _with_lead(lead, H, D, lengths, seed):
    cases = [core_case(0, H, D, seed - 1 - i, 0.05) for i in range(lead)]
    return cases + [core_case(T, H, D, seed + s, 0.05) for s, T in enumerate(lengths)]


@pytest.mark.parametrize("lead", LEADS)
def test_varlen_sequence_outside_the_workspace_is_left_alone(lead):
    # total_chunks one short: the last sequence's blocks would not fit, so it
    # is skipped whole (state and core rows untouched); the others are exact
    H, D, C = 2, 128, 64
    lengths = [100, 64, 70]
    scale = D ** -0.5
    cases = _with_lead(lead, H, D, lengths, 1600)
    _, tot = kda.varlen_chunks(lengths, C)
    # the skip is reported (KDA_REPORT_SEQ_SKIPPED)
    cu, core, states = run_varlen(cases, H, D, C, scale, total_chunks=tot - 1, report=1)
    o = lead
    np.testing.assert_array_equal(states[o + 2], cases[o + 2]["S0"])
    assert np.all(core[cu[o + 2]:cu[o + 3]] == SENTINEL)
    for s in (o, o + 1):
        T = lengths[s - o]
        one_core, one_S = gpu_prefill(cases[s], T, -(-T // C) * C, C, scale)
        np.testing.assert_array_equal(core[cu[s]:cu[s + 1]], one_core[:T])
        np.testing.assert_array_equal(states[s], one_S)
    for s in range(lead):
        np.testing.assert_array_equal(states[s], cases[s]["S0"])


def test_varlen_single_chunk_prompts_same_bits_in_both_forward_instances():
    # every prompt within one chunk runs the forward instance without the
    # load-ahead register set; adding one longer prompt to the same call
    # switches the launch to the load-ahead instance, and the short prompts'
    # rows and states must come out bit for bit the same
    H, D, C = 32, 128, 64
    lengths = [64] * 60 + [33, 1, 64, 50]
    scale = D ** -0.5
    cases = [core_case(T, H, D, 1700 + s, 0.05, qkv_bf16=True) for s, T in enumerate(lengths)]
    cu_a, core_a, states_a = run_varlen(cases, H, D, C, scale)
    long_case = core_case(200, H, D, 1799, 0.05, qkv_bf16=True)
    cu_b, core_b, states_b = run_varlen(cases + [long_case], H, D, C, scale)
    for s in range(len(lengths)):
        np.testing.assert_array_equal(core_a[cu_a[s]:cu_a[s + 1]], core_b[cu_b[s]:cu_b[s + 1]],
                                      err_msg=f"seq {s} core")
        np.testing.assert_array_equal(states_a[s], states_b[s], err_msg=f"seq {s} state")
    for s in (0, 37, 60, 61):
        c = cases[s]
        ref_core, ref_S, _ = oracle.kda_recurrence(c["q"], c["k"], c["v"], c["gate"], c["beta"],
                                                   c["S0"], scale, threads=THREADS)
        assert relerr(core_a[cu_a[s]:cu_a[s + 1]], ref_core) < TOL, f"seq {s} core"
        assert relerr(states_a[s], ref_S) < TOL, f"seq {s} state"
    c = long_case
    ref_core, ref_S, _ = oracle.kda_recurrence(c["q"], c["k"], c["v"], c["gate"], c["beta"],
                                               c["S0"], scale, threads=THREADS)
    assert relerr(core_b[cu_b[-2]:cu_b[-1]], ref_core) < TOL
    assert relerr(states_b[-1], ref_S) < TOL


@pytest.mark.parametrize("lead", LEADS)
def test_varlen_clamped_offset_is_reported(lead):
    # cu_seqlens[0] = -5 is clamped to row 0 (KDA_REPORT_ROWS_CLAMPED); the
    # rows and states are those of the call with the offset given as 0
    H, D, C = 2, 16, 16
    lengths = [40, 17, 33]
    scale = D ** -0.5
    cases = _with_lead(lead, H, D, lengths, 1650)
    cu_a, core_a, states_a = run_varlen(cases, H, D, C, scale)
    cases_b = [dict(c, S0=c["S0"].copy()) for c in cases]
    cu_b, core_b, states_b = run_varlen(cases_b, H, D, C, scale, report=2, cu_first=-5)
    np.testing.assert_array_equal(core_a, core_b)
    for a, b in zip(states_a, states_b):
        np.testing.assert_array_equal(a, b)


def test_varlen_many_one_chunk_prompts_whole_head_walks():
    # 130 prompts of at most one chunk at 2 heads x 128: 260 (prompt, head)
    # pairs, so the walk takes whole heads per workgroup; every prompt's rows
    # and state are bitwise those of kda_prefill on it alone (16-column
    # walks), and a sample matches the oracle
    H, D, C = 2, 128, 64
    rng = np.random.default_rng(1800)
    lengths = [int(x) for x in rng.integers(1, 65, size=130)]
    scale = D ** -0.5
    cases = [core_case(T, H, D, 1800 + s, 0.05) for s, T in enumerate(lengths)]
    cu, core, states = run_varlen(cases, H, D, C, scale)
    for s in range(0, len(lengths), 7):
        c, T = cases[s], lengths[s]
        one_core, one_S = gpu_prefill(c, T, C, C, scale, fill=0.0)
        np.testing.assert_array_equal(core[cu[s]:cu[s + 1]], one_core[:T], err_msg=f"seq {s}")
        np.testing.assert_array_equal(states[s], one_S, err_msg=f"seq {s} state")
    for s in (0, 64, 129):
        c = cases[s]
        ref_core, ref_S, _ = oracle.kda_recurrence(c["q"], c["k"], c["v"], c["gate"], c["beta"],
                                                   c["S0"], scale)
        assert relerr(core[cu[s]:cu[s + 1]], ref_core) < TOL
        assert relerr(states[s], ref_S) < TOL
    assert np.all(core[cu[-1]:] == SENTINEL)


@pytest.mark.parametrize("lead", LEADS)
@pytest.mark.parametrize("skip", ["longer_than_max_chunks", "outside_total_chunks"])
def test_varlen_one_chunk_kernel_skips_and_reports(skip, lead):
    # max_chunks = 1 at 128 x 64 runs prepare and walk in one kernel; a prompt
    # longer than one chunk (max_chunks = 1 stated anyway) or one whose chunk
    # lies past total_chunks is skipped whole and reported, the others stay
    # bitwise those of kda_prefill alone
    H, D, C = 4, 128, 64
    lengths = [64, 30, 100, 1, 64] if skip == "longer_than_max_chunks" else [64, 30, 17, 1, 64]
    lengths = [0] * lead + lengths
    scale = D ** -0.5
    cases = [core_case(T, H, D, 1900 + s, 0.05, qkv_bf16=True) for s, T in enumerate(lengths)]
    if skip == "longer_than_max_chunks":
        cu, core, states = run_varlen(cases, H, D, C, scale, max_chunks=1, report=1)
        skipped = [lead + 2]
    else:
        cu, core, states = run_varlen(cases, H, D, C, scale, total_chunks=5 - 1, report=1)
        skipped = [lead + 4]
    for s, T in enumerate(lengths):
        if s in skipped or T == 0:
            np.testing.assert_array_equal(states[s], cases[s]["S0"])
            assert np.all(core[cu[s]:cu[s + 1]] == SENTINEL)
            continue
        one_core, one_S = gpu_prefill(cases[s], T, C, C, scale)
        np.testing.assert_array_equal(core[cu[s]:cu[s + 1]], one_core[:T], err_msg=f"seq {s}")
        np.testing.assert_array_equal(states[s], one_S, err_msg=f"seq {s} state")


def test_varlen_thousands_of_one_chunk_prompts():
    # 3000 prompts of at most one chunk (one launch of the fused kernel, no
    # segments): a sample bitwise equal to kda_prefill alone, and the oracle
    H, D, C = 2, 128, 64
    rng = np.random.default_rng(1950)
    lengths = [int(x) for x in rng.integers(0, 65, size=3000)]
    scale = D ** -0.5
    cases = [core_case(T, H, D, 20000 + s, 0.05) for s, T in enumerate(lengths)]
    cu, core, states = run_varlen(cases, H, D, C, scale)
    for s in list(range(0, len(lengths), 257)) + [len(lengths) - 1]:
        c, T = cases[s], lengths[s]
        if T == 0:
            np.testing.assert_array_equal(states[s], c["S0"])
            continue
        one_core, one_S = gpu_prefill(c, T, C, C, scale, fill=0.0)
        np.testing.assert_array_equal(core[cu[s]:cu[s + 1]], one_core[:T], err_msg=f"seq {s}")
        np.testing.assert_array_equal(states[s], one_S, err_msg=f"seq {s} state")
    for s in (1, 1500, 2999):
        c = cases[s]
        if lengths[s] == 0:
            continue
        ref_core, ref_S, _ = oracle.kda_recurrence(c["q"], c["k"], c["v"], c["gate"], c["beta"],
                                                   c["S0"], scale)
        assert relerr(core[cu[s]:cu[s + 1]], ref_core) < TOL
        assert relerr(states[s], ref_S) < TOL
    assert np.all(core[cu[-1]:] == SENTINEL)


@pytest.mark.parametrize("nseq,L", [(4, 1024), (16, 256)])
def test_varlen_wide_walk_workgroups_bitwise(nseq, L):
    # many (prompt, head) pairs per segment: the walk takes 2 or 4 value-
    # column tiles per workgroup; every prompt's rows and state are still
    # bitwise those of kda_prefill alone (one 16-column tile per workgroup)
    H, D, C = 32, 128, 64
    scale = D ** -0.5
    lengths = [L] * nseq
    cases = [core_case(L, H, D, 2100 + s, 0.05, qkv_bf16=True) for s in range(nseq)]
    cu, core, states = run_varlen(cases, H, D, C, scale)
    for s in sorted({0, nseq // 2, nseq - 1}):
        one_core, one_S = gpu_prefill(cases[s], L, L, C, scale)
        np.testing.assert_array_equal(core[cu[s]:cu[s + 1]], one_core[:L], err_msg=f"seq {s}")
        np.testing.assert_array_equal(states[s], one_S, err_msg=f"seq {s} state")
    c = cases[nseq - 1]
    ref_core, ref_S, _ = oracle.kda_recurrence(c["q"], c["k"], c["v"], c["gate"], c["beta"],
                                               c["S0"], scale, threads=THREADS)
    assert relerr(core[cu[-2]:cu[-1]], ref_core) < TOL
    assert relerr(states[-1], ref_S) < TOL


def test_varlen_many_multi_chunk_prompts_over_many_segments():
    # 1200 prompts of 0..400 tokens and one of 3000 (several chunks each,
    # empty ones between them) over 16 cache-sized segments, so that many
    # prompts straddle a segment boundary and the call's sequence tables span
    # two blocks of the plan kernel: every prompt that straddles a boundary,
    # and a sample of the rest, bitwise equal to kda_prefill alone
    H, D, C = 4, 128, 64
    rng = np.random.default_rng(1951)
    lengths = [int(x) for x in rng.integers(0, 401, size=1200)]
    lengths[700] = 3000
    scale = D ** -0.5
    cases = [core_case(T, H, D, 30000 + s, 0.05) for s, T in enumerate(lengths)]
    cu, core, states = run_varlen(cases, H, D, C, scale)
    nch = [-(-T // C) for T in lengths]
    c0 = np.concatenate([[0], np.cumsum(nch)])
    seg = kda.kda_prefill_segment_chunks(int(c0[-1]) * C, H, D, C)
    assert int(c0[-1]) > 15 * seg
    straddle = [s for s in range(len(lengths))
                if nch[s] > 1 and (c0[s] // seg) != ((c0[s + 1] - 1) // seg)]
    assert len(straddle) >= 10
    for s in sorted(set(straddle) | set(range(0, len(lengths), 97)) | {700, len(lengths) - 1}):
        c, T = cases[s], lengths[s]
        if T == 0:
            np.testing.assert_array_equal(states[s], c["S0"])
            assert np.all(core[cu[s]:cu[s + 1]] == SENTINEL)
            continue
        one_core, one_S = gpu_prefill(c, T, nch[s] * C, C, scale, fill=0.0)
        np.testing.assert_array_equal(core[cu[s]:cu[s + 1]], one_core[:T], err_msg=f"seq {s}")
        np.testing.assert_array_equal(states[s], one_S, err_msg=f"seq {s} state")
    for s in (straddle[0], 700):
        c = cases[s]
        ref_core, ref_S, _ = oracle.kda_recurrence(c["q"], c["k"], c["v"], c["gate"], c["beta"],
                                                   c["S0"], scale, threads=THREADS)
        assert relerr(core[cu[s]:cu[s + 1]], ref_core) < TOL
        assert relerr(states[s], ref_S) < TOL
    assert np.all(core[cu[-1]:] == SENTINEL)


def test_varlen_most_sequences_the_call_takes():
    # 65535 prompts (the most one call takes) of 0..3 tokens at 2 heads x 16,
    # chunk 16: the plan kernel walks 64 blocks of prompts, and each of the
    # four cache-sized segments launches ~12k chunks' prepare workgroups and
    # as many walks.  Empty prompts keep their state; a sample of the rest is
    # bitwise kda_prefill alone, and two match the oracle
    H, D, C, B = 2, 16, 16, 65535
    rng = np.random.default_rng(1952)
    lengths = rng.integers(0, 4, size=B)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    rows = int(cu[-1])

    def unit(x):
        return (x / np.linalg.norm(x, axis=-1, keepdims=True)).astype(np.float32)
    q = unit(rng.standard_normal((rows, H, D)))
    k = unit(rng.standard_normal((rows, H, D)))
    v = rng.standard_normal((rows, H, D)).astype(np.float32)
    g = (-np.exp(rng.uniform(-1, 0.5, (1, H, 1))) *
         np.log1p(np.exp(rng.standard_normal((rows, H, D))))).astype(np.float32)
    b = (1 / (1 + np.exp(-rng.standard_normal((rows, H))))).astype(np.float32)
    S0 = (rng.standard_normal((B, H, D, D)) * 0.05).astype(np.float32)
    states = cuda(S0)
    core = torch.full((rows, H, D), SENTINEL, dtype=torch.float32, device="cuda")
    mx, tot = kda.varlen_chunks([int(x) for x in lengths], C)
    ws = torch.empty(kda.kda_prefill_varlen_workspace_bytes(B, tot, H, D, C), dtype=torch.uint8,
                     device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    say("varlen 65535 prompts", H, D, C, tot)
    kda.kda_prefill_varlen(cuda(q), cuda(k), cuda(v), cuda(g), cuda(b), kda.ptr_table(states),
                           core, torch.from_numpy(cu).cuda(), ws, B=B, rows=rows, max_chunks=mx,
                           total_chunks=tot, heads=H, head_dim=D, chunk=C, scale=D ** -0.5,
                           status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    got_S, got_core = states.cpu().numpy(), core.cpu().numpy()
    empty = lengths == 0
    np.testing.assert_array_equal(got_S[empty], S0[empty])
    for s in sorted(set(range(0, B, 1311)) | {B - 1}):
        T = int(lengths[s])
        if T == 0:
            continue
        sl = slice(cu[s], cu[s + 1])
        case = dict(q=q[sl], k=k[sl], v=v[sl], gate=g[sl], beta=b[sl], S0=S0[s])
        one_core, one_S = gpu_prefill(case, T, C, C, D ** -0.5)
        np.testing.assert_array_equal(got_core[sl], one_core[:T], err_msg=f"seq {s}")
        np.testing.assert_array_equal(got_S[s], one_S, err_msg=f"seq {s} state")
    for s in [i for i in (7, 32768, B - 2) if lengths[i] > 0]:
        sl = slice(cu[s], cu[s + 1])
        ref_core, ref_S, _ = oracle.kda_recurrence(q[sl], k[sl], v[sl], g[sl], b[sl], S0[s],
                                                   D ** -0.5)
        assert relerr(got_core[sl], ref_core) < TOL
        assert relerr(got_S[s], ref_S) < TOL
