"""kda_decode / kda_decode_k on the GPU.

Against the oracle: max relative error < 2e-3 on core and states (fp32 work).
decode_k against K serial decode calls: bit-identical core, final state and
every snapshot ("Glm5NextKdaLayer" page, decode_k).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from conftest import relerr
from kda_cases import THREADS, cuda, say

pytestmark = pytest.mark.gpu
TOL = 2e-3


def _steps(B, H, D, n_steps, seed):
    """Per step: qkv bf16 [B, 3HD] (q/k unit-normalised), gate fp32 [B,H,D],
    beta fp32 [B,H] (gate/beta from the oracle's gate on the seeded draws)."""
    a_log, dt = workloads.gate_params(H, D, seed)
    out = []
    for s in range(n_steps):
        r = workloads.decode_step_raw(B, H, D, seed + 1 + s)
        g, b = oracle.kda_gate(r["g_raw"], a_log, dt, H, D, b_raw=r["b_raw"])
        out.append(dict(qkv=r["qkv"], gate=g.astype(np.float32), beta=b.astype(np.float32)))
    return out


def _oracle_seq(steps, S0_b, b, H, D, scale):
    """Oracle over the steps of sequence b: returns core [n, H, D], S, snaps."""
    qkv = np.stack([s["qkv"][b].double().numpy() for s in steps])        # [n, 3HD]
    n = qkv.shape[0]
    q = qkv[:, : H * D].reshape(n, H, D)
    k = qkv[:, H * D: 2 * H * D].reshape(n, H, D)
    v = qkv[:, 2 * H * D:].reshape(n, H, D)
    g = np.stack([s["gate"][b] for s in steps])
    bt = np.stack([s["beta"][b] for s in steps])
    return oracle.kda_recurrence(q, k, v, g, bt, S0_b, scale, snapshots=True, threads=THREADS)


@pytest.mark.parametrize("B,H,D,n_steps", [(3, 2, 16, 8), (4, 4, 128, 5)])
def test_decode_matches_oracle(B, H, D, n_steps):
    import gated_delta_rule_bounded_amd as kda
    scale = D ** -0.5
    S0 = workloads.state(H, D, 0.05, 2002, B=B)
    steps = _steps(B, H, D, n_steps, 3000)
    st = cuda(S0)
    table = kda.ptr_table(st)
    cores = []
    say("decode", B, H, D, n_steps)
    for s in steps:
        core = torch.empty(B, H, D, device="cuda")
        kda.kda_decode(cuda(s["qkv"], torch.bfloat16), cuda(s["gate"]), cuda(s["beta"]), table,
                       core, B=B, heads=H, head_dim=D, scale=scale)
        cores.append(core)
    torch.cuda.synchronize()
    got_core = torch.stack(cores, 1).cpu().numpy()      # [B, n, H, D]
    got_S = st.cpu().numpy()
    for b in range(B):
        ref_core, ref_S, _ = _oracle_seq(steps, S0[b], b, H, D, scale)
        assert relerr(got_core[b], ref_core) < TOL
        assert relerr(got_S[b], ref_S) < TOL


def _decode_k_vs_serial(B, K, H, D, seed, snapshots=True):
    import gated_delta_rule_bounded_amd as kda
    scale = D ** -0.5
    S0 = workloads.state(H, D, 0.05, seed, B=B)
    rows = _steps(B, H, D, K, seed)                        # K steps of B sequences
    # sequence-major [B*K] layout for decode_k
    qkv = torch.stack([r["qkv"] for r in rows], 1).reshape(B * K, -1)
    gate = np.stack([r["gate"] for r in rows], 1).reshape(B * K, H, D)
    beta = np.stack([r["beta"] for r in rows], 1).reshape(B * K, H)

    st_k = cuda(S0)
    snaps = torch.full((B * max(K - 1, 1), H, D, D), float("nan"), device="cuda")
    core_k = torch.empty(B * K, H, D, device="cuda")
    say("decode_k", B, K, H, D)
    kda.kda_decode_k(cuda(qkv, torch.bfloat16), cuda(gate), cuda(beta), kda.ptr_table(st_k),
                     core_k, B=B, K=K, heads=H, head_dim=D, scale=scale,
                     snap=kda.ptr_table(snaps) if snapshots and K > 1 else None)

    st_s = cuda(S0)
    tab_s = kda.ptr_table(st_s)
    serial_core, serial_states = [], []
    for t, r in enumerate(rows):
        c = torch.empty(B, H, D, device="cuda")
        kda.kda_decode(cuda(r["qkv"], torch.bfloat16), cuda(r["gate"]), cuda(r["beta"]), tab_s, c,
                       B=B, heads=H, head_dim=D, scale=scale)
        serial_core.append(c)
        serial_states.append(st_s.clone())
    torch.cuda.synchronize()
    ck = core_k.view(B, K, H, D)
    for t in range(K):
        assert torch.equal(ck[:, t].view(torch.int32), serial_core[t].view(torch.int32))
    assert torch.equal(st_k.view(torch.int32), st_s.view(torch.int32))
    if snapshots and K > 1:
        sn = snaps.view(B, K - 1, H, D, D)
        for t in range(K - 1):
            assert torch.equal(sn[:, t].view(torch.int32), serial_states[t].view(torch.int32))
    return rows, S0, ck.cpu().numpy(), st_k.cpu().numpy(), snaps


@pytest.mark.parametrize("B,K,H,D", [(3, 4, 2, 16), (5, 4, 4, 128), (2, 1, 4, 128), (2, 7, 2, 128)])
def test_decode_k_bitwise_equals_serial_decode(B, K, H, D):
    rows, S0, ck, sk, _ = _decode_k_vs_serial(B, K, H, D, 4000 + K)
    for b in range(B):
        ref_core, ref_S, _ = _oracle_seq(rows, S0[b], b, H, D, D ** -0.5)
        assert relerr(ck[b], ref_core) < TOL
        assert relerr(sk[b], ref_S) < TOL


def test_decode_k_full_size_b64_k4():
    """Speculative-verify workload: 64 sequences, K=4, H=32, D=128, three
    snapshots per sequence; bitwise vs 4 serial decodes, oracle on a sample."""
    B, K, H, D = 64, 4, 32, 128
    rows, S0, ck, sk, snaps = _decode_k_vs_serial(B, K, H, D, 2003)
    sn = snaps.view(B, K - 1, H, D, D)
    for b in (0, 37, 63):
        ref_core, ref_S, ref_snaps = _oracle_seq(rows, S0[b], b, H, D, D ** -0.5)
        assert relerr(ck[b], ref_core) < TOL
        assert relerr(sk[b], ref_S) < TOL
        for t in range(K - 1):
            assert relerr(sn[b, t].cpu().numpy(), ref_snaps[t]) < TOL


def test_decode_full_size_b256():
    """Batched decode workload: 256 sequences, H=32, D=128, state ~ N(0, 0.05),
    64 steps on the GPU; the oracle follows 3 sampled sequences through all 64
    steps and all 256 sequences through the first step."""
    import gated_delta_rule_bounded_amd as kda
    B, H, D, n_steps = 256, 32, 128, 64
    scale = D ** -0.5
    S0 = workloads.state(H, D, 0.05, 2002, B=B)
    steps = _steps(B, H, D, n_steps, 3002)
    st = cuda(S0)
    table = kda.ptr_table(st)
    say("decode full", B, n_steps)
    first_S = None
    cores = torch.empty(n_steps, B, H, D, device="cuda")
    for i, s in enumerate(steps):
        kda.kda_decode(cuda(s["qkv"], torch.bfloat16), cuda(s["gate"]), cuda(s["beta"]), table,
                       cores[i], B=B, heads=H, head_dim=D, scale=scale)
        if i == 0:
            first_S = st.cpu().numpy()
    torch.cuda.synchronize()
    got = cores.cpu().numpy()
    # step 1, every sequence
    for b in range(B):
        ref_core, ref_S, _ = _oracle_seq(steps[:1], S0[b], b, H, D, scale)
        assert relerr(got[0, b], ref_core[0]) < TOL
        assert relerr(first_S[b], ref_S) < TOL
    # 64 steps, sampled sequences
    final = st.cpu().numpy()
    for b in (0, 101, 255):
        ref_core, ref_S, _ = _oracle_seq(steps, S0[b], b, H, D, scale)
        assert relerr(got[:, b], ref_core) < TOL
        assert relerr(final[b], ref_S) < TOL


@pytest.mark.parametrize("B,K,H,D", [(6, 4, 2, 16), (6, 4, 4, 128), (64, 4, 32, 128), (3, 1, 2, 128)])
def test_write_on_accept_equals_snapshots(B, K, H, D):
    """Verify then fold ("Glm5NextLayer" page, write-on-accept): the verify's
    rows are bitwise those of decode_k and leave the states alone; folding
    n_accept rows leaves exactly decode_k's snapshot after that row (the
    starting state for 0, decode_k's final state for K).  n_accept runs over
    every value 0..K and two out-of-range values, which clamp."""
    import gated_delta_rule_bounded_amd as kda
    scale = D ** -0.5
    seed = 4100 + B + K
    rows, S0, ck, sk, snaps = _decode_k_vs_serial(B, K, H, D, seed)
    qkv = cuda(torch.stack([r["qkv"] for r in rows], 1).reshape(B * K, -1), torch.bfloat16)
    gate = cuda(np.stack([r["gate"] for r in rows], 1).reshape(B * K, H, D))
    beta = cuda(np.stack([r["beta"] for r in rows], 1).reshape(B * K, H))
    st = cuda(S0)
    tab = kda.ptr_table(st)
    core = torch.empty(B * K, H, D, device="cuda")
    say("verify_k", B, K, H, D)
    kda.kda_verify_k(qkv, gate, beta, tab, core, B=B, K=K, heads=H, head_dim=D, scale=scale)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(core.view(B, K, H, D).cpu().numpy(), ck)
    np.testing.assert_array_equal(st.cpu().numpy(), S0)
    na = np.array([(b % (K + 3)) - 1 for b in range(B)], np.int32)   # -1, 0, .., K, K+1, ...
    # the run-time report: out-of-range counts set KDA_REPORT_ACCEPT_CLAMPED
    # (4), in-range ones leave the word as it was
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    say("fold_accepted", B, K, H, D)
    kda.kda_fold_accepted(qkv, gate, beta, tab, torch.from_numpy(na).cuda(), B=B, K=K, heads=H,
                          head_dim=D, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == (4 if np.any((na < 0) | (na > K)) else 0)
    st_in = cuda(S0)
    ok_na = torch.from_numpy(np.clip(na, 0, K)).cuda()
    status.zero_()
    kda.kda_fold_accepted(qkv, gate, beta, kda.ptr_table(st_in), ok_na, B=B, K=K, heads=H,
                          head_dim=D, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    np.testing.assert_array_equal(st_in.cpu().numpy(), st.cpu().numpy())
    got = st.cpu().numpy()
    sn = snaps.view(B, K - 1, H, D, D).cpu().numpy() if K > 1 else None
    for b in range(B):
        n = min(max(int(na[b]), 0), K)
        want = S0[b] if n == 0 else (sk[b] if n == K else sn[b, n - 1])
        np.testing.assert_array_equal(got[b], want, err_msg=f"seq {b} n_accept {na[b]}")


@pytest.mark.parametrize("B,K,H,D", [(6, 4, 2, 16), (6, 4, 4, 128), (64, 4, 32, 128),
                                     (24, 20, 2, 128), (300, 3, 1, 128)])
def test_write_on_accept_table_form(B, K, H, D):
    """Table form of write-on-accept ("Glm5NextLayer" page, the WY tables of
    gdn_verify_run_batched / gdn_fold_accepted): the verify's rows are bitwise
    those of decode_k and leave the states alone; folding n_accept rows from
    the verify's u rows in one pass gives decode_k's snapshot after that row
    up to rounding, and the oracle's state after that row.  n_accept runs
    over 0..K and two out-of-range values, which clamp and are reported;
    0 leaves the state bitwise as it was.  K = 20 takes the fold's row
    blocks (16 rows) twice; 300 x 1 heads the whole-head launch."""
    import gated_delta_rule_bounded_amd as kda
    scale = D ** -0.5
    seed = 4300 + B + K
    rows, S0, ck, sk, snaps = _decode_k_vs_serial(B, K, H, D, seed)
    qkv = cuda(torch.stack([r["qkv"] for r in rows], 1).reshape(B * K, -1), torch.bfloat16)
    gate = cuda(np.stack([r["gate"] for r in rows], 1).reshape(B * K, H, D))
    beta = cuda(np.stack([r["beta"] for r in rows], 1).reshape(B * K, H))
    st = cuda(S0)
    tab = kda.ptr_table(st)
    wy = torch.full((B, H, K, D), float("nan"), device="cuda")
    core = torch.empty(B * K, H, D, device="cuda")
    say("verify_wy_k", B, K, H, D)
    kda.kda_verify_wy_k(qkv, gate, beta, tab, kda.ptr_table(wy), core, B=B, K=K, heads=H,
                        head_dim=D, scale=scale)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(core.view(B, K, H, D).cpu().numpy(), ck)
    np.testing.assert_array_equal(st.cpu().numpy(), S0)
    assert torch.isfinite(wy).all()
    na = np.array([(b % (K + 3)) - 1 for b in range(B)], np.int32)   # -1, 0, .., K, K+1, ...
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    say("fold_wy", B, K, H, D)
    kda.kda_fold_wy(qkv, gate, tab, kda.ptr_table(wy), torch.from_numpy(na).cuda(), B=B, K=K,
                    heads=H, head_dim=D, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == (4 if np.any((na < 0) | (na > K)) else 0)
    got = st.cpu().numpy()
    sn = snaps.view(B, K - 1, H, D, D).cpu().numpy() if K > 1 else None
    checked = 0
    for b in range(B):
        n = min(max(int(na[b]), 0), K)
        if n == 0:
            np.testing.assert_array_equal(got[b], S0[b], err_msg=f"seq {b} untouched")
            continue
        want = sk[b] if n == K else sn[b, n - 1]
        # the closed form against decode_k's row-by-row state: rounding only
        assert relerr(got[b], want) < 1e-5, f"seq {b} n_accept {na[b]}"
        if checked < 4:   # and against the oracle's state after row n - 1
            checked += 1
            _, ref_S, _ = _oracle_seq(rows[:n], S0[b], b, H, D, scale)
            assert relerr(got[b], ref_S) < TOL, f"seq {b} n_accept {na[b]} vs oracle"


def test_decode_k_bits_do_not_depend_on_batch_size():
    """The recurrent kernel splits each head's state over 4, 2 or 1
    workgroups by value columns depending on the batch size, with the key-axis
    sums in one fixed order, so a sequence's rows, final state and snapshots
    are the same bits whatever batch it is decoded in (B = 1, 2 and 6 run
    column slices; 16 runs whole heads) — a verify at one batch size matches
    plain decode at another."""
    import gated_delta_rule_bounded_amd as kda
    H, D, K = 32, 128, 3
    scale = D ** -0.5
    Bmax = 16
    S0 = workloads.state(H, D, 0.05, 4300, B=Bmax)
    rows = _steps(Bmax, H, D, K, 4310)
    qkv = torch.stack([r["qkv"] for r in rows], 1)                      # [B, K, 3HD]
    gate = np.stack([r["gate"] for r in rows], 1)
    beta = np.stack([r["beta"] for r in rows], 1)
    results = {}
    for B in (1, 2, 6, 16):
        st = cuda(S0[:B])
        snaps = torch.empty(B * (K - 1), H, D, D, device="cuda")
        core = torch.empty(B * K, H, D, device="cuda")
        say("decode_k batch", B)
        kda.kda_decode_k(cuda(qkv[:B].reshape(B * K, -1), torch.bfloat16),
                         cuda(gate[:B].reshape(B * K, H, D)), cuda(beta[:B].reshape(B * K, H)),
                         kda.ptr_table(st), core, B=B, K=K, heads=H, head_dim=D, scale=scale,
                         snap=kda.ptr_table(snaps))
        torch.cuda.synchronize()
        results[B] = (core.view(B, K, H, D)[0].clone(), st[0].clone(), snaps.view(B, K - 1, H, D, D)[0].clone())
    ref = results[16]
    for B in (1, 2, 6):
        for a, b_ in zip(results[B], ref):
            assert torch.equal(a, b_), B
    ref_core, ref_S, _ = _oracle_seq(rows, S0[0], 0, H, D, scale)
    assert relerr(ref[0].cpu().numpy(), ref_core) < TOL
    assert relerr(ref[1].cpu().numpy(), ref_S) < TOL
