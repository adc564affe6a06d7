"""kda_gate, conv_silu_l2 and gated_rmsnorm on the GPU against the oracle.

Tolerances: fp32 outputs (gate, beta) max relative error < 2e-3; bf16 stage
outputs (conv_out, o_norm_out) < 2e-2.  The conv state and snapshots are
copies of input rows and must match bit for bit.  The conv's K-row snapshot
mode must equal K single-row calls bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from conftest import relerr
from kda_cases import cuda, say

pytestmark = pytest.mark.gpu
TOL32, TOL16 = 2e-3, 2e-2


@pytest.mark.parametrize("T,H,D", [(300, 4, 128), (37, 2, 16), (8192, 32, 128)])
def test_kda_gate_matches_oracle(T, H, D):
    import gated_delta_rule_bounded_amd as kda
    r = np.random.default_rng(5000 + T)
    g_raw = workloads.to_bf16(r.standard_normal((T, H * D)) * 2.0)
    b_raw = workloads.to_bf16(r.standard_normal((T, H)) * 3.0)
    a_log, dt = workloads.gate_params(H, D, 5001)
    T_pad = T + 5
    gate = torch.full((T_pad, H, D), 7.0, device="cuda")
    beta = torch.full((T_pad, H), 7.0, device="cuda")
    say("gate", T, H, D)
    kda.kda_gate(cuda(g_raw, torch.bfloat16), cuda(a_log), cuda(dt), gate, T=T, heads=H,
                 head_dim=D, b_raw=cuda(b_raw, torch.bfloat16), beta=beta)
    torch.cuda.synchronize()
    ref_g, ref_b = oracle.kda_gate(g_raw.double().numpy(), a_log, dt, H, D,
                                   b_raw=b_raw.double().numpy())
    g, b = gate.cpu().numpy(), beta.cpu().numpy()
    assert relerr(g[:T], ref_g) < TOL32
    assert relerr(b[:T], ref_b) < TOL32
    # elementwise too: every decay factor is close, not only the largest
    assert np.max(np.abs(g[:T] - ref_g) / np.maximum(np.abs(ref_g), 1e-3)) < TOL32
    assert np.all(g[T:] == 7.0) and np.all(b[T:] == 7.0)
    assert np.all(g[:T] <= 0.0)


def _conv_gpu(x, w, states, n_seq, rows, H, D, snaps=False, widen=False):
    import gated_delta_rule_bounded_amd as kda
    cd = 3 * H * D
    xs = cuda(x, torch.bfloat16)
    st = cuda(states, torch.bfloat16).contiguous()             # [n_seq, 4, cd]
    y = torch.zeros(n_seq * rows, cd, dtype=torch.bfloat16, device="cuda")
    sn = (torch.zeros(n_seq * max(rows - 1, 1), 4, cd, dtype=torch.bfloat16, device="cuda")
          if snaps else None)
    w32 = [torch.full((n_seq * rows + 3, H * D), 7.0, device="cuda") for _ in range(3)] if widen else [None] * 3
    kda.conv_silu_l2(xs, cuda(w, torch.bfloat16), y, n_seq=n_seq, rows=rows, heads=H, head_dim=D,
                     conv_state=kda.ptr_table(st), conv_snap=kda.ptr_table(sn) if snaps else None,
                     q32=w32[0], k32=w32[1], v32=w32[2])
    torch.cuda.synchronize()
    return y, st, sn, w32


@pytest.mark.parametrize("rows,H,D", [(37, 2, 128), (5, 2, 16), (2, 4, 128), (1, 2, 16)])
def test_conv_matches_oracle(rows, H, D):
    raw = workloads.conv_raw(rows, H, D, 4, 6000 + rows, n_seq=1)
    say("conv", rows, H, D)
    y, st, _, w32 = _conv_gpu(raw["x"], raw["w"], raw["state"], 1, rows, H, D, widen=True)
    ref_y, ref_st, _ = oracle.conv_silu_l2(raw["x"].double().numpy(), raw["w"].double().numpy(),
                                           raw["state"][0].double().numpy(), H, D)
    yg = y.float().cpu().numpy()
    assert relerr(yg, ref_y) < TOL16
    for blk in range(3 * H):           # per head section, so small heads are checked too
        sl = slice(blk * D, (blk + 1) * D)
        assert relerr(yg[:, sl], ref_y[:, sl]) < TOL16
    assert np.array_equal(st[0].float().cpu().numpy(), ref_st)
    qkv = H * D
    for i, t in enumerate(w32):        # exact widening of y, rows past the end untouched
        assert torch.equal(t[:rows], y[:, i * qkv:(i + 1) * qkv].float())
        assert bool((t[rows:] == 7.0).all())


def test_conv_prefill_full_size_t8192():
    """T=8192 rows, H=32, D=128 (conv_dim 12288), zero initial conv state:
    the conv stage of the full block prefill."""
    T, H, D = 8192, 32, 128
    raw = workloads.conv_raw(T, H, D, 4, 6100, n_seq=1)
    zero = torch.zeros(1, 4, 3 * H * D, dtype=torch.bfloat16)
    say("conv full", T)
    y, st, _, _ = _conv_gpu(raw["x"], raw["w"], zero, 1, T, H, D)
    ref_y, ref_st, _ = oracle.conv_silu_l2(raw["x"].double().numpy(), raw["w"].double().numpy(),
                                           np.zeros((4, 3 * H * D)), H, D)
    assert relerr(y.float().cpu().numpy(), ref_y) < TOL16
    assert np.array_equal(st[0].float().cpu().numpy(), ref_st)


@pytest.mark.parametrize("n_seq,K,H,D", [(3, 4, 2, 16), (64, 4, 32, 128), (2, 20, 2, 128)])
def test_conv_k_rows_bitwise_equals_single_rows(n_seq, K, H, D):
    """K-row mode with snapshots == K single-row calls (y, state, snapshots),
    and both match the oracle."""
    import gated_delta_rule_bounded_amd as kda
    cd = 3 * H * D
    raw = workloads.conv_raw(n_seq * K, H, D, 4, 6200 + K, n_seq=n_seq)
    say("conv K-rows", n_seq, K, H, D)
    y, st, sn, _ = _conv_gpu(raw["x"], raw["w"], raw["state"], n_seq, K, H, D, snaps=True)
    # serial: one row per call; row t of every sequence via a strided view
    xs = cuda(raw["x"], torch.bfloat16).view(n_seq, K, cd)
    st2 = cuda(raw["state"], torch.bfloat16).contiguous()
    tab = kda.ptr_table(st2)
    w = cuda(raw["w"], torch.bfloat16)
    for t in range(K):
        yt = torch.zeros(n_seq, cd, dtype=torch.bfloat16, device="cuda")
        kda.conv_silu_l2(xs[:, t], w, yt, n_seq=n_seq, rows=1, heads=H, head_dim=D,
                         conv_state=tab)
        torch.cuda.synchronize()
        assert torch.equal(yt.view(torch.int16), y.view(n_seq, K, cd)[:, t].view(torch.int16))
        if t < K - 1:
            assert torch.equal(st2.view(torch.int16),
                               sn.view(n_seq, K - 1, 4, cd)[:, t].view(torch.int16))
    assert torch.equal(st2.view(torch.int16), st.view(torch.int16))
    for s in (0, n_seq - 1):
        ref_y, ref_st, ref_sn = oracle.conv_silu_l2(
            raw["x"][s * K:(s + 1) * K].double().numpy(), raw["w"].double().numpy(),
            raw["state"][s].double().numpy(), H, D, snapshots=True)
        assert relerr(y[s * K:(s + 1) * K].float().cpu().numpy(), ref_y) < TOL16
        assert np.array_equal(st[s].float().cpu().numpy(), ref_st)
        assert np.array_equal(sn.view(n_seq, K - 1, 4, cd)[s].float().cpu().numpy(), ref_sn)


@pytest.mark.parametrize("T,H,D", [(300, 4, 128), (33, 2, 16), (8192, 32, 128)])
def test_gated_rmsnorm_matches_oracle(T, H, D):
    import gated_delta_rule_bounded_amd as kda
    raw = workloads.norm_raw(T, H, D, 7000 + T)
    out = torch.zeros(T, H * D, dtype=torch.bfloat16, device="cuda")
    say("rmsnorm", T, H, D)
    kda.gated_rmsnorm(cuda(raw["core"]).view(T, H * D), cuda(raw["out_gate"], torch.bfloat16),
                      cuda(raw["w"], torch.bfloat16), out, T=T, heads=H, head_dim=D, eps=1e-5)
    torch.cuda.synchronize()
    ref = oracle.gated_rmsnorm(raw["core"], raw["out_gate"].double().numpy(),
                               raw["w"].double().numpy(), eps=1e-5)
    got = out.float().cpu().numpy()
    assert relerr(got, ref) < TOL16
    for h in range(H):
        assert relerr(got[:, h * D:(h + 1) * D], ref[:, h * D:(h + 1) * D]) < TOL16
