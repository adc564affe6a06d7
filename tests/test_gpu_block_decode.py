"""Block-level decode on the GPU: the row-order-exact batched-M projection
(dense_gemv_bf16_batchm) and kda_block_decode / kda_block_decode_k against
the oracle's block, and K-row verify against K serial single-token calls.

Tolerances.  A projection's fp32-accumulated sum may round to the bf16
neighbour of the oracle's fp64 sum, so the projection outputs and
everything downstream of them are held to the bf16-stage bound 2e-2 (max
relative error per tensor), as for the block prefill.  K-row verify against
K single-token calls is bitwise: every stage buffer, the block output, the
final recurrent and conv states and every snapshot ("Glm5NextKdaLayer" page,
decode_k: an accepted draft token must be exactly what plain decode emits).
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_bounded_amd as kda
import workloads
from conftest import relerr
from kda_cases import say

pytestmark = pytest.mark.gpu
TOL = 2e-2

STAGES = ("qkv_proj", "conv_out", "fa", "g_raw", "b_raw", "gate", "beta", "core", "ga",
          "out_gate", "o_norm_out")


# --------------------------------------------------------------------------
# dense_gemv_bf16_batchm
# --------------------------------------------------------------------------

@pytest.mark.parametrize("M,N,Kd", [(1, 48, 96), (4, 4096, 4096), (7, 40, 4096), (70, 136, 256),
                                    (16, 32, 4096), (3, 4096, 128), (5, 64, 4224), (12, 48, 4224),
                                    (24, 96, 4096), (33, 40, 4096)])
def test_gemv_matches_oracle(orc, M, N, Kd):
    r = np.random.default_rng(M * 7 + N + Kd)
    x = workloads.to_bf16(r.standard_normal((M, Kd)))
    w = workloads.to_bf16(r.normal(0.0, 0.02, size=(N, Kd)))
    y = torch.full((M, N), 7.0, dtype=torch.bfloat16, device="cuda")
    say("gemv", M, N, Kd)
    kda.dense_gemv_bf16_batchm(x.cuda(), w.cuda(), y, M=M, N=N, Kd=Kd)
    torch.cuda.synchronize()
    ref = orc.linear(x.double().numpy(), w.double().numpy())
    got = y.float().cpu().numpy()
    assert relerr(got, ref) < TOL
    # fp32 accumulation of bf16 products: at most one bf16 step off per element
    step = np.abs(ref) * 2.0 ** -7 + 1e-30
    assert np.all(np.abs(got - ref) <= step + 1e-5 * np.max(np.abs(ref)))


def test_gemv_rows_are_order_exact():
    # each row's result is the same bits whether computed alone, among M rows,
    # at another position among them, or past the first 64-row group
    # N = 4096: a different accumulation order flips the bf16 rounding of
    # about one element in 30 000, so ~290 k compared elements expose it
    M, N, Kd = 70, 4096, 4096
    r = np.random.default_rng(99)
    x = workloads.to_bf16(r.standard_normal((M, Kd))).cuda()
    w = workloads.to_bf16(r.normal(0.0, 0.02, size=(N, Kd))).cuda()
    say("gemv rows", M, N, Kd)
    y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    kda.dense_gemv_bf16_batchm(x, w, y, M=M, N=N, Kd=Kd)
    perm = torch.from_numpy(r.permutation(M)).cuda()
    yp = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    kda.dense_gemv_bf16_batchm(x[perm].contiguous(), w, yp, M=M, N=N, Kd=Kd)
    singles = []
    for m in (0, 3, 17, 63, 64, 69):
        y1 = torch.empty(1, N, dtype=torch.bfloat16, device="cuda")
        kda.dense_gemv_bf16_batchm(x[m:m + 1], w, y1, M=1, N=N, Kd=Kd)
        singles.append((m, y1))
    # the row counts run different kernel instances (one row tile with
    # four-step load stages up to 16 rows, its x rows through LDS past 8;
    # two row tiles up to 32 and four past that, two-step stages, x rows
    # through LDS); all accumulate in one order
    groups = {}
    for m0, M_ in ((30, 4), (40, 3), (8, 8), (20, 16), (2, 5), (50, 12), (10, 24), (5, 32),
                   (1, 40)):
        yg = torch.empty(M_, N, dtype=torch.bfloat16, device="cuda")
        kda.dense_gemv_bf16_batchm(x[m0:m0 + M_], w, yg, M=M_, N=N, Kd=Kd)
        groups[(m0, M_)] = yg
    torch.cuda.synchronize()
    assert torch.equal(yp, y[perm])
    for m, y1 in singles:
        assert torch.equal(y1[0], y[m]), m
    for (m0, M_), yg in groups.items():
        assert torch.equal(yg, y[m0:m0 + M_]), (m0, M_)


def test_gemv_rows_are_order_exact_with_ragged_steps():
    # Kd = 4224: 33 contraction steps per wave, a whole number of load stages
    # for neither kernel instance, so both run passes with dummy slots; the
    # accumulation order must still be the same in both
    M, N, Kd = 70, 2048, 4224
    r = np.random.default_rng(123)
    x = workloads.to_bf16(r.standard_normal((M, Kd))).cuda()
    w = workloads.to_bf16(r.normal(0.0, 0.02, size=(N, Kd))).cuda()
    say("gemv ragged steps", M, N, Kd)
    y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    kda.dense_gemv_bf16_batchm(x, w, y, M=M, N=N, Kd=Kd)
    parts = []
    for m0, M_ in ((0, 1), (69, 1), (10, 4), (33, 16), (40, 20), (3, 9), (20, 33)):
        yg = torch.empty(M_, N, dtype=torch.bfloat16, device="cuda")
        kda.dense_gemv_bf16_batchm(x[m0:m0 + M_], w, yg, M=M_, N=N, Kd=Kd)
        parts.append((m0, M_, yg))
    torch.cuda.synchronize()
    for m0, M_, yg in parts:
        assert torch.equal(yg, y[m0:m0 + M_]), (m0, M_)


# --------------------------------------------------------------------------
# kda_block_decode / kda_block_decode_k
# --------------------------------------------------------------------------

def _case(B, K, H, D, hidden, rank, seed, w_std=0.05):
    x, w = workloads.block_raw(B * K, hidden, H, D, rank, 4, seed, w_std=w_std)
    S0 = workloads.state(H, D, 0.05, seed + 1000, B=B)
    conv0 = workloads.conv_raw(1, H, D, 4, seed + 2000, n_seq=B)["state"]
    return x, w, S0, conv0


def _gpu_decode_k(x, w, S0, conv0, B, K, H, D, hidden, rank, scale, snapshots=True):
    dev = torch.device("cuda")
    wd = {n: t.to(dev).contiguous() for n, t in w.items()}
    states = [torch.from_numpy(np.ascontiguousarray(S0[b])).to(dev) for b in range(B)]
    convs = [conv0[b].to(dev).contiguous() for b in range(B)]
    snaps = [torch.full((H, D, D), 5.0, device=dev) for _ in range(B * (K - 1))]
    csnaps = [torch.zeros(4, 3 * H * D, dtype=torch.bfloat16, device=dev)
              for _ in range(B * (K - 1))]
    buf = kda.block_decode_buffers(B * K, heads=H, head_dim=D, rank=rank, device=dev)
    out = torch.empty(B * K, hidden, dtype=torch.bfloat16, device=dev)
    say("block decode_k", B, K, hidden, H, D, rank)
    kda.kda_block_decode_k(x.to(dev).contiguous(), wd, kda.ptr_table(states),
                           kda.ptr_table(convs), buf, out, B=B, K=K, hidden_size=hidden,
                           heads=H, head_dim=D, rank=rank, scale=scale,
                           snap=kda.ptr_table(snaps) if snapshots and K > 1 else None,
                           conv_snap=kda.ptr_table(csnaps) if snapshots and K > 1 else None)
    torch.cuda.synchronize()
    res = {n: buf[n].float().cpu().numpy() for n in STAGES}
    res["final_out"] = out.float().cpu().numpy()
    res["state"] = np.stack([s.cpu().numpy() for s in states])
    res["conv_state"] = np.stack([c.float().cpu().numpy() for c in convs])
    if K > 1:
        res["state_snaps"] = np.stack([s.cpu().numpy() for s in snaps]).reshape(B, K - 1, H, D, D)
        res["conv_snaps"] = np.stack([c.float().cpu().numpy() for c in csnaps]).reshape(
            B, K - 1, 4, 3 * H * D)
    return res


def _gpu_serial(x, w, S0, conv0, B, K, H, D, hidden, rank, scale):
    """K kda_block_decode calls, one token of each sequence per call."""
    dev = torch.device("cuda")
    wd = {n: t.to(dev).contiguous() for n, t in w.items()}
    states = [torch.from_numpy(np.ascontiguousarray(S0[b])).to(dev) for b in range(B)]
    convs = [conv0[b].to(dev).contiguous() for b in range(B)]
    xs = x.view(B, K, hidden)
    per_row, snaps, csnaps = [], [], []
    for t in range(K):
        buf = kda.block_decode_buffers(B, heads=H, head_dim=D, rank=rank, device=dev)
        out = torch.empty(B, hidden, dtype=torch.bfloat16, device=dev)
        say("block decode", B, t, hidden, H, D, rank)
        kda.kda_block_decode(xs[:, t].contiguous().to(dev), wd, kda.ptr_table(states),
                             kda.ptr_table(convs), buf, out, B=B, hidden_size=hidden, heads=H,
                             head_dim=D, rank=rank, scale=scale)
        torch.cuda.synchronize()
        row = {n: buf[n].float().cpu().numpy() for n in STAGES}
        row["final_out"] = out.float().cpu().numpy()
        per_row.append(row)
        if t < K - 1:
            snaps.append(np.stack([s.cpu().numpy() for s in states]))
            csnaps.append(np.stack([c.float().cpu().numpy() for c in convs]))
    res = {n: np.stack([r[n] for r in per_row], 1).reshape((B * K,) + per_row[0][n].shape[1:])
           for n in per_row[0]}
    res["state"] = np.stack([s.cpu().numpy() for s in states])
    res["conv_state"] = np.stack([c.float().cpu().numpy() for c in convs])
    if K > 1:
        res["state_snaps"] = np.stack(snaps, 1)
        res["conv_snaps"] = np.stack(csnaps, 1)
    return res


def _check_oracle(orc, got, x, w, S0, conv0, B, K, H, D, hidden, scale):
    wd = {n: t.double().numpy() for n, t in w.items()}
    ref = orc.kda_block_decode_k(x.double().numpy().reshape(B, K, hidden), wd,
                                 np.asarray(S0, np.float64), conv0.double().numpy(), H, D, scale)
    for n in STAGES + ("final_out",):
        g = got[n].reshape((B, K) + ref[0][n].shape[1:])
        for b in range(B):
            e = relerr(g[b], ref[b][n])
            assert e < TOL, f"{n} seq {b}: relerr {e:.3e}"
    for b in range(B):
        assert relerr(got["state"][b], ref[b]["state"]) < TOL
        assert relerr(got["conv_state"][b], ref[b]["conv_state"]) < TOL
        if K > 1:
            for t in range(K - 1):
                assert relerr(got["state_snaps"][b, t], ref[b]["state_snaps"][t]) < TOL
                assert relerr(got["conv_snaps"][b, t], ref[b]["conv_snaps"][t]) < TOL


@pytest.mark.parametrize("B,K,H,D,hidden,rank", [
    (3, 4, 2, 16, 128, 32),
    (2, 5, 2, 128, 256, 32),
    (4, 1, 2, 16, 64, 32),
    (2, 5, 2, 16, 640, 32),      # f_a, g_a, b_proj split over the contraction
])
def test_block_decode_k_small_against_oracle(orc, B, K, H, D, hidden, rank):
    x, w, S0, conv0 = _case(B, K, H, D, hidden, rank, 1101 + K)
    scale = D ** -0.5
    got = _gpu_decode_k(x, w, S0, conv0, B, K, H, D, hidden, rank, scale)
    _check_oracle(orc, got, x, w, S0, conv0, B, K, H, D, hidden, scale)


@pytest.mark.parametrize("B,K,H,D,hidden,rank", [
    (3, 4, 2, 16, 128, 32),
    (2, 5, 2, 128, 256, 32),
    (5, 4, 2, 128, 256, 32),     # 20 verify rows against 5-row steps: two kernel instances
    (1, 17, 2, 16, 128, 32),     # the four-launch path against fused single rows
    (1, 17, 2, 16, 640, 32),     # the same with the low-rank products split
])
def test_block_decode_k_bitwise_equals_serial_decodes(B, K, H, D, hidden, rank):
    x, w, S0, conv0 = _case(B, K, H, D, hidden, rank, 1201 + K)
    scale = D ** -0.5
    got = _gpu_decode_k(x, w, S0, conv0, B, K, H, D, hidden, rank, scale)
    ser = _gpu_serial(x, w, S0, conv0, B, K, H, D, hidden, rank, scale)
    for n in STAGES + ("final_out", "state", "conv_state", "state_snaps", "conv_snaps"):
        np.testing.assert_array_equal(got[n], ser[n], err_msg=n)


@pytest.mark.parametrize("B,K,H,D,hidden,rank", [
    (3, 4, 2, 16, 128, 32),
    (2, 5, 4, 128, 256, 32),
    (2, 1, 4, 128, 256, 32),
    (1, 3, 2, 128, 256, 96),     # rank 96: three contraction steps, one quarter empty
    (1, 4, 2, 128, 256, 224),    # rank 224: uneven quarters, the four-launch path
    (2, 16, 2, 16, 128, 64),     # the most rows the fused kernel takes
    (1, 17, 2, 16, 128, 32),     # one more: the four-launch path
    (1, 17, 2, 16, 640, 32),     # the same with the low-rank products split
    (65, 2, 2, 16, 128, 32),     # many sequences in the fused kernel
    (65, 2, 2, 16, 640, 32),     # the same with the low-rank products split
    (3, 4, 2, 16, 640, 32),      # the fused kernel finishing the split products
])
def test_block_decode_k_stages_equal_standalone_kernels(B, K, H, D, hidden, rank):
    """The block decode runs the rank-R gate products, conv + SiLU + L2, the
    recurrence and the gated RMSNorm of each (head, sequence) in one kernel;
    its buffers and states must be the bits of dense_gemv_bf16_batchm,
    kda_gate, conv_silu_l2, kda_decode_k and gated_rmsnorm run one after the
    other on the block's own projection outputs."""
    x, w, S0, conv0 = _case(B, K, H, D, hidden, rank, 1251 + K)
    scale = D ** -0.5
    dev = torch.device("cuda")
    wd = {n: t.to(dev).contiguous() for n, t in w.items()}

    def fresh():
        st = [torch.from_numpy(np.ascontiguousarray(S0[b])).to(dev) for b in range(B)]
        cv = [conv0[b].to(dev).contiguous() for b in range(B)]
        sn = [torch.full((H, D, D), 5.0, device=dev) for _ in range(B * (K - 1))]
        cs = [torch.zeros(4, 3 * H * D, dtype=torch.bfloat16, device=dev)
              for _ in range(B * (K - 1))]
        return st, cv, sn, cs

    tab = lambda ts: kda.ptr_table(ts) if ts else None  # noqa: E731
    states, convs, snaps, csnaps = fresh()
    buf = kda.block_decode_buffers(B * K, heads=H, head_dim=D, rank=rank, device=dev)
    out = torch.empty(B * K, hidden, dtype=torch.bfloat16, device=dev)
    say("block decode_k vs stage kernels", B, K, H, D)
    kda.kda_block_decode_k(x.to(dev).contiguous(), wd, kda.ptr_table(states),
                           kda.ptr_table(convs), buf, out, B=B, K=K, hidden_size=hidden,
                           heads=H, head_dim=D, rank=rank, scale=scale, snap=tab(snaps),
                           conv_snap=tab(csnaps))
    states2, convs2, snaps2, csnaps2 = fresh()
    M, qkv = B * K, H * D
    g_raw = torch.empty_like(buf["g_raw"])
    kda.dense_gemv_bf16_batchm(buf["fa"], wd["f_b"], g_raw, M=M, N=qkv, Kd=rank)
    out_gate = torch.empty_like(buf["out_gate"])
    kda.dense_gemv_bf16_batchm(buf["ga"], wd["g_b"], out_gate, M=M, N=qkv, Kd=rank)
    gate = torch.empty_like(buf["gate"])
    beta = torch.empty_like(buf["beta"])
    kda.kda_gate(g_raw, wd["a_log"], wd["dt_bias"], gate, T=M, heads=H, head_dim=D,
                 b_raw=buf["b_raw"], beta=beta)
    y = torch.empty_like(buf["conv_out"])
    kda.conv_silu_l2(buf["qkv_proj"], wd["conv"], y, n_seq=B, rows=K, heads=H, head_dim=D,
                     conv_state=kda.ptr_table(convs2), conv_snap=tab(csnaps2))
    core = torch.empty_like(buf["core"])
    kda.kda_decode_k(y, buf["gate"], buf["beta"], kda.ptr_table(states2), core, B=B, K=K,
                     heads=H, head_dim=D, scale=scale, snap=tab(snaps2))
    onorm = torch.empty_like(buf["o_norm_out"])
    kda.gated_rmsnorm(core, buf["out_gate"], wd["o_norm"], onorm, T=B * K, heads=H, head_dim=D)
    torch.cuda.synchronize()
    assert torch.equal(g_raw, buf["g_raw"])
    assert torch.equal(out_gate, buf["out_gate"])
    assert torch.equal(gate, buf["gate"])
    assert torch.equal(beta, buf["beta"])
    assert torch.equal(y, buf["conv_out"])
    assert torch.equal(core, buf["core"])
    assert torch.equal(onorm, buf["o_norm_out"])
    for a, b in zip(states + convs + snaps + csnaps, states2 + convs2 + snaps2 + csnaps2):
        assert torch.equal(a, b)


@pytest.mark.parametrize("B,K", [
    (1, 4),
    (3, 4),      # several sequences in the fused kernel
    (1, 17),     # the six-launch path (with the split low-rank products and their finish)
])
def test_block_decode_k_full_size(orc, B, K):
    # the layer at full size (hidden 4096, 32 heads x 128, rank 128, weights
    # ~ N(0, 0.02)): sequences verifying K draft tokens, against the oracle
    # and bitwise against K single-token decodes
    H, D, hidden, rank = 32, 128, 4096, 128
    x, w, S0, conv0 = _case(B, K, H, D, hidden, rank, 1301 + 7 * B + K, w_std=0.02)
    scale = D ** -0.5
    got = _gpu_decode_k(x, w, S0, conv0, B, K, H, D, hidden, rank, scale)
    _check_oracle(orc, got, x, w, S0, conv0, B, K, H, D, hidden, scale)
    ser = _gpu_serial(x, w, S0, conv0, B, K, H, D, hidden, rank, scale)
    for n in STAGES + ("final_out", "state", "conv_state", "state_snaps", "conv_snaps"):
        np.testing.assert_array_equal(got[n], ser[n], err_msg=n)
    for n in STAGES + ("final_out",):
        assert np.all(np.isfinite(got[n])), n


@pytest.mark.parametrize("B,K,H,D,hidden,rank", [
    (7, 4, 2, 16, 128, 32),
    (6, 4, 2, 128, 256, 32),
    (1, 4, 32, 128, 4096, 128),
])
def test_block_write_on_accept_equals_snapshots(B, K, H, D, hidden, rank):
    """Block verify then fold ("Glm5NextLayer" page, write-on-accept): the
    verify's stage buffers and output are bitwise those of kda_block_decode_k
    and no state is written; folding n_accept rows leaves the recurrent and
    conv states bitwise equal to decode_k's snapshots after that row (the
    carried states for 0, decode_k's final states for K; out-of-range counts
    clamp)."""
    x, w, S0, conv0 = _case(B, K, H, D, hidden, rank, 1701 + B, w_std=0.05 if hidden < 4096 else 0.02)
    scale = D ** -0.5
    ref = _gpu_decode_k(x, w, S0, conv0, B, K, H, D, hidden, rank, scale)
    dev = torch.device("cuda")
    wd = {n: t.to(dev).contiguous() for n, t in w.items()}
    states = [torch.from_numpy(np.ascontiguousarray(S0[b])).to(dev) for b in range(B)]
    convs = [conv0[b].to(dev).contiguous() for b in range(B)]
    st_tab, cv_tab = kda.ptr_table(states), kda.ptr_table(convs)
    buf = kda.block_decode_buffers(B * K, heads=H, head_dim=D, rank=rank, device=dev)
    out = torch.empty(B * K, hidden, dtype=torch.bfloat16, device=dev)
    say("block verify_k", B, K, hidden, H, D, rank)
    kda.kda_block_verify_k(x.to(dev).contiguous(), wd, st_tab, cv_tab, buf, out, B=B, K=K,
                           hidden_size=hidden, heads=H, head_dim=D, rank=rank, scale=scale)
    torch.cuda.synchronize()
    for n in STAGES:
        np.testing.assert_array_equal(buf[n].float().cpu().numpy(), ref[n], err_msg=n)
    np.testing.assert_array_equal(out.float().cpu().numpy(), ref["final_out"])
    for b in range(B):
        np.testing.assert_array_equal(states[b].cpu().numpy(), S0[b])
        np.testing.assert_array_equal(convs[b].float().cpu().numpy(), conv0[b].float().numpy())
    na = np.array([(b % (K + 3)) - 1 for b in range(B)], np.int32) if B > 1 else np.array([2], np.int32)
    say("block fold_accepted", B, K, list(na))
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    kda.kda_block_fold_accepted(buf, st_tab, cv_tab, torch.from_numpy(na).cuda(), B=B, K=K,
                                heads=H, head_dim=D, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == (4 if np.any((na < 0) | (na > K)) else 0)
    for b in range(B):
        n = min(max(int(na[b]), 0), K)
        if n == 0:
            want_s, want_c = S0[b], conv0[b].float().numpy()
        elif n == K:
            want_s, want_c = ref["state"][b], ref["conv_state"][b]
        else:
            want_s, want_c = ref["state_snaps"][b, n - 1], ref["conv_snaps"][b, n - 1]
        np.testing.assert_array_equal(states[b].cpu().numpy(), want_s, err_msg=f"seq {b} state")
        np.testing.assert_array_equal(convs[b].float().cpu().numpy(), want_c,
                                      err_msg=f"seq {b} conv state")


@pytest.mark.parametrize("B,K,H,D,hidden,rank", [
    (7, 4, 2, 16, 128, 32),
    (6, 4, 2, 128, 256, 32),
    (1, 4, 32, 128, 4096, 128),
    (2, 1, 2, 128, 256, 32),
    (2, 17, 2, 16, 128, 32),     # 17 rows: the four-launch path
])
def test_block_write_on_accept_table_form(B, K, H, D, hidden, rank):
    """The block's write-on-accept in table form ("Glm5NextLayer" page, the
    verify's WY tables and the fold through them): the verify's stage
    buffers and output are bitwise those of kda_block_decode_k and no state
    is written; folding n_accept rows from the u rows leaves the recurrent
    state equal to decode_k's snapshot after that row up to rounding and the
    conv state bitwise equal to it; 0 rows leave both untouched."""
    x, w, S0, conv0 = _case(B, K, H, D, hidden, rank, 1801 + B, w_std=0.05 if hidden < 4096 else 0.02)
    scale = D ** -0.5
    ref = _gpu_decode_k(x, w, S0, conv0, B, K, H, D, hidden, rank, scale)
    dev = torch.device("cuda")
    wd = {n: t.to(dev).contiguous() for n, t in w.items()}
    states = [torch.from_numpy(np.ascontiguousarray(S0[b])).to(dev) for b in range(B)]
    convs = [conv0[b].to(dev).contiguous() for b in range(B)]
    st_tab, cv_tab = kda.ptr_table(states), kda.ptr_table(convs)
    wy = torch.full((B, H, K, D), float("nan"), device=dev)
    wy_tab = kda.ptr_table(wy)
    buf = kda.block_decode_buffers(B * K, heads=H, head_dim=D, rank=rank, device=dev)
    out = torch.empty(B * K, hidden, dtype=torch.bfloat16, device=dev)
    say("block verify_wy_k", B, K, hidden, H, D, rank)
    kda.kda_block_verify_wy_k(x.to(dev).contiguous(), wd, st_tab, cv_tab, wy_tab, buf, out, B=B,
                              K=K, hidden_size=hidden, heads=H, head_dim=D, rank=rank,
                              scale=scale)
    torch.cuda.synchronize()
    for n in STAGES:
        np.testing.assert_array_equal(buf[n].float().cpu().numpy(), ref[n], err_msg=n)
    np.testing.assert_array_equal(out.float().cpu().numpy(), ref["final_out"])
    assert torch.isfinite(wy).all()
    for b in range(B):
        np.testing.assert_array_equal(states[b].cpu().numpy(), S0[b])
        np.testing.assert_array_equal(convs[b].float().cpu().numpy(), conv0[b].float().numpy())
    na = (np.array([(b % (K + 3)) - 1 for b in range(B)], np.int32) if B > 2
          else np.array([min(2, K), 0][:B], np.int32))
    say("block fold_wy", B, K, list(na))
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    kda.kda_block_fold_wy(buf, st_tab, cv_tab, wy_tab, torch.from_numpy(na).cuda(), B=B, K=K,
                          heads=H, head_dim=D, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == (4 if np.any((na < 0) | (na > K)) else 0)
    for b in range(B):
        n = min(max(int(na[b]), 0), K)
        got_s, got_c = states[b].cpu().numpy(), convs[b].float().cpu().numpy()
        if n == 0:
            np.testing.assert_array_equal(got_s, S0[b])
            np.testing.assert_array_equal(got_c, conv0[b].float().numpy())
            continue
        want_s, want_c = ((ref["state"][b], ref["conv_state"][b]) if n == K else
                          (ref["state_snaps"][b, n - 1], ref["conv_snaps"][b, n - 1]))
        assert relerr(got_s, want_s) < 1e-5, f"seq {b} n_accept {na[b]} state"
        np.testing.assert_array_equal(got_c, want_c, err_msg=f"seq {b} conv state")


@pytest.mark.parametrize("B,K,H,D,hidden,rank", [
    (2, 4, 2, 128, 256, 32),
    (2, 4, 2, 16, 640, 32),      # the low-rank products split (chunk sums in the output buffer)
    (1, 17, 2, 16, 640, 32),     # the six-launch path with the split and its finish kernel
])
def test_block_decode_k_graph_replay_matches_eager(B, K, H, D, hidden, rank):
    """The block verify (stream-ordered launches, no allocation, no memset,
    no synchronisation) captured once in a HIP graph and replayed
    several times, with eager work and synchronisation between replays: every
    replay equals the eager call bit for bit (output, states, snapshots)."""
    x, w, S0, conv0 = _case(B, K, H, D, hidden, rank, 1801)
    scale = D ** -0.5
    ref = _gpu_decode_k(x, w, S0, conv0, B, K, H, D, hidden, rank, scale)
    dev = torch.device("cuda")
    wd = {n: t.to(dev).contiguous() for n, t in w.items()}
    xg = x.to(dev).contiguous()
    S0g = torch.from_numpy(np.ascontiguousarray(S0)).to(dev)
    C0g = conv0.to(dev).contiguous()
    states = [torch.empty(H, D, D, device=dev) for _ in range(B)]
    convs = [torch.empty(4, 3 * H * D, dtype=torch.bfloat16, device=dev) for _ in range(B)]
    snaps = [torch.empty(H, D, D, device=dev) for _ in range(B * (K - 1))]
    csnaps = [torch.empty(4, 3 * H * D, dtype=torch.bfloat16, device=dev) for _ in range(B * (K - 1))]
    tabs = [kda.ptr_table(t) for t in (states, convs, snaps, csnaps)]
    buf = kda.block_decode_buffers(B * K, heads=H, head_dim=D, rank=rank, device=dev)
    out = torch.empty(B * K, hidden, dtype=torch.bfloat16, device=dev)

    def reset():
        for b in range(B):
            states[b].copy_(S0g[b])
            convs[b].copy_(C0g[b])

    def call():
        kda.kda_block_decode_k(xg, wd, tabs[0], tabs[1], buf, out, B=B, K=K, hidden_size=hidden,
                               heads=H, head_dim=D, rank=rank, scale=scale, snap=tabs[2],
                               conv_snap=tabs[3])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        reset()
        call()                      # warm-up outside capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    say("graph capture block decode_k", B, K)
    with torch.cuda.graph(graph):
        call()
    for rep in range(4):
        reset()                     # eager work between replays
        out.fill_(-1.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(out.float().cpu().numpy(), ref["final_out"], err_msg=f"replay {rep}")
        got_s = np.stack([s.cpu().numpy() for s in states])
        np.testing.assert_array_equal(got_s, ref["state"], err_msg=f"replay {rep} state")
        got_sn = np.stack([s.cpu().numpy() for s in snaps]).reshape(B, K - 1, H, D, D)
        np.testing.assert_array_equal(got_sn, ref["state_snaps"], err_msg=f"replay {rep} snaps")
        got_c = np.stack([c.float().cpu().numpy() for c in convs])
        np.testing.assert_array_equal(got_c, ref["conv_state"], err_msg=f"replay {rep} conv")


def test_block_decode_k_bound_call_matches_direct():
    """kda.bind: the block verify marshalled once and re-issued three times
    (states reset in between) gives the direct call's bits every time."""
    B, K, H, D, hidden, rank = 2, 4, 2, 128, 256, 32
    x, w, S0, conv0 = _case(B, K, H, D, hidden, rank, 1901)
    scale = D ** -0.5
    ref = _gpu_decode_k(x, w, S0, conv0, B, K, H, D, hidden, rank, scale)
    dev = torch.device("cuda")
    wd = {n: t.to(dev).contiguous() for n, t in w.items()}
    xg = x.to(dev).contiguous()
    S0g = torch.from_numpy(np.ascontiguousarray(S0)).to(dev)
    C0g = conv0.to(dev).contiguous()
    states = [torch.empty(H, D, D, device=dev) for _ in range(B)]
    convs = [torch.empty(4, 3 * H * D, dtype=torch.bfloat16, device=dev) for _ in range(B)]
    snaps = [torch.empty(H, D, D, device=dev) for _ in range(B * (K - 1))]
    csnaps = [torch.empty(4, 3 * H * D, dtype=torch.bfloat16, device=dev) for _ in range(B * (K - 1))]
    tabs = [kda.ptr_table(t) for t in (states, convs, snaps, csnaps)]
    buf = kda.block_decode_buffers(B * K, heads=H, head_dim=D, rank=rank, device=dev)
    out = torch.empty(B * K, hidden, dtype=torch.bfloat16, device=dev)
    say("bound block decode_k", B, K)
    again = kda.bind(kda.kda_block_decode_k, xg, wd, tabs[0], tabs[1], buf, out, B=B, K=K,
                     hidden_size=hidden, heads=H, head_dim=D, rank=rank, scale=scale,
                     snap=tabs[2], conv_snap=tabs[3])
    for rep in range(3):
        for b in range(B):
            states[b].copy_(S0g[b])
            convs[b].copy_(C0g[b])
        out.fill_(-1.0)
        again()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(out.float().cpu().numpy(), ref["final_out"], err_msg=f"call {rep}")
        np.testing.assert_array_equal(np.stack([s.cpu().numpy() for s in states]), ref["state"],
                                      err_msg=f"call {rep} state")
        np.testing.assert_array_equal(
            np.stack([s.cpu().numpy() for s in snaps]).reshape(B, K - 1, H, D, D),
            ref["state_snaps"], err_msg=f"call {rep} snaps")
