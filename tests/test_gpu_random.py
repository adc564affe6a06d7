"""Seeded random sweep over shapes on the GPU: each case draws T, chunk,
head_dim, heads, a pad fill and a state scale (or B and K for decode), runs
the entry point and checks it against the oracle (2e-3 max relative error,
fp32 work) or bitwise against the serial path, as the fixed-shape tests do.
The draws are fixed by the seed, so a failure names a reproducible case."""
import numpy as np
import pytest
import torch

import gated_delta_rule_bounded_amd as kda
import oracle
import workloads
from conftest import relerr
from kda_cases import core_case, cuda, gpu_prefill, oracle_core, say

pytestmark = pytest.mark.gpu
TOL = 2e-3
FILLS = (0.0, 1e30, np.nan, -7.0)


def _prefill_case(i):
    r = np.random.default_rng(9000 + i)
    D = int(r.choice([16, 128]))
    C = int(r.choice([16, 64]))
    H = int(r.integers(1, 5))
    T = int(r.integers(1, 300))
    T_pad = -(-T // C) * C + C * int(r.integers(0, 2))
    fill = FILLS[int(r.integers(0, len(FILLS)))]
    std = float(r.choice([0.0, 0.05, 0.5]))
    return D, C, H, T, T_pad, fill, std


@pytest.mark.parametrize("i", range(12))
def test_prefill_random_shapes(i):
    D, C, H, T, T_pad, fill, std = _prefill_case(i)
    scale = D ** -0.5
    case = core_case(T, H, D, 9100 + i, std)
    say("random prefill", i, D, C, H, T, T_pad, fill, std)
    core, S = gpu_prefill(case, T, T_pad, C, scale, fill=fill)
    ref_core, ref_S = oracle_core(case, scale)
    assert relerr(core[:T], ref_core) < TOL
    assert relerr(S, ref_S) < TOL
    assert np.all(core[T:] == 7.0)                   # rows past T untouched


@pytest.mark.parametrize("i", range(6))
def test_varlen_random_prompts(i):
    r = np.random.default_rng(9200 + i)
    D, C = int(r.choice([16, 128])), int(r.choice([16, 64]))
    H = int(r.integers(1, 4))
    lengths = [int(x) for x in r.integers(0, 150, size=int(r.integers(1, 7)))]
    scale = D ** -0.5
    cases = [core_case(T, H, D, 9300 + 10 * i + s, 0.05) for s, T in enumerate(lengths)]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    rows = int(cu[-1]) + C
    stack = lambda n, shape: cuda(np.concatenate(
        [c[n] for c in cases] + [np.full((C,) + shape, np.nan, np.float32)]))
    q, k, v, g = (stack(n, (H, D)) for n in ("q", "k", "v", "gate"))
    b = stack("beta", (H,))
    states = [cuda(c["S0"]).contiguous() for c in cases]
    core = torch.full((rows, H, D), 7.0, device="cuda")
    mx, tot = kda.varlen_chunks(lengths, C)
    ws = torch.empty(max(1, kda.kda_prefill_varlen_workspace_bytes(len(cases), tot, H, D, C)),
                     dtype=torch.uint8, device="cuda")
    say("random varlen", i, D, C, H, lengths)
    kda.kda_prefill_varlen(q, k, v, g, b, kda.ptr_table(states), core, torch.from_numpy(cu).cuda(),
                           ws, B=len(cases), rows=rows, max_chunks=mx, total_chunks=tot, heads=H,
                           head_dim=D, chunk=C, scale=scale)
    torch.cuda.synchronize()
    got = core.cpu().numpy()
    for s, (c, T) in enumerate(zip(cases, lengths)):
        if T == 0:
            np.testing.assert_array_equal(states[s].cpu().numpy(), c["S0"])
            continue
        ref_core, ref_S = oracle_core(c, scale)
        assert relerr(got[cu[s]:cu[s + 1]], ref_core) < TOL, s
        assert relerr(states[s].cpu().numpy(), ref_S) < TOL, s
    assert np.all(got[cu[-1]:] == 7.0)


@pytest.mark.parametrize("i", range(6))
def test_decode_k_verify_fold_random(i):
    r = np.random.default_rng(9400 + i)
    D = int(r.choice([16, 128]))
    H = int(r.integers(1, 5))
    B, K = int(r.integers(1, 9)), int(r.integers(1, 7))
    scale = D ** -0.5
    a_log, dt = workloads.gate_params(H, D, 9500 + i)
    steps = []
    for t in range(K):
        raw = workloads.decode_step_raw(B, H, D, 9600 + 10 * i + t)
        gg, bb = oracle.kda_gate(raw["g_raw"], a_log, dt, H, D, b_raw=raw["b_raw"])
        steps.append((raw["qkv"], gg.astype(np.float32), bb.astype(np.float32)))
    S0 = workloads.state(H, D, 0.05, 9700 + i, B=B)
    qkv = cuda(torch.stack([s[0] for s in steps], 1).reshape(B * K, -1), torch.bfloat16)
    gate = cuda(np.stack([s[1] for s in steps], 1).reshape(B * K, H, D))
    beta = cuda(np.stack([s[2] for s in steps], 1).reshape(B * K, H))
    st = cuda(S0)
    snaps = torch.empty(B * max(K - 1, 1), H, D, D, device="cuda")
    core = torch.empty(B * K, H, D, device="cuda")
    say("random decode_k", i, D, H, B, K)
    kda.kda_decode_k(qkv, gate, beta, kda.ptr_table(st), core, B=B, K=K, heads=H, head_dim=D,
                     scale=scale, snap=kda.ptr_table(snaps) if K > 1 else None)
    st2 = cuda(S0)
    core2 = torch.empty_like(core)
    kda.kda_verify_k(qkv, gate, beta, kda.ptr_table(st2), core2, B=B, K=K, heads=H, head_dim=D,
                     scale=scale)
    na = torch.from_numpy(r.integers(0, K + 1, size=B).astype(np.int32)).cuda()
    kda.kda_fold_accepted(qkv, gate, beta, kda.ptr_table(st2), na, B=B, K=K, heads=H, head_dim=D)
    torch.cuda.synchronize()
    assert torch.equal(core, core2)
    sn = snaps.view(B, max(K - 1, 1), H, D, D)
    for b in range(B):
        n = int(na[b])
        want = (cuda(S0[b]) if n == 0 else st[b] if n == K else sn[b, n - 1])
        assert torch.equal(st2[b], want), (b, n)
        qf = torch.stack([s[0][b] for s in steps]).double().numpy()
        ref_core, ref_S, _ = oracle.kda_recurrence(
            qf[:, :H * D].reshape(K, H, D), qf[:, H * D:2 * H * D].reshape(K, H, D),
            qf[:, 2 * H * D:].reshape(K, H, D), np.stack([s[1][b] for s in steps]),
            np.stack([s[2][b] for s in steps]), S0[b], scale)
        assert relerr(core.view(B, K, H, D)[b].cpu().numpy(), ref_core) < TOL
        assert relerr(st[b].cpu().numpy(), ref_S) < TOL
