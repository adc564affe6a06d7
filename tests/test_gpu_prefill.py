"""kda_prefill on the GPU against the token-serial oracle.

Tolerance: max relative error (max |gpu - oracle| / max |oracle|, per tensor)
below 2e-3 on core rows < T and on the carried state (fp32 work).  Poison in
the pad tail must change nothing, bit for bit.
"""
import numpy as np
import pytest
import torch

from conftest import relerr
from kda_cases import core_case, cuda, gpu_prefill, oracle_core, pad_rows, say

pytestmark = pytest.mark.gpu
TOL = 2e-3


@pytest.mark.parametrize("T,T_pad,C,state_std", [
    (64, 64, 16, 0.0), (64, 64, 16, 0.1),        # the tiny workload, both initial states
    (57, 64, 16, 0.1), (64, 80, 16, 0.1),         # ragged tail; a wholly padded chunk
    (64, 64, 64, 0.1), (50, 128, 64, 0.1),
])
def test_prefill_tiny_d16(T, T_pad, C, state_std):
    H, D = 2, 16
    case = core_case(T, H, D, 1000, state_std)
    scale = D ** -0.5
    say("prefill tiny", T, T_pad, C, state_std)
    core, S = gpu_prefill(case, T, T_pad, C, scale)
    ref_core, ref_S = oracle_core(case, scale)
    assert relerr(core[:T], ref_core) < TOL
    assert relerr(S, ref_S) < TOL
    assert np.all(core[T:] == 7.0), "core rows >= T must not be written"


@pytest.mark.parametrize("T,T_pad,C", [(300, 320, 64), (300, 304, 16), (128, 128, 64), (1, 64, 64)])
def test_prefill_d128_ragged(T, T_pad, C):
    H, D = 4, 128
    case = core_case(T, H, D, 1101, 0.05, qkv_bf16=True)
    scale = D ** -0.5
    say("prefill d128", T, T_pad, C)
    core, S = gpu_prefill(case, T, T_pad, C, scale)
    ref_core, ref_S = oracle_core(case, scale)
    assert relerr(core[:T], ref_core) < TOL
    assert relerr(S, ref_S) < TOL
    for h in range(H):
        assert relerr(core[:T, h], ref_core[:, h]) < TOL
        assert relerr(S[h], ref_S[h]) < TOL
    assert np.all(core[T:] == 7.0)


@pytest.mark.parametrize("fill", [1e30, float("nan"), -3.0])
@pytest.mark.parametrize("T,T_pad,C", [(57, 64, 16), (200, 256, 64), (64, 128, 64)])
def test_prefill_poisoned_tail_is_bitwise_inert(T, T_pad, C, fill):
    H, D = (2, 16) if C == 16 else (4, 128)
    case = core_case(T, H, D, 1202, 0.1)
    say("poison", T, T_pad, C, fill)
    core0, S0 = gpu_prefill(case, T, T_pad, C, D ** -0.5, fill=0.0)
    core1, S1 = gpu_prefill(case, T, T_pad, C, D ** -0.5, fill=fill)
    assert np.array_equal(core0[:T].view(np.int32), core1[:T].view(np.int32))
    assert np.array_equal(S0.view(np.int32), S1.view(np.int32))
    assert np.all(core1[T:] == 7.0)


@pytest.mark.parametrize("a", [1, 63, 64, 100])
def test_prefill_split_invariance(a):
    """[0,T) in one call equals [0,a) then [a,T) from the carried state."""
    T, H, D, C = 200, 4, 128, 64
    case = core_case(T, H, D, 1303, 0.05)
    scale = D ** -0.5
    say("split", a)
    core_all, S_all = gpu_prefill(case, T, 256, C, scale)
    first = {n: case[n][:a] for n in ("q", "k", "v", "gate", "beta")}
    first["S0"] = case["S0"]
    c1, S1 = gpu_prefill(first, a, ((a + C - 1) // C) * C, C, scale)
    second = {n: case[n][a:] for n in ("q", "k", "v", "gate", "beta")}
    second["S0"] = S1
    c2, S2 = gpu_prefill(second, T - a, ((T - a + C - 1) // C) * C, C, scale)
    ref_core, ref_S = oracle_core(case, scale)
    assert relerr(np.concatenate([c1[:a], c2[:T - a]]), ref_core) < TOL
    assert relerr(S2, ref_S) < TOL
    assert relerr(S2, S_all) < TOL


def test_prefill_unnormalised_qk_used_as_given():
    """q, k scaled by 1.01 (not unit): the kernel must not re-normalise."""
    T, H, D, C = 130, 2, 128, 64
    case = core_case(T, H, D, 1404, 0.05, qk_scale=1.01)
    say("prenorm contract")
    core, S = gpu_prefill(case, T, 192, C, 1.0)
    ref_core, ref_S = oracle_core(case, 1.0)
    assert relerr(core[:T], ref_core) < TOL
    assert relerr(S, ref_S) < TOL


@pytest.mark.parametrize("C", [16, 64])
def test_prefill_steep_decay_takes_exact_diagonal_path(C):
    """Gates scaled so some 16-row blocks decay by more than 2^86 inside the
    block (the fp32 chunk-16 form's limit for factoring its diagonal block)
    and others less; at chunk 64 the same gates run the split form.  Both
    must match the oracle."""
    T, H, D = 128, 2, 128
    case = core_case(T, H, D, 1505, 0.05, gate_scale=1.6)
    g2 = case["gate"] / np.log(2)           # log2 units, as the kernel measures spans
    spans = np.array([[(-g2[16 * b + 1:16 * b + 16, h].sum(0)).max() for h in range(H)]
                      for b in range(T // 16)])
    assert (spans > 86.0).any() and (spans <= 86.0).any(), "need both diagonal paths"
    say("steep decay", C)
    core, S = gpu_prefill(case, T, T, C, D ** -0.5)
    ref_core, ref_S = oracle_core(case, D ** -0.5)
    assert np.all(np.isfinite(core[:T])) and np.all(np.isfinite(S))
    assert relerr(core[:T], ref_core) < TOL
    assert relerr(S, ref_S) < TOL


def test_prefill_wide_chunks_take_exact_pairwise_path():
    """Split form (D = 128, chunk 64): chunks 1 and 3 get gates steep enough
    that a 16-row block decays by more than 2^96 (their A and P come from
    the exact pairwise sums), chunks 0 and 2 keep the factored path; both
    must match the oracle."""
    T, H, D, C = 256, 2, 128, 64
    case = core_case(T, H, D, 1507, 0.05)
    g = case["gate"].copy()
    g[64:128] *= 6.0
    g[192:256] *= 6.0
    case["gate"] = g.astype(np.float32)
    g2 = case["gate"] / np.log(2)
    blk = np.array([[(-g2[16 * b:16 * b + 16, h].sum(0)).max() for h in range(H)]
                    for b in range(T // 16)])
    assert (blk[4:8] > 96.0).any() and (blk[0:4] <= 96.0).all(), "need both paths"
    say("wide chunks", C)
    core, S = gpu_prefill(case, T, T, C, D ** -0.5)
    ref_core, ref_S = oracle_core(case, D ** -0.5)
    assert np.all(np.isfinite(core)) and np.all(np.isfinite(S))
    assert relerr(core, ref_core) < TOL
    assert relerr(S, ref_S) < TOL


def test_prefill_growing_gate_rows():
    """A few positive log-gates (growth instead of decay) in one chunk: the
    factored decay references do not apply there and that chunk takes the
    exact pairwise path; results still match the oracle."""
    T, H, D, C = 192, 2, 128, 64
    case = core_case(T, H, D, 1508, 0.05)
    g = case["gate"].copy()
    g[66:80] = 0.3
    case["gate"] = g.astype(np.float32)
    assert g[64:80].sum(0).max() > 0.0, "need a positive in-block cumulative log-gate"
    say("growing gate", C)
    core, S = gpu_prefill(case, T, T, C, D ** -0.5)
    ref_core, ref_S = oracle_core(case, D ** -0.5)
    assert relerr(core, ref_core) < TOL
    assert relerr(S, ref_S) < TOL


def test_prefill_empty_is_noop():
    import gated_delta_rule_bounded_amd as kda
    H, D = 2, 16
    st = torch.randn(H, D, D, device="cuda")
    before = st.clone()
    z = torch.zeros(64, H, D, device="cuda")
    core = torch.full((64, H, D), 7.0, device="cuda")
    ws = torch.empty(kda.kda_prefill_workspace_bytes(64, H, D, 16), dtype=torch.uint8, device="cuda")
    kda.kda_prefill(z, z, z, z, torch.zeros(64, H, device="cuda"), st, core, ws, T=0, T_pad=64,
                    heads=H, head_dim=D, chunk=16, scale=1.0)
    torch.cuda.synchronize()
    assert torch.equal(st, before) and bool((core == 7.0).all())


@pytest.mark.parametrize("T,T_pad,fill", [(4096, 4096, 0.0), (4059, 4096, 1e30), (4096, 4160, float("nan"))])
def test_prefill_full_size_h32_d128(T, T_pad, fill):
    """The chunked-prefill workload at full size: T=4096, H=32, D=128, chunk 64,
    q/k/v generated in bf16 and widened, state ~ N(0, 0.05); every output
    element against the oracle."""
    H, D, C = 32, 128, 64
    case = core_case(4096, H, D, 1001, 0.05, qkv_bf16=True)
    scale = D ** -0.5
    say("prefill full", T, T_pad, fill)
    core, S = gpu_prefill(case, T, T_pad, C, scale, fill=fill)
    ref_core, ref_S = oracle_core(case, scale, T=T)
    e_core, e_S = relerr(core[:T], ref_core), relerr(S, ref_S)
    print(f"relerr core {e_core:.3e} state {e_S:.3e}")
    assert e_core < TOL and e_S < TOL
    # and per head, for the core rows and the carried state alike
    for h in range(H):
        eh_c, eh_s = relerr(core[:T, h], ref_core[:, h]), relerr(S[h], ref_S[h])
        assert eh_c < TOL and eh_s < TOL, f"head {h}: core {eh_c:.3e} state {eh_s:.3e}"
    if T_pad > T:
        assert np.all(core[T:] == 7.0)


@pytest.mark.parametrize("T", [50, 64])
def test_prefill_one_chunk_whole_head_walks_bitwise(T):
    """A one-chunk prefill over 256 heads (the walk takes a whole head per
    workgroup) equals the same heads run 32 at a time (16-column walks), bit
    for bit, and the oracle."""
    H, D, C, G = 256, 128, 64, 32
    case = core_case(T, H, D, 1707, 0.05, qkv_bf16=True)
    say("one-chunk whole-head walks", T, H)
    core, S = gpu_prefill(case, T, 64, C, D ** -0.5)
    for h0 in range(0, H, G):
        sub = {n: np.ascontiguousarray(a[:, h0:h0 + G]) for n, a in case.items() if n != "S0"}
        sub["S0"] = np.ascontiguousarray(case["S0"][h0:h0 + G])
        core_g, S_g = gpu_prefill(sub, T, 64, C, D ** -0.5)
        assert np.array_equal(core[:, h0:h0 + G].view(np.int32), core_g.view(np.int32)), h0
        assert np.array_equal(S[h0:h0 + G].view(np.int32), S_g.view(np.int32)), h0
    heads = [0, 97, 255]
    sub = {n: np.ascontiguousarray(a[:, heads]) for n, a in case.items() if n != "S0"}
    sub["S0"] = np.ascontiguousarray(case["S0"][heads])
    ref_core, ref_S = oracle_core(sub, D ** -0.5)
    for i, h in enumerate(heads):
        assert relerr(core[:T, h], ref_core[:, i]) < TOL
        assert relerr(S[h], ref_S[i]) < TOL
    assert np.all(core[T:] == 7.0)


def test_prefill_phases_equal_one_call_bitwise():
    """kda_prefill_prepare then kda_prefill_forward == kda_prefill, bit for bit."""
    import gated_delta_rule_bounded_amd as kda
    from kda_cases import cuda, pad_rows
    T, T_pad, H, D, C = 300, 320, 4, 128, 64
    case = core_case(T, H, D, 1606, 0.05)
    core_a, S_a = gpu_prefill(case, T, T_pad, C, D ** -0.5)
    q, k, v, g, b = (cuda(pad_rows(case[n], T_pad, 0.0)) for n in ("q", "k", "v", "gate", "beta"))
    st = cuda(case["S0"]).contiguous()
    core = torch.full((T_pad, H, D), 7.0, device="cuda")
    ws = torch.empty(kda.kda_prefill_workspace_bytes(T_pad, H, D, C), dtype=torch.uint8, device="cuda")
    kw = dict(T=T, T_pad=T_pad, heads=H, head_dim=D, chunk=C)
    say("phases")
    kda.kda_prefill_prepare(q, k, v, g, b, ws, **kw)
    kda.kda_prefill_forward(st, core, ws, scale=D ** -0.5, **kw)
    torch.cuda.synchronize()
    assert np.array_equal(core.cpu().numpy().view(np.int32), core_a.view(np.int32))
    assert np.array_equal(st.cpu().numpy().view(np.int32), S_a.view(np.int32))



def test_prefill_prepare_longer_than_one_grid_dimension():
    """kda_prefill_prepare over more chunks than one grid dimension holds
    (65,537 chunks of 64 rows, one head of 128): it prepares them in pieces,
    and the two phases still equal kda_prefill, which walks cache-sized
    segments, bit for bit.  Inputs are generated on the GPU (about 23 GB of
    buffers), keys unit-norm and log-decays small, so the walk stays finite."""
    import gated_delta_rule_bounded_amd as kda
    H, D, C = 1, 128, 64
    NC = 65537
    T_pad = NC * C
    T = T_pad - 5
    say("prepare in pieces", T, H, D, C)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(2024)

    def rnd(*shape):
        return torch.randn(*shape, device="cuda", generator=gen)

    q = rnd(T_pad, H, D).mul_(D ** -0.5)
    k = rnd(T_pad, H, D)
    k.div_(k.norm(dim=-1, keepdim=True))
    v = rnd(T_pad, H, D)
    gate = torch.rand(T_pad, H, D, device="cuda", generator=gen).mul_(-0.1)
    beta = torch.sigmoid(rnd(T_pad, H))
    S0 = rnd(H, D, D).mul_(0.05)
    ws = torch.empty(kda.kda_prefill_workspace_bytes(T_pad, H, D, C), dtype=torch.uint8,
                     device="cuda")
    kw = dict(T=T, T_pad=T_pad, heads=H, head_dim=D, chunk=C)
    st_a = S0.clone()
    core_a = torch.full((T_pad, H, D), 7.0, device="cuda")
    kda.kda_prefill(q, k, v, gate, beta, st_a, core_a, ws, scale=D ** -0.5, **kw)
    st_b = S0.clone()
    core_b = torch.full((T_pad, H, D), 7.0, device="cuda")
    kda.kda_prefill_prepare(q, k, v, gate, beta, ws, **kw)
    kda.kda_prefill_forward(st_b, core_b, ws, scale=D ** -0.5, **kw)
    torch.cuda.synchronize()
    assert torch.isfinite(st_a).all()
    assert torch.equal(core_a.view(torch.int32), core_b.view(torch.int32))
    assert torch.equal(st_a.view(torch.int32), st_b.view(torch.int32))

@pytest.mark.parametrize("T,T_pad,H", [(2200, 2240, 64), (2200, 2240, 3), (513, 576, 32),
                                       (512, 512, 32), (65, 128, 5), (1, 64, 32),
                                       (4059, 4160, 32)])
def test_prefill_segments_equal_one_pass_bitwise(T, T_pad, H):
    """kda_prefill walks segments of kda_prefill_segment_chunks chunks, each
    prepared into the start of the workspace; at H = 64 a 2200-token prefill
    takes three segments (the last one ragged).  Core and state must equal one
    prepare + forward over all rows, bit for bit, at that size and at one-
    segment sizes; rows past T untouched; and the bf16-row form on the same
    values gives the same bits."""
    import gated_delta_rule_bounded_amd as kda
    D, C = 128, 64
    seg = kda.kda_prefill_segment_chunks(T, H, D, C)
    if H == 64:
        assert 1 < seg < -(-T // C), "need more than one segment"
    g = torch.Generator(device="cuda").manual_seed(1707 + T + H)
    rnd = lambda *shape: torch.randn(*shape, device="cuda", generator=g)
    bf = lambda x: x.to(torch.bfloat16).float()   # noqa: E731  (values a bf16 row holds)
    q = bf(torch.nn.functional.normalize(rnd(T_pad, H, D), dim=-1))
    k = bf(torch.nn.functional.normalize(rnd(T_pad, H, D), dim=-1))
    v = bf(rnd(T_pad, H, D) * 0.5)
    gate = -torch.rand(T_pad, H, D, device="cuda", generator=g) * 0.3
    beta = torch.rand(T_pad, H, device="cuda", generator=g)
    S0 = rnd(H, D, D) * 0.05
    kw = dict(T=T, T_pad=T_pad, heads=H, head_dim=D, chunk=C)
    ws = torch.empty(kda.kda_prefill_workspace_bytes(T_pad, H, D, C), dtype=torch.uint8, device="cuda")
    say("segments", T, H, seg)
    st_a, core_a = S0.clone(), torch.full((T_pad, H, D), 7.0, device="cuda")
    kda.kda_prefill(q, k, v, gate, beta, st_a, core_a, ws, scale=D ** -0.5, **kw)
    st_b, core_b = S0.clone(), torch.full((T_pad, H, D), 7.0, device="cuda")
    kda.kda_prefill_prepare(q, k, v, gate, beta, ws, **kw)
    kda.kda_prefill_forward(st_b, core_b, ws, scale=D ** -0.5, **kw)
    torch.cuda.synchronize()
    assert torch.equal(core_a.view(torch.int32), core_b.view(torch.int32))
    assert torch.equal(st_a.view(torch.int32), st_b.view(torch.int32))
    assert bool((core_a[T:] == 7.0).all())
    qkv = torch.cat([x.reshape(T_pad, H * D) for x in (q, k, v)], 1).to(torch.bfloat16)
    st_c, core_c = S0.clone(), torch.full((T_pad, H, D), 7.0, device="cuda")
    kda.kda_prefill_bf16(qkv, gate, beta, st_c, core_c, ws, scale=D ** -0.5, **kw)
    torch.cuda.synchronize()
    assert torch.equal(core_c.view(torch.int32), core_b.view(torch.int32))
    assert torch.equal(st_c.view(torch.int32), st_b.view(torch.int32))


@pytest.mark.parametrize("T,cap,T_pad,C,D", [(200, 37, 256, 64, 128), (200, 1, 320, 64, 128),
                                             (200, 0, 256, 64, 128), (200, 200, 256, 64, 128),
                                             (57, 20, 80, 16, 16), (4059, 2101, 4160, 64, 128)])
def test_prefill_split_captures_state_at_cap(T, cap, T_pad, C, D):
    """Replay-tail split ("Glm5NextLayer" page): rows from cap get the bits of
    a prefill starting at cap, and the state at cap is captured.  Bitwise
    against two kda_prefill calls; against the oracle's state after cap rows
    and its whole run (the token-serial recurrence does not see the split)."""
    import gated_delta_rule_bounded_amd as kda
    H = 4 if D == 128 else 2
    if T > 1000:
        H = 32
    scale = D ** -0.5
    case = core_case(T, H, D, 7100 + cap, 0.05)
    ins = [cuda(pad_rows(case[n], T_pad, np.nan)) for n in ("q", "k", "v", "gate", "beta")]
    st = cuda(case["S0"]).contiguous()
    cap_st = torch.full_like(st, 3.0)
    core = torch.full((T_pad, H, D), 7.0, device="cuda")
    ws = torch.empty(kda.kda_prefill_workspace_bytes(T_pad, H, D, C), dtype=torch.uint8,
                     device="cuda")
    say("prefill_split", T, cap, T_pad, C, D)
    kda.kda_prefill_split(*ins, st, core, cap_st, ws, T=T, cap=cap, T_pad=T_pad, heads=H,
                          head_dim=D, chunk=C, scale=scale)
    torch.cuda.synchronize()
    got_core, got_S, got_cap = core.cpu().numpy(), st.cpu().numpy(), cap_st.cpu().numpy()
    # two plain calls: [0, cap), then [cap, T) from the carried state
    if cap > 0:
        a_core, a_S = gpu_prefill(case, cap, -(-cap // C) * C, C, scale)
    else:
        a_core, a_S = np.zeros((0, H, D), np.float32), case["S0"]
    np.testing.assert_array_equal(got_cap, a_S)
    np.testing.assert_array_equal(got_core[:cap], a_core[:cap])
    if T > cap:
        tail = {n: case[n][cap:] for n in ("q", "k", "v", "gate", "beta")}
        tail["S0"] = a_S
        Tb = T - cap
        b_core, b_S = gpu_prefill(tail, Tb, -(-Tb // C) * C, C, scale)
        np.testing.assert_array_equal(got_core[cap:T], b_core[:Tb])
        np.testing.assert_array_equal(got_S, b_S)
    assert np.all(got_core[T:] == 7.0)
    ref_core, ref_S = oracle_core(case, scale)
    assert relerr(got_core[:T], ref_core) < TOL
    assert relerr(got_S, ref_S) < TOL
    if cap > 0:
        _, ref_cap = oracle_core(case, scale, T=cap)
        assert relerr(got_cap, ref_cap) < TOL


@pytest.mark.parametrize("T,T_pad,C,D,gate_scale", [(57, 64, 16, 16, 1.0), (100, 128, 64, 16, 1.0),
                                                    (77, 80, 16, 128, 1.0), (200, 256, 64, 128, 1.0),
                                                    (130, 192, 64, 128, 40.0), (70, 80, 16, 128, 40.0),
                                                    (4059, 4096, 64, 128, 1.0)])
def test_prefill_bf16_rows_equal_fp32_widening_bitwise(T, T_pad, C, D, gate_scale):
    """kda_prefill_bf16 reads q | k | v from bf16 rows (the conv output); on
    the exact fp32 widening of the same rows kda_prefill gives the same bits.
    Rows past T hold NaN in both; the row stride has 8 spare columns; a steep
    gate sends chunks down the exact pairwise path, which reads the rows too."""
    import gated_delta_rule_bounded_amd as kda
    H = 32 if T > 1000 else 3
    scale = D ** -0.5
    case = core_case(T, H, D, 7300 + T, 0.05, qkv_bf16=True, gate_scale=gate_scale)
    qw = H * D
    rows = np.full((T_pad, 3 * qw + 8), np.nan, np.float32)
    for i, n in enumerate(("q", "k", "v")):
        rows[:T, i * qw:(i + 1) * qw] = case[n].reshape(T, qw)
    qkv16 = torch.from_numpy(rows).to(torch.bfloat16).cuda()      # exact: values are bf16
    assert torch.equal(qkv16.float().cpu()[:T, :3 * qw], torch.from_numpy(rows[:T, :3 * qw]))
    g = cuda(pad_rows(case["gate"], T_pad, np.nan))
    b = cuda(pad_rows(case["beta"], T_pad, np.nan))
    st = cuda(case["S0"]).contiguous()
    core = torch.full((T_pad, H, D), 7.0, device="cuda")
    ws = torch.empty(kda.kda_prefill_workspace_bytes(T_pad, H, D, C), dtype=torch.uint8,
                     device="cuda")
    say("prefill_bf16", T, T_pad, C, D, gate_scale)
    kda.kda_prefill_bf16(qkv16, g, b, st, core, ws, T=T, T_pad=T_pad, heads=H, head_dim=D,
                         chunk=C, scale=scale)
    torch.cuda.synchronize()
    ref_core, ref_S = gpu_prefill(case, T, T_pad, C, scale, fill=np.nan)
    got = core.cpu().numpy()
    np.testing.assert_array_equal(got[:T], ref_core[:T])
    np.testing.assert_array_equal(st.cpu().numpy(), ref_S)
    assert np.all(got[T:] == 7.0)
