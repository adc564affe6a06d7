"""Pins for the oracle: each check ties it to something other than itself.

Kinds of pin used here:
  * hand-derived worked examples (tests/golden/*.json, each with its citation);
  * brute force with an independent formulation (dense transition matrices,
    and the chunked UT/WY algebra written with numpy linear algebra);
  * closed forms and special cases (beta = 0, one-hot overwrite memory,
    identity conv, softplus/sigmoid points);
  * library routines (torch's bf16 cast, numpy convolve / logaddexp, scipy
    expit);
  * invariants (delta-rule identity per step, linearity, split invariance,
    snapshot consistency, unit L2 norm, unit RMS).
A plausible slip anywhere in the oracle (decay on the wrong axis, output read
before the write, a sign, a transposed state, a tap order, a per-head /
per-channel broadcast swap) fails at least one of them.
"""
import json
import os

import numpy as np
import pytest
import torch
from scipy.special import expit

import workloads
from conftest import relerr

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------
# bf16 rounding vs torch's cast (a library routine) on fp32-representable input
# --------------------------------------------------------------------------
def test_bf16_matches_torch_cast(orc):
    r = np.random.default_rng(7)
    vals = [r.standard_normal(2000) * s for s in (1e-3, 1.0, 1e3, 1e30)]
    # exact ties: a bf16 value plus half a bf16 ulp, both parities
    base = torch.tensor(r.standard_normal(500), dtype=torch.float32).to(torch.bfloat16).float().numpy()
    ulp = np.abs(base) * 2.0 ** -7
    ulp = 2.0 ** np.floor(np.log2(np.abs(base))) * 2.0 ** -7
    vals.append((base + ulp / 2).astype(np.float32))
    vals.append((base - ulp / 2).astype(np.float32))
    # subnormals, near-overflow, signed zero
    vals.append(np.array([1e-40, -3e-39, 1.1754942e-38, 2.0 ** -133, 2.0 ** -134 * 3,
                          3.3895e38, 3.39e38, -3.4e38, 0.0, -0.0], dtype=np.float32))
    x = np.concatenate([np.asarray(v, dtype=np.float32) for v in vals])
    want = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    got = orc.bf16(x.astype(np.float64))
    np.testing.assert_array_equal(got, want)


# --------------------------------------------------------------------------
# Recurrence
# --------------------------------------------------------------------------
def test_recurrence_hand_example(orc):
    g = _golden("recurrence_hand_d2.json")
    T, D = 2, 2
    q = np.array(g["q"]).reshape(T, 1, D)
    k = np.array(g["k"]).reshape(T, 1, D)
    v = np.array(g["v"]).reshape(T, 1, D)
    gate = np.log(np.array(g["exp_g"])).reshape(T, 1, D)
    beta = np.array(g["beta"]).reshape(T, 1)
    S0 = np.array(g["S0"]).reshape(1, D, D)
    core, S, snaps = orc.kda_recurrence(q, k, v, gate, beta, S0, g["scale"], snapshots=True)
    np.testing.assert_allclose(core[:, 0], np.array(g["core"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(S[0], np.array(g["S_T"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(snaps[0, 0], np.array(g["S_after_t0"]), rtol=0, atol=1e-12)


def _cfg0(seed, T=64, H=2, D=16, state_std=None):
    raw = workloads.core_raw(T, H, D, seed)
    return raw


def _gate_beta(orc, raw, H, D):
    gate, beta = orc.kda_gate(raw["g_raw"], raw["a_log"], raw["dt_bias"], H, D, b_raw=raw["b_raw"])
    return gate, beta


def _brute_force(q, k, v, g, beta, S0, scale):
    """S_t = (I - b k k^T) diag(e^g) S_{t-1} + b k v^T ;  o_t = scale S_t^T q."""
    T, H, D = q.shape
    S = S0.astype(np.float64).copy()
    core = np.zeros((T, H, D))
    I = np.eye(D)
    for t in range(T):
        for h in range(H):
            kk = k[t, h][:, None]
            M = (I - beta[t, h] * kk @ kk.T) @ np.diag(np.exp(g[t, h]))
            S[h] = M @ S[h] + beta[t, h] * kk @ v[t, h][None, :]
            core[t, h] = scale * S[h].T @ q[t, h]
    return core, S


@pytest.mark.parametrize("state_std", [0.0, 0.1])
def test_recurrence_brute_force_dense(orc, state_std):
    T, H, D = 64, 2, 16
    raw = _cfg0(workloads.SEED_INPUT + 0, T, H, D)
    g, beta = _gate_beta(orc, raw, H, D)
    S0 = workloads.state(H, D, state_std, workloads.SEED_STATE + 0) if state_std else np.zeros((H, D, D))
    scale = D ** -0.5
    core, S, _ = orc.kda_recurrence(raw["q"], raw["k"], raw["v"], g, beta, S0, scale)
    core_bf, S_bf = _brute_force(raw["q"].astype(np.float64), raw["k"].astype(np.float64),
                                 raw["v"].astype(np.float64), g, beta, S0, scale)
    assert relerr(core, core_bf) < 1e-12
    assert relerr(S, S_bf) < 1e-12


def _chunked_reference(q, k, v, g, beta, S0, scale, C):
    """Chunked (UT/WY) form written with numpy linear algebra, fp64, pairwise
    decay factors.  An independent formulation of the same recurrence."""
    T, H, D = q.shape
    S = S0.astype(np.float64).copy()
    core = np.zeros((T, H, D))
    for h in range(H):
        for c0 in range(0, T, C):
            sl = slice(c0, min(c0 + C, T))
            Q, K, V, Gc = q[sl, h], k[sl, h], v[sl, h], np.cumsum(g[sl, h], axis=0)
            b = beta[sl, h]
            n = Q.shape[0]
            dec = np.exp(Gc[:, None, :] - Gc[None, :, :])            # [r, s, d]
            A = np.einsum("rd,sd,rsd->rs", K, K, dec) * np.tril(np.ones((n, n)), -1)
            P = np.einsum("rd,sd,rsd->rs", Q, K, dec) * np.tril(np.ones((n, n)), 0)
            Tm = np.linalg.inv(np.eye(n) + np.diag(b) @ A)
            W = Tm @ np.diag(b) @ (K * np.exp(Gc))
            U = Tm @ np.diag(b) @ V - W @ S[h]
            core[sl, h] = scale * ((Q * np.exp(Gc)) @ S[h] + P @ U)
            S[h] = np.diag(np.exp(Gc[-1])) @ S[h] + (K * np.exp(Gc[-1] - Gc)).T @ U
    return core, S


@pytest.mark.parametrize("C,T", [(16, 64), (16, 57), (64, 130)])
def test_recurrence_matches_chunked_algebra(orc, C, T):
    H, D = 2, 16
    raw = _cfg0(workloads.SEED_INPUT + 0, T, H, D)
    g, beta = _gate_beta(orc, raw, H, D)
    S0 = workloads.state(H, D, 0.1, workloads.SEED_STATE + 0)
    scale = D ** -0.5
    args = [raw["q"].astype(np.float64), raw["k"].astype(np.float64), raw["v"].astype(np.float64), g, beta]
    core, S, _ = orc.kda_recurrence(*args, S0, scale)
    core_c, S_c = _chunked_reference(*args, S0, scale, C)
    assert relerr(core, core_c) < 1e-10
    assert relerr(S, S_c) < 1e-10


def test_recurrence_delta_identity_each_step(orc):
    """k_t^T S_t = (1 - b|k|^2) k_t^T diag(e^g) S_{t-1} + b |k|^2 v_t^T."""
    T, H, D = 32, 2, 16
    raw = _cfg0(11, T, H, D)
    g, beta = _gate_beta(orc, raw, H, D)
    k = raw["k"].astype(np.float64) * 1.3            # not unit: the identity holds for any k
    S0 = workloads.state(H, D, 0.1, 12)
    _, S_T, snaps = orc.kda_recurrence(raw["q"], k, raw["v"], g, beta, S0, 1.0, snapshots=True)
    states = np.concatenate([S0[None].astype(np.float64), snaps, S_T[None]], axis=0)  # S_0..S_T
    for t in range(T):
        for h in range(H):
            kt, n2, b = k[t, h], float(k[t, h] @ k[t, h]), beta[t, h]
            lhs = kt @ states[t + 1, h]
            rhs = (1 - b * n2) * (kt @ (np.exp(g[t, h])[:, None] * states[t, h])) + b * n2 * raw["v"][t, h]
            np.testing.assert_allclose(lhs, rhs, rtol=1e-11, atol=1e-11)


def test_recurrence_beta_zero_closed_form(orc):
    """beta = 0: no writes, the state only decays along the key axis."""
    T, H, D = 40, 2, 16
    raw = _cfg0(21, T, H, D)
    g, _ = _gate_beta(orc, raw, H, D)
    S0 = workloads.state(H, D, 0.3, 22).astype(np.float64)
    scale = 0.7
    core, S_T, _ = orc.kda_recurrence(raw["q"], raw["k"], raw["v"], g, np.zeros((T, H)), S0, scale)
    G = np.cumsum(g, axis=0)                          # [T, H, D]
    for h in range(H):
        np.testing.assert_allclose(S_T[h], np.exp(G[-1, h])[:, None] * S0[h], rtol=1e-13, atol=0)
        for t in range(T):
            want = scale * (np.exp(G[t, h])[:, None] * S0[h]).T @ raw["q"][t, h]
            np.testing.assert_allclose(core[t, h], want, rtol=1e-12, atol=1e-15)


def test_recurrence_one_hot_overwrite_memory(orc):
    """g = 0, beta = 1, k_t = e_t, S_0 = 0: row t of the state becomes v_t
    exactly, and reading with q = e_t returns v_t (textbook delta rule)."""
    H, D = 2, 16
    T = D
    r = np.random.default_rng(31)
    v = r.standard_normal((T, H, D))
    k = np.zeros((T, H, D))
    q = np.zeros((T, H, D))
    for t in range(T):
        k[t, :, t] = 1.0
        q[t, :, t] = 1.0
    core, S_T, _ = orc.kda_recurrence(q, k, v, np.zeros((T, H, D)), np.ones((T, H)),
                                      np.zeros((H, D, D)), 1.0)
    for h in range(H):
        np.testing.assert_array_equal(S_T[h], v[:, h, :])
        np.testing.assert_array_equal(core[:, h], v[:, h])


def test_recurrence_overwrite_replaces_old_value(orc):
    """Writing key e_0 twice with beta = 1: the second value replaces the first
    (the delta rule subtracts the old association; a plain additive memory
    would hold their sum)."""
    D = 4
    k = np.zeros((2, 1, D)); k[:, 0, 0] = 1.0
    v = np.array([[[1.0, 2.0, 3.0, 4.0]], [[-5.0, 6.0, 0.5, 0.0]]])
    _, S_T, _ = orc.kda_recurrence(k, k, v, np.zeros((2, 1, D)), np.ones((2, 1)),
                                   np.zeros((1, D, D)), 1.0)
    np.testing.assert_array_equal(S_T[0, 0], v[1, 0])


def test_recurrence_linear_in_state_and_values(orc):
    T, H, D = 48, 2, 16
    raw = _cfg0(41, T, H, D)
    g, beta = _gate_beta(orc, raw, H, D)
    S0 = workloads.state(H, D, 0.5, 42)
    zS = np.zeros_like(S0)
    zV = np.zeros_like(raw["v"])
    c1, s1, _ = orc.kda_recurrence(raw["q"], raw["k"], raw["v"], g, beta, S0, 0.5)
    c2, s2, _ = orc.kda_recurrence(raw["q"], raw["k"], zV, g, beta, S0, 0.5)
    c3, s3, _ = orc.kda_recurrence(raw["q"], raw["k"], raw["v"], g, beta, zS, 0.5)
    assert relerr(c1, c2 + c3) < 1e-13
    assert relerr(s1, s2 + s3) < 1e-13


@pytest.mark.parametrize("a", [1, 17, 32, 63])
def test_recurrence_split_invariance_and_snapshots(orc, a):
    T, H, D = 64, 2, 16
    raw = _cfg0(51, T, H, D)
    g, beta = _gate_beta(orc, raw, H, D)
    S0 = workloads.state(H, D, 0.1, 52)
    args = (raw["q"], raw["k"], raw["v"], g, beta)
    c_all, s_all, snaps = orc.kda_recurrence(*args, S0, 0.25, snapshots=True)
    c1, s1, _ = orc.kda_recurrence(*(x[:a] for x in args), S0, 0.25)
    c2, s2, _ = orc.kda_recurrence(*(x[a:] for x in args), s1, 0.25)
    np.testing.assert_array_equal(np.concatenate([c1, c2]), c_all)
    np.testing.assert_array_equal(s2, s_all)
    np.testing.assert_array_equal(snaps[a - 1], s1)       # state after row a-1


def test_recurrence_empty_is_noop(orc):
    H, D = 2, 16
    S0 = workloads.state(H, D, 0.1, 61)
    e = np.zeros((0, H, D))
    core, S, _ = orc.kda_recurrence(e, e, e, e, np.zeros((0, H)), S0, 1.0)
    assert core.shape == (0, H, D)
    np.testing.assert_array_equal(S, S0)


def test_recurrence_does_not_renormalise_qk(orc):
    """Scaling q by c scales the output by c; scaling k changes the write
    (no hidden normalisation of either)."""
    T, H, D = 16, 1, 16
    raw = _cfg0(71, T, H, D)
    g, beta = _gate_beta(orc, raw, H, D)
    S0 = workloads.state(H, D, 0.1, 72)
    c1, s1, _ = orc.kda_recurrence(raw["q"], raw["k"], raw["v"], g, beta, S0, 1.0)
    q64, k64 = raw["q"].astype(np.float64), raw["k"].astype(np.float64)
    c2, s2, _ = orc.kda_recurrence(q64 * 1.01, raw["k"], raw["v"], g, beta, S0, 1.0)
    np.testing.assert_allclose(c2, 1.01 * c1, rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(s1, s2)
    _, s3, _ = orc.kda_recurrence(raw["q"], k64 * 1.01, raw["v"], g, beta, S0, 1.0)
    assert relerr(s3, s1) > 1e-4


# --------------------------------------------------------------------------
# Gate and beta
# --------------------------------------------------------------------------
def test_gate_hand_values(orc):
    gd = _golden("gate_norm_hand.json")
    for c in gd["gate_cases"]:
        gate, _ = orc.kda_gate(np.array([[c["z"]]]), np.array([c["a_log"]]), np.array([0.0]), 1, 1)
        assert abs(gate[0, 0, 0] - c["gate"]) < 1e-14
    for c in gd["beta_cases"]:
        _, beta = orc.kda_gate(np.zeros((1, 1)), np.zeros(1), np.zeros(1), 1, 1,
                               b_raw=np.array([[c["b"]]]))
        assert abs(beta[0, 0] - c["beta"]) < 1e-15


def test_gate_per_head_and_per_channel_broadcast(orc):
    """a_log indexes the head, dt_bias the channel (the highest-risk line):
    with a_log[h] = ln(h+1) and g_raw = 0, gate[t,h,d] / (h+1) must equal
    softplus(dt_bias[h*D+d]) for every head (numpy logaddexp as softplus)."""
    T, H, D = 3, 4, 8
    a_log = np.log(np.arange(1, H + 1, dtype=np.float64))
    dt = np.linspace(-3.0, 3.0, H * D)
    gate, _ = orc.kda_gate(np.zeros((T, H * D)), a_log, dt, H, D)
    sp = np.logaddexp(0.0, dt).reshape(H, D)
    for h in range(H):
        np.testing.assert_allclose(-gate[:, h, :] / (h + 1), np.broadcast_to(sp[h], (T, D)), rtol=1e-14)


def test_gate_against_library_softplus_sigmoid(orc):
    T, H, D = 50, 3, 8
    r = np.random.default_rng(81)
    z = r.normal(0, 6, size=(T, H * D))
    z[0, :4] = [19.99, 20.0, 20.01, 40.0]           # around the softplus threshold
    a_log = r.uniform(-1, 0.5, size=H)
    dt = r.normal(0, 0.5, size=H * D)
    b = r.normal(0, 4, size=(T, H))
    gate, beta = orc.kda_gate(z, a_log, dt, H, D, b_raw=b)
    want = -np.exp(a_log)[None, :, None] * np.logaddexp(0.0, (z + dt).reshape(T, H, D) * 1.0)
    # logaddexp has no threshold: the dropped term is below 2.1e-9 relative
    np.testing.assert_allclose(gate, want, rtol=3e-9)
    np.testing.assert_allclose(beta, expit(b), rtol=1e-15)
    assert np.all(gate <= 0.0)                      # bounded: decay factor in (0, 1]


# --------------------------------------------------------------------------
# Conv + SiLU + L2
# --------------------------------------------------------------------------
def _conv_inputs(seed, rows, H, D, kc=4):
    raw = workloads.conv_raw(rows, H, D, kc, seed, n_seq=1, w_std=0.5)
    return raw["x"].double().numpy(), raw["w"].double().numpy(), raw["state"][0].double().numpy()


def test_conv_taps_match_numpy_convolve(orc):
    """Pre-activation = causal depthwise convolution with the window history.
    Checked on the v section (no L2) through SiLU via scipy's expit, against
    numpy.convolve per channel with the flipped kernel."""
    H, D, kc, rows = 2, 8, 4, 9
    x, w, st = _conv_inputs(91, rows, H, D, kc)
    y, new_state, _ = orc.conv_silu_l2(x, w, st, H, D)
    cd = 3 * H * D
    xfull = np.concatenate([st[1:], x], axis=0)          # the kc-1 most recent history rows
    for c in range(2 * H * D, cd):
        pre = np.convolve(xfull[:, c], w[c, ::-1], mode="full")[kc - 1:kc - 1 + rows]
        np.testing.assert_allclose(y[:, c], orc.bf16(pre * expit(pre)), rtol=0, atol=0)
    np.testing.assert_array_equal(new_state, x[-kc:])


def test_conv_identity_kernel_and_unit_norm(orc):
    """w = e_{kc-1} (identity conv): v section = bf16(silu(x)); every q/k head
    has unit L2 norm up to bf16 rounding and points along silu(x)."""
    H, D, kc, rows = 2, 16, 4, 5
    x, _, st = _conv_inputs(101, rows, H, D, kc)
    w = np.zeros((3 * H * D, kc)); w[:, kc - 1] = 1.0
    y, _, _ = orc.conv_silu_l2(x, w, st, H, D, eps_l2=0.0)
    s = x * expit(x)
    np.testing.assert_array_equal(y[:, 2 * H * D:], orc.bf16(s[:, 2 * H * D:]))
    for blk in range(2 * H):
        sl = slice(blk * D, (blk + 1) * D)
        n = np.linalg.norm(y[:, sl], axis=1)
        np.testing.assert_allclose(n, 1.0, atol=2 * 2.0 ** -8)
        cos = np.sum(y[:, sl] * s[:, sl], axis=1) / (n * np.linalg.norm(s[:, sl], axis=1))
        np.testing.assert_allclose(cos, 1.0, atol=1e-4)


def test_conv_state_window_and_snapshots(orc):
    """Rows processed one call at a time equal one multi-row call, and the
    snapshot after row t is the window state after t+1 single-row calls.
    The oldest window row never reaches an output (it is dropped first)."""
    H, D, kc, rows = 2, 8, 4, 6
    x, w, st = _conv_inputs(111, rows, H, D, kc)
    y, fin, snaps = orc.conv_silu_l2(x, w, st, H, D, snapshots=True)
    cur = st.copy()
    for t in range(rows):
        yt, cur, _ = orc.conv_silu_l2(x[t:t + 1], w, cur, H, D)
        np.testing.assert_array_equal(yt[0], y[t])
        if t < rows - 1:
            np.testing.assert_array_equal(snaps[t], cur)
    np.testing.assert_array_equal(cur, fin)
    st2 = st.copy(); st2[0] += 100.0
    y2, _, _ = orc.conv_silu_l2(x, w, st2, H, D)
    np.testing.assert_array_equal(y2, y)


# --------------------------------------------------------------------------
# Gated RMSNorm
# --------------------------------------------------------------------------
def test_rmsnorm_hand_case(orc):
    c = _golden("gate_norm_hand.json")["norm_case"]
    out = orc.gated_rmsnorm(np.array(c["x"]).reshape(1, 1, 4), np.array([c["gate"]]),
                            np.array(c["w"]), eps=c["eps"])
    np.testing.assert_array_equal(out[0], np.array(c["out"]))


def test_rmsnorm_unit_rms_and_scale_free(orc):
    T, H, D = 20, 3, 16
    raw = workloads.norm_raw(T, H, D, 121)
    x = raw["core"].astype(np.float64)
    out = orc.gated_rmsnorm(x, np.full((T, H * D), 30.0), np.ones(D), eps=1e-5)
    rms = np.sqrt(np.mean(out.reshape(T, H, D) ** 2, axis=2))
    np.testing.assert_allclose(rms, 1.0, atol=2 * 2.0 ** -8)
    gate = raw["out_gate"].double().numpy()
    w = raw["w"].double().numpy()
    o1 = orc.gated_rmsnorm(x, gate, w, eps=0.0)
    o2 = orc.gated_rmsnorm(x * 3.7, gate, w, eps=0.0)
    assert relerr(o2, o1) < 2.0 ** -7


# --------------------------------------------------------------------------
# Block: projections around the stages
# --------------------------------------------------------------------------
def test_linear_layout_hand_example_and_plain_loops(orc):
    # torch Linear layout [out, in]: y = x W^T.  A transposed weight would not
    # even have the right shape here, and a swapped operand order gives 3 rows.
    y = orc.linear(np.array([[1.0, 2.0]]), np.array([[1.0, 0.0], [0.0, 2.0], [1.0, 1.0]]))
    np.testing.assert_array_equal(y, [[1.0, 4.0, 3.0]])
    # the output is a bf16 buffer: 1 + 2^-8 is a tie and rounds to even (1.0)
    y = orc.linear(np.array([[1.0, 2.0 ** -8]]), np.array([[1.0, 1.0]]))
    np.testing.assert_array_equal(y, [[1.0]])
    # the matmul form equals the definition written as loops
    r = np.random.default_rng(5)
    x, w = r.standard_normal((6, 37)), r.standard_normal((11, 37))
    np.testing.assert_array_equal(orc.linear(x, w), orc.linear_plain(x, w))


def _tiny_block(T=24, H=2, D=16, rank=8, seed=131):
    hidden = H * D
    x, w = workloads.block_raw(T, hidden, H, D, rank, 4, seed, w_std=0.1)
    wd = {n: t.double().numpy() for n, t in w.items()}
    return x.double().numpy(), wd, H, D


def _run_block(orc, x, wd, H, D, S0=None, conv_state=None):
    qkv = H * D
    S0 = np.zeros((H, D, D)) if S0 is None else S0
    cs = np.zeros((4, 3 * qkv)) if conv_state is None else conv_state
    return orc.kda_block_prefill(x, wd, S0, cs, H, D, D ** -0.5)


def test_block_is_causal_prefix(orc):
    # every stage is row-local or causal, so the block over the first T'
    # rows equals the first T' rows of the block over T rows
    x, wd, H, D = _tiny_block()
    full = _run_block(orc, x, wd, H, D)
    part = _run_block(orc, x[:10], wd, H, D)
    for name in ("qkv_proj", "conv_out", "g_raw", "gate", "beta", "core", "out_gate",
                 "o_norm_out", "final_out"):
        np.testing.assert_array_equal(part[name], full[name][:10], err_msg=name)


def test_block_zero_gate_projections_give_closed_forms(orc):
    # f_b = 0: g_raw = 0, so the decay is -exp(a_log[h]) softplus(dt_bias[c]);
    # b_proj = 0: beta = sigmoid(0) = 1/2 exactly
    x, wd, H, D = _tiny_block()
    wd = dict(wd, f_b=np.zeros_like(wd["f_b"]), b_proj=np.zeros_like(wd["b_proj"]))
    out = _run_block(orc, x, wd, H, D)
    T = x.shape[0]
    sp = np.logaddexp(0.0, wd["dt_bias"]).reshape(H, D)
    want = -np.exp(wd["a_log"])[:, None] * sp
    assert relerr(out["gate"], np.broadcast_to(want, (T, H, D))) < 1e-14
    np.testing.assert_array_equal(out["beta"], np.full((T, H), 0.5))


def test_block_wires_sections_norm_and_output(orc):
    # hidden = H*D.  q/k/v projections 1, 2, 3 times the identity make the
    # pre-conv rows [x, 2x, 3x] (bf16); an identity conv tap; g_b = 0 makes
    # the output gate sigmoid(0) = 1/2; o_proj = I passes o_norm_out through.
    # Each stage then has an independently pinned reference, so a swapped
    # q/k/v section, a wrong gate input or a skipped norm fails here.
    x, wd, H, D = _tiny_block()
    qkv = H * D
    eye = np.eye(qkv)
    conv = np.zeros((3 * qkv, 4))
    conv[:, 3] = 1.0
    wd = dict(wd, q_proj=eye, k_proj=2 * eye, v_proj=3 * eye, conv=conv,
              g_b=np.zeros_like(wd["g_b"]), o_proj=eye)
    r = np.random.default_rng(17)
    S0 = r.normal(0.0, 0.1, size=(H, D, D))
    out = _run_block(orc, x, wd, H, D, S0=S0)
    T = x.shape[0]
    pre = np.concatenate([orc.bf16(x), orc.bf16(2 * x), orc.bf16(3 * x)], axis=1)
    np.testing.assert_array_equal(out["qkv_proj"], pre)
    y, _, _ = orc.conv_silu_l2(pre, conv, np.zeros((4, 3 * qkv)), H, D)
    np.testing.assert_array_equal(out["conv_out"], y)
    gate, beta = orc.kda_gate(out["g_raw"], wd["a_log"], wd["dt_bias"], H, D,
                              b_raw=out["b_raw"])
    core, S, _ = orc.kda_recurrence(y[:, :qkv].reshape(T, H, D),
                                    y[:, qkv:2 * qkv].reshape(T, H, D),
                                    y[:, 2 * qkv:].reshape(T, H, D), gate, beta, S0, D ** -0.5)
    np.testing.assert_array_equal(out["core"], core)
    np.testing.assert_array_equal(out["state"], S)
    np.testing.assert_array_equal(out["out_gate"], np.zeros((T, qkv)))
    norm = orc.gated_rmsnorm(core, np.zeros((T, qkv)), wd["o_norm"])
    np.testing.assert_array_equal(out["o_norm_out"], norm)
    np.testing.assert_array_equal(out["final_out"], norm)


def test_block_decode_k_snapshots_are_prefix_states(orc):
    # decode_k over K rows from carried states: the recurrent snapshot after
    # row t is the final state of the block over rows 0..t alone, and the conv
    # snapshot after row t is the window of the last 4 pre-conv rows (a copy
    # of the carried window followed by the projected rows); K single-row
    # decodes chained through their states give the same rows and states
    x, wd, H, D = _tiny_block(T=5)
    qkv = H * D
    r = np.random.default_rng(23)
    S0 = r.normal(0.0, 0.1, size=(2, H, D, D))
    cs = orc.bf16(r.standard_normal((2, 4, 3 * qkv)))
    xb = np.stack([x, x[::-1]])                        # two sequences, K = 5
    res = orc.kda_block_decode_k(xb, wd, S0, cs, H, D, D ** -0.5)
    for b in range(2):
        out = res[b]
        assert out["state_snaps"].shape == (4, H, D, D)
        for t in range(4):
            pre = orc.kda_block_prefill(xb[b, :t + 1], wd, S0[b], cs[b], H, D, D ** -0.5)
            np.testing.assert_array_equal(out["state_snaps"][t], pre["state"])
            window = np.concatenate([cs[b], out["qkv_proj"][:t + 1]])[-4:]
            np.testing.assert_array_equal(out["conv_snaps"][t], window)
        np.testing.assert_array_equal(out["conv_state"],
                                      np.concatenate([cs[b], out["qkv_proj"]])[-4:])
        S, c = S0[b], cs[b]
        for t in range(5):
            one = orc.kda_block_decode_k(xb[b, t][None, None], wd, S[None], c[None], H, D,
                                         D ** -0.5)[0]
            np.testing.assert_array_equal(one["final_out"][0], out["final_out"][t])
            S, c = one["state"], one["conv_state"]
        np.testing.assert_array_equal(S, out["state"])
        np.testing.assert_array_equal(c, out["conv_state"])
