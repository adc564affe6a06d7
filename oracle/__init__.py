"""KDA oracle: plain, slow, token-serial fp64 reference (CPU).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code
with the GPU path (``gated_delta_rule_bounded_amd``) and never imports it.

The arithmetic lives in ``kda_oracle.c`` (one loop per step of the definition);
this module only marshals numpy arrays.  Each function cites the page passage
it follows in the C source.  Pins that tie it to the pages and to mathematics
outside itself are in ``tests/test_oracle_pins.py``.

Readings of what the pages leave open (all exposed as arguments where cheap):
  * recurrence: decay first, then the delta update against the decayed state,
    then read the output from the updated state;
  * state S[h][i][j], i = key channel (the decayed axis), j = value channel;
  * gate = -exp(a_log[h]) * softplus(g_raw + dt_bias[c]), softplus threshold 20;
  * conv: tap kc-1 meets the current row, no bias, window of kc rows newest
    last; L2 = s / sqrt(sum s^2 + eps_l2);
  * o_norm: x / sqrt(mean x^2 + eps) * w * sigmoid(out_gate).
"""
import ctypes
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from . import build as _build

_lib = None

_D = ctypes.POINTER(ctypes.c_double)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_build.LIB):
        _build.build()
    lib = ctypes.CDLL(_build.LIB)
    lib.orc_bf16.restype = ctypes.c_double
    lib.orc_bf16.argtypes = [ctypes.c_double]
    lib.orc_conv_silu_l2.restype = None
    lib.orc_conv_silu_l2.argtypes = [ctypes.c_int] * 4 + [ctypes.c_double] + [_D] * 5
    lib.orc_kda_gate.restype = None
    lib.orc_kda_gate.argtypes = [ctypes.c_int] * 3 + [_D] * 6
    lib.orc_kda_recurrence.restype = None
    lib.orc_kda_recurrence.argtypes = ([ctypes.c_int] * 5 + [_D] * 5
                                       + [ctypes.c_double] + [_D] * 3)
    lib.orc_bf16_array.restype = None
    lib.orc_bf16_array.argtypes = [ctypes.c_int64, _D, _D]
    lib.orc_linear.restype = None
    lib.orc_linear.argtypes = [ctypes.c_int] * 3 + [_D] * 3
    lib.orc_gated_rmsnorm.restype = None
    lib.orc_gated_rmsnorm.argtypes = [ctypes.c_int] * 3 + [ctypes.c_double] + [_D] * 4
    _lib = lib
    return lib


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _p(a):
    if a is None:
        return None
    return a.ctypes.data_as(_D)


def bf16(x):
    """Round every element to the nearest bfloat16 (ties to even), as float64."""
    lib = _load()
    x = _f64(x)
    out = np.empty_like(x)
    lib.orc_bf16_array(x.size, _p(x), _p(out))
    return out


def linear_plain(x, w):
    """One projection written out as loops in C: bf16(x w^T), w in torch
    Linear layout [out, in] (small shapes: the definition the matmul form is
    checked against)."""
    lib = _load()
    x, w = _f64(x), _f64(w)
    T, n_in = x.shape
    n_out = w.shape[0]
    assert w.shape == (n_out, n_in)
    y = np.empty((T, n_out))
    lib.orc_linear(T, n_in, n_out, _p(x), _p(w), _p(y))
    return y


def linear(x, w):
    """The same projection with the product taken by numpy's fp64 matmul."""
    x, w = _f64(x), _f64(w)
    assert x.shape[1] == w.shape[1]
    return bf16(x @ w.T)


def kda_block_prefill(hidden, wts, S0, conv_state, heads, head_dim, scale,
                      eps_l2=1e-6, eps_rms=1e-5, threads=1, snapshots=False):
    """One KDA block over one sequence ("Glm5NextKdaLayer" page, prefill;
    buffers of the "Glm5NextKdaWorkspace" page; weights of the
    "Glm5NextKdaWeights" page):

      qkv_proj  = [x q_proj^T | x k_proj^T | x v_proj^T]        (bf16 each)
      conv_out  = conv_silu_l2(qkv_proj) from conv_state
      g_raw     = f_b(f_a(x)),  b_raw = b_proj(x)                (bf16 each)
      gate, beta = kda_gate(g_raw, b_raw)
      core, S   = token-serial recurrence over conv_out's q|k|v from S0
      out_gate  = g_b(g_a(x))                                    (bf16 each)
      o_norm_out = gated_rmsnorm(core, out_gate, o_norm)
      final_out = o_norm_out o_proj^T                            (bf16)

    Readings: the rank-128 intermediates f_a(x) and g_a(x) are rounded to
    bf16 like every projection output; the recurrence reads the conv output's
    bf16 values (their fp32 widening is exact).  ``wts`` maps the weight
    names of the weights page to arrays in [out, in] layout (conv [conv_dim,
    kc], a_log [H], dt_bias [H*D], o_norm [D]).  Returns a dict of every
    stage buffer plus the final state and conv state; with ``snapshots`` also
    the recurrent and conv states after each row but the last ("state_snaps"
    [T-1, H, D, D], "conv_snaps" [T-1, kc, 3*H*D])."""
    H, D = heads, head_dim
    qkv = H * D
    x = _f64(hidden)
    T = x.shape[0]
    qkv_proj = np.concatenate([linear(x, wts["q_proj"]), linear(x, wts["k_proj"]),
                               linear(x, wts["v_proj"])], axis=1)
    conv_out, conv_st, conv_snaps = conv_silu_l2(qkv_proj, wts["conv"], conv_state, H, D,
                                                 eps_l2, snapshots=snapshots)
    fa = linear(x, wts["f_a"])
    g_raw = linear(fa, wts["f_b"])
    b_raw = linear(x, wts["b_proj"])
    gate, beta = kda_gate(g_raw, wts["a_log"], wts["dt_bias"], H, D, b_raw=b_raw)
    qf = conv_out[:, :qkv].reshape(T, H, D)
    kf = conv_out[:, qkv:2 * qkv].reshape(T, H, D)
    vf = conv_out[:, 2 * qkv:].reshape(T, H, D)
    core, S, state_snaps = kda_recurrence(qf, kf, vf, gate, beta, S0, scale,
                                          snapshots=snapshots, threads=threads)
    ga = linear(x, wts["g_a"])
    out_gate = linear(ga, wts["g_b"])
    o_norm_out = gated_rmsnorm(core, out_gate, wts["o_norm"], eps_rms)
    final_out = linear(o_norm_out, wts["o_proj"])
    return dict(qkv_proj=qkv_proj, conv_out=conv_out, fa=fa, g_raw=g_raw, b_raw=b_raw,
                gate=gate, beta=beta, core=core, ga=ga, out_gate=out_gate,
                o_norm_out=o_norm_out, final_out=final_out, state=S, conv_state=conv_st,
                state_snaps=state_snaps, conv_snaps=conv_snaps)


def kda_block_decode_k(hidden, wts, S0, conv_state, heads, head_dim, scale,
                       eps_l2=1e-6, eps_rms=1e-5):
    """K tokens of each of B sequences through one KDA block ("Glm5NextKdaLayer"
    page, decode_k; decode is K = 1).  The block is causal and token-serial,
    so each sequence's K rows are exactly kda_block_prefill over those rows
    from that sequence's carried states, with the snapshots after rows
    0..K-2.  hidden [B, K, hidden]; S0 [B, H, D, D]; conv_state [B, kc,
    3*H*D].  Returns a list of B result dicts of kda_block_prefill."""
    hidden = _f64(hidden)
    return [kda_block_prefill(hidden[b], wts, S0[b], conv_state[b], heads, head_dim, scale,
                              eps_l2, eps_rms, snapshots=True)
            for b in range(hidden.shape[0])]


def conv_silu_l2(x, w, state, heads, head_dim, eps_l2=1e-6, snapshots=False):
    """One sequence.  x [rows, 3*H*D], w [3*H*D, kc], state [kc, 3*H*D].

    Returns (y [rows, 3*H*D] bf16-valued, new_state, snaps [rows-1, kc, 3*H*D]
    or None)."""
    lib = _load()
    x, w = _f64(x), _f64(w)
    st = _f64(state).copy()
    rows, conv_dim = x.shape
    kc = w.shape[1]
    assert conv_dim == 3 * heads * head_dim and w.shape[0] == conv_dim
    assert st.shape == (kc, conv_dim)
    y = np.empty_like(x)
    snaps = np.zeros((max(rows - 1, 0), kc, conv_dim)) if snapshots else None
    lib.orc_conv_silu_l2(rows, heads, head_dim, kc, float(eps_l2), _p(x), _p(w),
                         _p(st), _p(snaps) if snapshots and rows > 1 else None, _p(y))
    return y, st, snaps


def kda_gate(g_raw, a_log, dt_bias, heads, head_dim, b_raw=None):
    """g_raw [T, H*D], a_log [H], dt_bias [H*D], b_raw [T, H] or None.

    Returns (gate [T, H, D], beta [T, H] or None)."""
    lib = _load()
    g_raw, a_log, dt_bias = _f64(g_raw), _f64(a_log), _f64(dt_bias)
    T = g_raw.shape[0]
    assert g_raw.shape == (T, heads * head_dim)
    assert a_log.shape == (heads,) and dt_bias.shape == (heads * head_dim,)
    gate = np.empty((T, heads, head_dim))
    beta = None
    if b_raw is not None:
        b_raw = _f64(b_raw)
        assert b_raw.shape == (T, heads)
        beta = np.empty((T, heads))
    lib.orc_kda_gate(T, heads, head_dim, _p(g_raw), _p(b_raw), _p(a_log),
                     _p(dt_bias), _p(gate), _p(beta))
    return gate, beta


def kda_recurrence(q, k, v, g, beta, S0, scale, snapshots=False, threads=1):
    """Token-serial KDA over one sequence.

    q, k, v, g [T, H, D]; beta [T, H]; S0 [H, D, D] (S[h][key][value]).
    Returns (core [T, H, D], S_T [H, D, D], snaps [T-1, H, D, D] or None).
    ``threads`` > 1 runs disjoint head ranges on a thread pool (the C call
    releases the GIL); the arithmetic per head is unchanged."""
    lib = _load()
    q, k, v, g, beta = (_f64(a) for a in (q, k, v, g, beta))
    S = _f64(S0).copy()
    T, H, D = q.shape
    for a in (k, v, g):
        assert a.shape == (T, H, D)
    assert beta.shape == (T, H) and S.shape == (H, D, D)
    core = np.zeros((T, H, D))
    snaps = np.zeros((max(T - 1, 0), H, D, D)) if snapshots else None
    sp = _p(snaps) if snapshots and T > 1 else None

    def run(h0, h1):
        lib.orc_kda_recurrence(T, H, D, h0, h1, _p(q), _p(k), _p(v), _p(g),
                               _p(beta), float(scale), _p(S), _p(core), sp)

    threads = max(1, min(int(threads), H))
    if threads == 1:
        run(0, H)
    else:
        bounds = np.linspace(0, H, threads + 1).astype(int)
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(lambda i: run(int(bounds[i]), int(bounds[i + 1])), range(threads)))
    return core, S, snaps


def gated_rmsnorm(core, out_gate, w, eps=1e-5):
    """core [T, H, D]; out_gate [T, H*D]; w [D].  Returns bf16-valued [T, H*D]."""
    lib = _load()
    core, out_gate, w = _f64(core), _f64(out_gate), _f64(w)
    T, H, D = core.shape
    assert out_gate.shape == (T, H * D) and w.shape == (D,)
    out = np.empty((T, H * D))
    lib.orc_gated_rmsnorm(T, H, D, float(eps), _p(core), _p(out_gate), _p(w), _p(out))
    return out
