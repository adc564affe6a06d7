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
    flat_in, flat_out = x.reshape(-1), out.reshape(-1)
    for i in range(flat_in.size):
        flat_out[i] = lib.orc_bf16(float(flat_in[i]))
    return out


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
