"""Seeded synthetic inputs for the KDA core, shared by tests, smoke and bench.

This module draws random numbers and rounds them to the storage types of the
buffer contract; it holds none of the method's arithmetic (no gate, no conv,
no recurrence, no norm).  Both the GPU path and the oracle receive exactly the
arrays made here.

Distributions follow the documented workload recipe: normal draws are written
N(mean, std); bf16 values are round-to-nearest-even from fp32 (torch's cast).
"""
import numpy as np
import torch

# Seeds: inputs 1000 + workload index, initial states 2000 + workload index.
SEED_INPUT = 1000
SEED_STATE = 2000


def to_bf16(a) -> torch.Tensor:
    """fp32 numpy/torch -> torch.bfloat16 (CPU), round to nearest even."""
    t = torch.as_tensor(np.asarray(a, dtype=np.float32))
    return t.to(torch.bfloat16)


def _unit_rows(x):
    """Scale each trailing-axis vector to unit Euclidean length (the recipe
    draws q, k from N(0,1) 'then L2-normalised per head')."""
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True))


def core_raw(T, H, D, seed, qkv_bf16=False):
    """Raw draws for the recurrence core over one sequence.

    q, k ~ N(0,1) unit-normalised per head, v ~ N(0,1)           [T, H, D]
    x ~ N(0,1) per channel (the gate's input g_raw)              [T, H*D]
    a_log ~ U(-1, 0.5) per head, dt_bias ~ N(0, 0.5) per channel
    b ~ N(0,1) per token-head (beta's pre-activation)            [T, H]
    With qkv_bf16, q/k/v are rounded to bf16 and widened back to fp32.
    Everything is returned as float32 numpy arrays."""
    r = np.random.default_rng(seed)
    q = _unit_rows(r.standard_normal((T, H, D)))
    k = _unit_rows(r.standard_normal((T, H, D)))
    v = r.standard_normal((T, H, D))
    x = r.standard_normal((T, H * D))
    a_log = r.uniform(-1.0, 0.5, size=H)
    dt_bias = r.normal(0.0, 0.5, size=H * D)
    b = r.standard_normal((T, H))
    out = dict(q=q, k=k, v=v, g_raw=x, a_log=a_log, dt_bias=dt_bias, b_raw=b)
    out = {n: a.astype(np.float32) for n, a in out.items()}
    if qkv_bf16:
        for n in ("q", "k", "v"):
            out[n] = to_bf16(out[n]).float().numpy()
    return out


def state(H, D, std, seed, B=None):
    """Initial recurrent state ~ N(0, std), [H, D, D] or [B, H, D, D], fp32."""
    r = np.random.default_rng(seed)
    shape = (H, D, D) if B is None else (B, H, D, D)
    return r.normal(0.0, std, size=shape).astype(np.float32)


def decode_step_raw(B, H, D, seed):
    """One decode step for B sequences: q|k|v rows as the conv writes them
    (bf16, q/k unit-normalised per head before rounding), plus the gate and
    beta draws as in core_raw.  Returns qkv as torch.bfloat16 [B, 3*H*D]."""
    r = np.random.default_rng(seed)
    q = _unit_rows(r.standard_normal((B, H, D)))
    k = _unit_rows(r.standard_normal((B, H, D)))
    v = r.standard_normal((B, H, D))
    qkv = np.concatenate([q.reshape(B, -1), k.reshape(B, -1), v.reshape(B, -1)], axis=1)
    return dict(
        qkv=to_bf16(qkv),
        g_raw=r.standard_normal((B, H * D)).astype(np.float32),
        b_raw=r.standard_normal((B, H)).astype(np.float32),
    )


def gate_params(H, D, seed):
    r = np.random.default_rng(seed)
    return (r.uniform(-1.0, 0.5, size=H).astype(np.float32),
            r.normal(0.0, 0.5, size=H * D).astype(np.float32))


def conv_raw(n_rows, H, D, kc, seed, n_seq=1, w_std=0.02):
    """Pre-conv q|k|v rows x ~ N(0,1) bf16 [n_rows, 3*H*D], depthwise conv
    weight ~ N(0, w_std) bf16 [3*H*D, kc], conv states ~ N(0,1) bf16
    [n_seq, kc, 3*H*D]."""
    r = np.random.default_rng(seed)
    cd = 3 * H * D
    return dict(
        x=to_bf16(r.standard_normal((n_rows, cd))),
        w=to_bf16(r.normal(0.0, w_std, size=(cd, kc))),
        state=to_bf16(r.standard_normal((n_seq, kc, cd))),
    )


def norm_raw(T, H, D, seed):
    """Inputs of the gated RMSNorm: core ~ N(0,1) fp32 [T, H, D], out_gate
    ~ N(0,1) bf16 [T, H*D], o_norm weight ~ N(1, 0.1) bf16 [D]."""
    r = np.random.default_rng(seed)
    return dict(
        core=r.standard_normal((T, H, D)).astype(np.float32),
        out_gate=to_bf16(r.standard_normal((T, H * D))),
        w=to_bf16(r.normal(1.0, 0.1, size=D)),
    )


def block_raw(T, hidden, H, D, rank, kc, seed, w_std=0.02):
    """Inputs of one KDA block: hidden ~ N(0,1) bf16 [T, hidden]; every bf16
    weight ~ N(0, w_std) in torch Linear layout [out, in]: q/k/v_proj
    [H*D, hidden], conv [3*H*D, kc], f_a/g_a [rank, hidden], f_b/g_b
    [H*D, rank], b_proj [H, hidden], o_norm [D], o_proj [hidden, H*D]; the
    two fp32 gate parameters a_log ~ U(-1, 0.5) [H], dt_bias ~ N(0, 0.5)
    [H*D].  Returns (hidden, weights) as torch CPU tensors (bf16 / fp32)."""
    r = np.random.default_rng(seed)
    qkv = H * D
    x = to_bf16(r.standard_normal((T, hidden)))
    shapes = dict(q_proj=(qkv, hidden), k_proj=(qkv, hidden), v_proj=(qkv, hidden),
                  conv=(3 * qkv, kc), f_a=(rank, hidden), f_b=(qkv, rank),
                  b_proj=(H, hidden), g_a=(rank, hidden), g_b=(qkv, rank), o_norm=(D,),
                  o_proj=(hidden, qkv))
    w = {n: to_bf16(r.normal(0.0, w_std, size=s)) for n, s in shapes.items()}
    w["a_log"] = torch.from_numpy(r.uniform(-1.0, 0.5, size=H).astype(np.float32))
    w["dt_bias"] = torch.from_numpy(r.normal(0.0, 0.5, size=qkv).astype(np.float32))
    return x, w
