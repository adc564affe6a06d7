"""Shared case builders for the GPU parity tests.

Inputs come from ``workloads`` (seeded draws) and, where the method's own
arithmetic produces an input of a later stage (the gate and beta feeding the
recurrence), from the oracle.  Nothing here takes a value from the GPU path
and hands it to the oracle.
"""
import os

import numpy as np
import torch

import oracle
import workloads

THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


def say(*a):
    """Name the case before a GPU step, flushed, so a fault can be placed."""
    print("[case]", *a, flush=True)


def cuda(a, dtype=torch.float32):
    t = a if isinstance(a, torch.Tensor) else torch.from_numpy(np.ascontiguousarray(a))
    return t.to(dtype).cuda()


def core_case(T, H, D, seed, state_std, qkv_bf16=False, gate_scale=1.0, qk_scale=1.0):
    """Recurrence inputs for one sequence: q, k, v [T,H,D] fp32, gate [T,H,D]
    and beta [T,H] from the oracle's gate (rounded to fp32), S0 [H,D,D]."""
    raw = workloads.core_raw(T, H, D, seed, qkv_bf16=qkv_bf16)
    g64, b64 = oracle.kda_gate(raw["g_raw"], raw["a_log"], raw["dt_bias"], H, D, b_raw=raw["b_raw"])
    S0 = (workloads.state(H, D, state_std, seed + 1000) if state_std
          else np.zeros((H, D, D), np.float32))
    return dict(q=raw["q"] * np.float32(qk_scale), k=raw["k"] * np.float32(qk_scale), v=raw["v"],
                gate=(g64 * gate_scale).astype(np.float32), beta=b64.astype(np.float32), S0=S0)


def oracle_core(case, scale, T=None):
    T = case["q"].shape[0] if T is None else T
    core, S, _ = oracle.kda_recurrence(case["q"][:T], case["k"][:T], case["v"][:T],
                                       case["gate"][:T], case["beta"][:T], case["S0"], scale,
                                       threads=THREADS)
    return core, S


def pad_rows(a, T_pad, fill):
    out = np.full((T_pad,) + a.shape[1:], fill, dtype=np.float32)
    out[: a.shape[0]] = a
    return out


def gpu_prefill(case, T, T_pad, C, scale, fill=0.0, state=None, core_sentinel=7.0):
    """Run kda_prefill on rows [0, T) of the case, tails filled with `fill`.
    Returns (core [T_pad,H,D] numpy, state numpy)."""
    import gated_delta_rule_bounded_amd as kda
    H, D = case["q"].shape[1:]
    ins = [cuda(pad_rows(case[n][:T], T_pad, fill)) for n in ("q", "k", "v", "gate", "beta")]
    st = cuda(case["S0"] if state is None else state).contiguous()
    core = torch.full((T_pad, H, D), core_sentinel, dtype=torch.float32, device="cuda")
    ws = torch.empty(max(1, kda.kda_prefill_workspace_bytes(T_pad, H, D, C)), dtype=torch.uint8,
                     device="cuda")
    kda.kda_prefill(*ins, st, core, ws, T=T, T_pad=T_pad, heads=H, head_dim=D, chunk=C,
                    scale=scale)
    torch.cuda.synchronize()
    return core.cpu().numpy(), st.cpu().numpy()
