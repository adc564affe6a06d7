"""kda_block_prefill on the GPU (projections on the vendor GEMM around this
library's stage kernels) against the oracle's block.

Tolerance 2e-2 (max relative error per tensor) on every stage buffer, the
block output and the carried state: every stage after the projections reads
bf16 projection outputs, and a projection's fp32-accumulated sum may round
to the bf16 neighbour of the oracle's fp64 sum, so everything downstream
carries bf16-level differences (the bf16-stage bound).  At the full block
size (T = 8192, hidden 4096, 32 heads) the oracle runs the causal prefix of
the first rows: every stage is row-local or causal, so those rows of the
GPU's full-length run must match it.
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


def run_gpu(x, w, T, T_pad, hidden, H, D, rank, C, S0, conv0, scale, packed=False,
            f32_copies=False, keep=None):
    """One kda_block_prefill call; returns every stage buffer's first T rows,
    the output and the carried states as numpy.  ``keep``, a dict, receives
    the device buffers for further GPU calls."""
    dev = torch.device("cuda")
    wd = {n: t.to(dev).contiguous() for n, t in w.items()}
    if packed:   # weights back to back: the block runs q|k|v and f_a|g_a|b_proj as one GEMM each
        qkv = H * D
        wqkv = torch.cat([wd["q_proj"], wd["k_proj"], wd["v_proj"]]).contiguous()
        wd["q_proj"], wd["k_proj"], wd["v_proj"] = wqkv[:qkv], wqkv[qkv:2 * qkv], wqkv[2 * qkv:]
        wlr = torch.cat([wd["f_a"], wd["g_a"], wd["b_proj"]]).contiguous()
        wd["f_a"], wd["g_a"], wd["b_proj"] = wlr[:rank], wlr[rank:2 * rank], wlr[2 * rank:]
    xg = x[:T].to(dev).contiguous()
    st = torch.from_numpy(np.ascontiguousarray(S0, dtype=np.float32)).to(dev)
    cs = conv0.to(dev).contiguous()
    buf = kda.block_buffers(T_pad, heads=H, head_dim=D, rank=rank, chunk=C, device=dev,
                            f32_copies=f32_copies)
    out = torch.empty(T, hidden, dtype=torch.bfloat16, device=dev)
    say("block", T, T_pad, hidden, H, D, rank, C)
    kda.kda_block_prefill(xg, wd, st, kda.ptr_table([cs]), buf, out, T=T, T_pad=T_pad,
                          hidden_size=hidden, heads=H, head_dim=D, rank=rank, chunk=C,
                          scale=scale)
    torch.cuda.synchronize()
    if keep is not None:
        keep.update(buf)
    res = {n: buf[n][:T].float().cpu().numpy() for n in STAGES}
    res["final_out"] = out.float().cpu().numpy()
    res["state"] = st.cpu().numpy()
    res["conv_state"] = cs.float().cpu().numpy()
    if f32_copies:   # the optional fp32 copies are the exact widening of conv_out
        co = buf["conv_out"][:T].float()
        for i, n in enumerate(("q32", "k32", "v32")):
            assert torch.equal(buf[n][:T].reshape(T, -1), co[:, i * H * D:(i + 1) * H * D]), n
    return res


def run_oracle(orc, x, w, T, H, D, S0, conv0, scale):
    wd = {n: t.double().numpy() for n, t in w.items()}
    return orc.kda_block_prefill(x[:T].double().numpy(), wd, np.asarray(S0, dtype=np.float64),
                                 conv0.double().numpy(), H, D, scale, threads=8)


def compare(got, ref, T, H, D, names):
    for n in names:
        g = got[n][:T].reshape(ref[n].shape)
        e = relerr(g, ref[n])
        assert e < TOL, f"{n}: relerr {e:.3e}"


@pytest.mark.parametrize("T,T_pad,H,D,hidden,rank,C,packed", [
    (50, 64, 2, 16, 64, 16, 16, False),
    (200, 256, 2, 128, 256, 32, 64, False),
    (200, 256, 2, 128, 256, 32, 64, True),
    (200, 256, 8, 16, 128, 32, 64, True),   # 8 heads: f_a | g_a | b_proj as one GEMM
])
def test_block_small_against_oracle(orc, T, T_pad, H, D, hidden, rank, C, packed):
    x, w = workloads.block_raw(T, hidden, H, D, rank, 4, 1004, w_std=0.05)
    S0 = workloads.state(H, D, 0.05, 2004)
    conv0 = workloads.conv_raw(1, H, D, 4, 3004)["state"][0]
    scale = D ** -0.5
    got = run_gpu(x, w, T, T_pad, hidden, H, D, rank, C, S0, conv0, scale, packed=packed,
                  f32_copies=packed)
    ref = run_oracle(orc, x, w, T, H, D, S0, conv0, scale)
    compare(got, ref, T, H, D, STAGES + ("final_out",))
    assert relerr(got["state"], ref["state"]) < TOL
    assert relerr(got["conv_state"], ref["conv_state"]) < TOL


def test_block_full_size_causal_prefix(orc):
    # the full KDA block workload: T = 8192, hidden 4096, 32 heads x 128,
    # rank-128 gates, weights ~ N(0, 0.02), zero initial state and conv state
    T, T_pad, H, D, hidden, rank, C = 8192, 8192, 32, 128, 4096, 128, 64
    Tp = 512
    x, w = workloads.block_raw(T, hidden, H, D, rank, 4, 1004)
    S0 = np.zeros((H, D, D), dtype=np.float32)
    conv0 = torch.zeros(4, 3 * H * D, dtype=torch.bfloat16)
    scale = D ** -0.5
    buf = {}
    got = run_gpu(x, w, T, T_pad, hidden, H, D, rank, C, S0, conv0, scale, packed=True, keep=buf)
    ref = run_oracle(orc, x, w, Tp, H, D, S0, conv0, scale)
    compare(got, ref, Tp, H, D, STAGES + ("final_out",))
    for n in STAGES + ("final_out",):
        assert np.all(np.isfinite(got[n])), n
    assert np.all(np.isfinite(got["state"]))
    # The block runs its core on its own conv_out, gate and beta: a
    # kda_prefill_bf16 call on those buffers from the same (zero) state gives
    # the block's core rows and carried state after all 8192 rows, bit for bit.
    dev = torch.device("cuda")
    st = torch.zeros(H, D, D, device=dev)
    core = torch.empty(T_pad, H, D, device=dev)
    ws = torch.empty(kda.kda_prefill_workspace_bytes(T_pad, H, D, C), dtype=torch.uint8,
                     device=dev)
    say("block core rerun", T)
    kda.kda_prefill_bf16(buf["conv_out"], buf["gate"], buf["beta"], st, core, ws, T=T,
                         T_pad=T_pad, heads=H, head_dim=D, chunk=C, scale=scale)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(st.cpu().numpy(), got["state"])
    np.testing.assert_array_equal(core[:T].cpu().numpy(), got["core"].reshape(T, H, D))


def test_block_split_equals_one_call():
    # the block carries its state and conv state: two calls over [0, a) and
    # [a, T) equal one call over [0, T) (a not a multiple of the chunk).  The
    # stage kernels are row-parallel and the core walks the same rows from
    # the carried state, so only the core's chunk boundaries move.  The
    # vendor GEMM may pick another algorithm for another row count, so the
    # projection outputs are held to the bf16-stage bound, not bit identity.
    T, H, D, hidden, rank, C = 300, 2, 128, 256, 32, 64
    a = 137
    x, w = workloads.block_raw(T, hidden, H, D, rank, 4, 1005, w_std=0.05)
    S0 = workloads.state(H, D, 0.05, 2005)
    conv0 = workloads.conv_raw(1, H, D, 4, 3005)["state"][0]
    scale = D ** -0.5
    one = run_gpu(x, w, T, 320, hidden, H, D, rank, C, S0, conv0, scale)
    first = run_gpu(x, w, a, 192, hidden, H, D, rank, C, S0, conv0, scale)
    conv_mid = torch.from_numpy(first["conv_state"]).to(torch.bfloat16)
    second = run_gpu(x[a:], w, T - a, 192, hidden, H, D, rank, C, first["state"], conv_mid, scale)
    for n in STAGES + ("final_out",):
        both = np.concatenate([first[n], second[n]])
        assert relerr(both, one[n][:T]) < TOL, n
    assert relerr(second["state"], one["state"]) < TOL
    assert relerr(second["conv_state"], one["conv_state"]) < TOL
