"""The Python binding checks every tensor against the sizes its call implies
before anything reaches the library: an undersized tensor, a short pointer
table or a wrong dtype raises here (ValueError / TypeError) instead of
becoming an out-of-bounds device access.  The tensors are CPU tensors, so a
call whose sizes are all right stops at the next check (the binding wants
device tensors) with a TypeError; no call reaches a kernel."""
import pytest
import torch

kda = pytest.importorskip("gated_delta_rule_bounded_amd")

f32, bf16, i32, i64 = torch.float32, torch.bfloat16, torch.int32, torch.int64
H, D, C = 2, 16, 16


def z(*shape, dtype=f32):
    return torch.zeros(*shape, dtype=dtype)


def _device_check(fn):
    """Right sizes: the call gets past every size check and stops where the
    binding asks for device tensors."""
    with pytest.raises(TypeError, match="CUDA"):
        fn()


def _size_error(fn, what):
    with pytest.raises(ValueError, match=what):
        fn()


def test_prefill_sizes():
    T, Tp = 57, 64
    ws = z(kda.kda_prefill_workspace_bytes(Tp, H, D, C), dtype=torch.uint8)

    def call(**kw):
        a = dict(q=z(Tp, H, D), k=z(Tp, H, D), v=z(Tp, H, D), gate=z(Tp, H, D), beta=z(Tp, H),
                 state=z(H, D, D), core=z(Tp, H, D), workspace=ws)
        a.update(kw)
        return lambda: kda.kda_prefill(*a.values(), T=T, T_pad=Tp, heads=H, head_dim=D, chunk=C,
                                       scale=0.25)

    _device_check(call())
    _size_error(call(q=z(Tp - 1, H, D)), "q holds")
    _size_error(call(beta=z(Tp - 1, H)), "beta holds")
    _size_error(call(state=z(H, D, D - 1)), "state holds")
    _size_error(call(core=z(Tp, H, D)[:, :, :8]), "contiguous")
    with pytest.raises(TypeError, match="float32"):
        call(gate=z(Tp, H, D, dtype=bf16))()
    # the phase entry points and the split and bf16-row forms check the same way
    _size_error(lambda: kda.kda_prefill_forward(z(H, D, D), z(Tp - 1, H, D), ws, T=T, T_pad=Tp,
                                                heads=H, head_dim=D, chunk=C, scale=0.25),
                "core holds")
    _size_error(lambda: kda.kda_prefill_split(
        z(Tp, H, D), z(Tp, H, D), z(Tp, H, D), z(Tp, H, D), z(Tp, H), z(H, D, D), z(Tp, H, D),
        z(H, D, D - 1), ws, T=T, cap=9, T_pad=Tp, heads=H, head_dim=D, chunk=C, scale=0.25),
        "cap_state holds")
    _size_error(lambda: kda.kda_prefill_bf16(
        z(Tp, 3 * H * D - 8, dtype=bf16), z(Tp, H, D), z(Tp, H), z(H, D, D), z(Tp, H, D), ws,
        T=T, T_pad=Tp, heads=H, head_dim=D, chunk=C, scale=0.25), "qkv is")


def test_decode_sizes():
    B, K = 3, 4
    n = B * K

    def call(**kw):
        a = dict(qkv=z(n, 3 * H * D, dtype=bf16), gate=z(n, H, D), beta=z(n, H),
                 state=z(B, dtype=i64), core=z(n, H, D))
        a.update(kw)
        snap = kw.pop("snap", z(B * (K - 1), dtype=i64))
        return lambda: kda.kda_decode_k(a["qkv"], a["gate"], a["beta"], a["state"], a["core"], B=B,
                                        K=K, heads=H, head_dim=D, scale=0.25, snap=snap)

    _device_check(call())
    _size_error(call(qkv=z(n - 1, 3 * H * D, dtype=bf16)), "qkv is")
    _size_error(call(state=z(B - 1, dtype=i64)), "state holds")
    _size_error(call(snap=z(B * (K - 1) - 1, dtype=i64)), "snap holds")
    _size_error(call(beta=z(n - 1, H)), "beta holds")
    with pytest.raises(TypeError, match="int64"):
        call(state=z(B, dtype=i32))()
    _size_error(lambda: kda.kda_decode(z(B, 3 * H * D, dtype=bf16), z(B, H, D), z(B, H),
                                       z(B, dtype=i64), z(B - 1, H, D), B=B, heads=H, head_dim=D,
                                       scale=0.25), "core holds")
    # write-on-accept: counts and the report word are checked too
    fold = lambda na, st=None: (lambda: kda.kda_fold_accepted(  # noqa: E731
        z(n, 3 * H * D, dtype=bf16), z(n, H, D), z(n, H), z(B, dtype=i64), na, B=B, K=K, heads=H,
        head_dim=D, status=st))
    _device_check(fold(z(B, dtype=i32)))
    _size_error(fold(z(B - 1, dtype=i32)), "n_accept holds")
    _size_error(fold(z(B, dtype=i32), z(0, dtype=i32)), "status holds")


def test_stage_sizes():
    rows, cd = 10, 3 * H * D
    conv = lambda x, y, tab=None: (lambda: kda.conv_silu_l2(  # noqa: E731
        x, z(cd * 4, dtype=bf16), y, n_seq=2, rows=rows // 2, heads=H, head_dim=D,
        conv_state=tab))
    _device_check(conv(z(rows, cd, dtype=bf16), z(rows, cd, dtype=bf16)))
    _size_error(conv(z(rows - 1, cd, dtype=bf16), z(rows, cd, dtype=bf16)), "x is")
    _size_error(conv(z(rows, cd, dtype=bf16), z(rows, cd - 8, dtype=bf16)), "y is")
    _size_error(conv(z(rows, cd, dtype=bf16), z(rows, cd, dtype=bf16), z(1, dtype=i64)),
                "conv_state holds")
    gate = lambda g, gt: (lambda: kda.kda_gate(g, z(H), z(H * D), gt, T=5, heads=H,  # noqa: E731
                                               head_dim=D))
    _device_check(gate(z(5, H * D, dtype=bf16), z(5, H, D)))
    _size_error(gate(z(5, H * D, dtype=bf16), z(4, H, D)), "gate holds")
    norm = lambda c, o: (lambda: kda.gated_rmsnorm(c, z(5, H * D, dtype=bf16),  # noqa: E731
                                                   z(D, dtype=bf16), o, T=5, heads=H, head_dim=D))
    _device_check(norm(z(5, H, D), z(5, H * D, dtype=bf16)))
    _size_error(norm(z(4, H, D), z(5, H * D, dtype=bf16)), "core is")
    gemv = lambda w: (lambda: kda.dense_gemv_bf16_batchm(  # noqa: E731
        z(4, 64, dtype=bf16), w, z(4, 48, dtype=bf16), M=4, N=48, Kd=64))
    _device_check(gemv(z(48, 64, dtype=bf16)))
    _size_error(gemv(z(47, 64, dtype=bf16)), "w holds")


def test_varlen_sizes():
    rows, B = 40, 3
    ws = z(kda.kda_prefill_varlen_workspace_bytes(B, 4, H, D, C), dtype=torch.uint8)

    def call(**kw):
        a = dict(q=z(rows, H, D), k=z(rows, H, D), v=z(rows, H, D), gate=z(rows, H, D),
                 beta=z(rows, H), state=z(B, dtype=i64), core=z(rows, H, D),
                 cu=z(B + 1, dtype=i32))
        a.update(kw)
        st = kw.get("status")
        return lambda: kda.kda_prefill_varlen(
            a["q"], a["k"], a["v"], a["gate"], a["beta"], a["state"], a["core"], a["cu"], ws,
            B=B, rows=rows, max_chunks=2, total_chunks=4, heads=H, head_dim=D, chunk=C,
            scale=0.25, status=st)

    _device_check(call())
    _device_check(call(status=z(1, dtype=i32)))
    _size_error(call(cu=z(B, dtype=i32)), "cu_seqlens holds")
    _size_error(call(state=z(B - 1, dtype=i64)), "state holds")
    _size_error(call(v=z(rows - 1, H, D)), "v holds")
    with pytest.raises(TypeError, match="int32"):
        call(status=z(1, dtype=i64))()


def test_block_sizes():
    T, Tp, hid, rank = 20, 32, 64, 32
    w = {n: z(c, dtype=f32 if n in ("a_log", "dt_bias") else bf16)
         for n, c in kda._weight_numel(hid, H, D, rank).items()}
    bufs = dict(qkv_proj=z(Tp, 3 * H * D, dtype=bf16), conv_out=z(Tp, 3 * H * D, dtype=bf16),
                fa=z(Tp, rank, dtype=bf16), g_raw=z(Tp, H * D, dtype=bf16),
                b_raw=z(Tp, H, dtype=bf16), gate=z(Tp, H, D), beta=z(Tp, H), core=z(Tp, H, D),
                ga=z(Tp, rank, dtype=bf16), out_gate=z(Tp, H * D, dtype=bf16),
                o_norm_out=z(Tp, H * D, dtype=bf16),
                prefill_ws=z(kda.kda_prefill_workspace_bytes(Tp, H, D, C), dtype=torch.uint8),
                gemm_ws=z(1 << 10, dtype=torch.uint8))

    def call(w_=w, b_=bufs, out=z(T, hid, dtype=bf16)):
        return lambda: kda.kda_block_prefill(z(T, hid, dtype=bf16), w_, z(H, D, D),
                                             z(1, dtype=i64), b_, out, T=T, T_pad=Tp,
                                             hidden_size=hid, heads=H, head_dim=D, rank=rank,
                                             chunk=C, scale=0.25)

    _device_check(call())
    _size_error(call(w_={**w, "o_proj": z(hid * H * D - 1, dtype=bf16)}), "weight o_proj holds")
    _size_error(call(b_={**bufs, "gate": z(Tp - 1, H, D)}), "buffer gate holds")
    _size_error(call(out=z(T - 1, hid, dtype=bf16)), "out holds")
    # block decode: rows of the stage buffers against B * K
    B, K = 2, 3
    dbufs = kda.block_decode_buffers(B * K, heads=H, head_dim=D, rank=rank, device="cpu")

    def dec(b_=dbufs, snap=None):
        return lambda: kda.kda_block_decode_k(z(B * K, hid, dtype=bf16), w, z(B, dtype=i64),
                                              z(B, dtype=i64), b_, z(B * K, hid, dtype=bf16),
                                              B=B, K=K, hidden_size=hid, heads=H, head_dim=D,
                                              rank=rank, scale=0.25, snap=snap)

    _device_check(dec())
    _size_error(dec(b_={**dbufs, "core": z(B * K - 1, H, D)}), "buffer core holds")
    _size_error(dec(snap=z(B * (K - 1) - 1, dtype=i64)), "snap holds")
