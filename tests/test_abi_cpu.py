"""The C-ABI library loads, exports every symbol include/kda.h declares, and
rejects bad arguments with the documented status codes.  Every call here
returns before any HIP call (validation only), so it runs without a GPU; the
pointer values are never dereferenced."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

OK, E_NULL, E_SHAPE, E_UNSUP, E_ALIAS, E_WS = 0, -1, -2, -3, -4, -5


@pytest.fixture(scope="module")
def lib():
    import gated_delta_rule_bounded_amd as kda
    return kda._lib.lib


def _declared_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", txt)) - {"defined"})


def test_header_declares_the_six_calls():
    names = _declared_functions()
    for n in ("conv_silu_l2", "kda_gate", "kda_prefill", "kda_decode", "kda_decode_k",
              "gated_rmsnorm", "kda_last_error", "kda_prefill_workspace_bytes",
              "kda_prefill_segment_chunks"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    import gated_delta_rule_bounded_amd as kda
    so = ctypes.CDLL(kda.library_path())
    for n in _declared_functions():
        assert hasattr(so, n), f"libkda.so does not export {n}"
    assert set(_declared_functions()) == set(kda._lib.SYMBOLS)


A = 1 << 20          # fake, 256-byte aligned device addresses: never dereferenced
B = 1 << 32
C = 1 << 36
Dp = 1 << 40
E = 1 << 44
F = 1 << 48


def test_prefill_validation(lib):
    ws = lib.kda_prefill_workspace_bytes(4096, 32, 128, 64)
    # one operand block per (chunk, head): 4*C*D + C*C + D floats
    assert ws == (4096 // 64) * 32 * (4 * 64 * 128 + 64 * 64 + 128) * 4
    assert lib.kda_prefill_workspace_bytes(100, 32, 128, 64) == 0     # T_pad % chunk
    # segments of kda_prefill: ceil(workspace of all chunks / 160 MiB) of them,
    # chunks spread evenly; 2 x 32 chunks at T = 4096, one segment when it fits
    per_chunk = 32 * (4 * 64 * 128 + 64 * 64 + 128) * 4
    for T, segs in ((4096, 2), (8192, 4), (2048, 1), (4059, 2), (64, 1), (0, 1)):
        nc = max(1, -(-T // 64))
        assert -(-nc * per_chunk // (160 << 20)) == segs or T == 0
        assert lib.kda_prefill_segment_chunks(T, 32, 128, 64) == -(-nc // segs)
    assert lib.kda_prefill_segment_chunks(4096, 32, 128, 32) == 0     # chunk not built
    assert lib.kda_prefill_segment_chunks(4096, 0, 128, 64) == 0
    args = lambda **kw: [kw.get(n, d) for n, d in (
        ("q", A), ("k", B), ("v", C), ("gate", Dp), ("beta", E), ("state", F), ("core", 1 << 52),
        ("T", 57), ("T_pad", 64), ("H", 2), ("D", 16), ("C", 16), ("scale", 1.0),
        ("ws", 1 << 56), ("wsb", 1 << 30), ("stream", None))]
    assert lib.kda_prefill(*args(D=64)) == E_UNSUP
    assert lib.kda_prefill(*args(C=32)) == E_UNSUP
    assert lib.kda_prefill(*args(T_pad=48)) == E_SHAPE
    assert lib.kda_prefill(*args(T_pad=72)) == E_SHAPE
    assert lib.kda_prefill(*args(T=-1)) == E_SHAPE
    assert lib.kda_prefill(*args(T=0, q=None)) == OK                   # no-op before pointer checks
    assert lib.kda_prefill(*args(q=None)) == E_NULL
    assert lib.kda_prefill(*args(wsb=100)) == E_WS
    assert lib.kda_prefill(*args(core=A)) == E_ALIAS                    # core == q
    assert lib.kda_prefill(*args(state=C + 64)) == E_ALIAS              # state inside v
    assert lib.kda_prefill(*args(q=A + 4)) == E_SHAPE                   # misaligned
    err = lib.kda_last_error().decode()
    assert "misaligned" in err


def test_decode_validation(lib):
    base = dict(qkv=A, ld=3 * 2 * 128, gate=B, beta=C, state=Dp, core=E, Bn=4, H=2, D=128,
                scale=1.0, stream=None)
    order = ("qkv", "ld", "gate", "beta", "state", "core", "Bn", "H", "D", "scale", "stream")
    call = lambda **kw: lib.kda_decode(*[{**base, **kw}[n] for n in order])
    assert call(D=64) == E_UNSUP
    assert call(Bn=-1) == E_SHAPE
    assert call(Bn=0, qkv=None) == OK
    assert call(state=None) == E_NULL
    assert call(ld=100) == E_SHAPE
    assert call(core=B) == E_ALIAS


def test_decode_k_validation(lib):
    base = dict(qkv=A, ld=3 * 2 * 16, gate=B, beta=C, state=Dp, snap=F, core=E, Bn=4, K=4,
                H=2, D=16, scale=1.0, stream=None)
    order = ("qkv", "ld", "gate", "beta", "state", "snap", "core", "Bn", "K", "H", "D", "scale",
             "stream")
    call = lambda **kw: lib.kda_decode_k(*[{**base, **kw}[n] for n in order])
    assert call(K=-1) == E_SHAPE
    assert call(K=0, qkv=None) == OK
    assert call(snap=Dp) == E_ALIAS
    assert call(gate=None) == E_NULL


def test_stage_validation(lib):
    # conv: kc must be 4; y must not alias x; q32/k32/v32 all or none
    conv = lambda **kw: lib.conv_silu_l2(*[{**dict(
        x=A, ldx=96, w=B, st=None, snap=None, n=1, rows=8, H=2, D=16, kc=4, eps=1e-6, y=C,
        ldy=96, q32=None, k32=None, v32=None, stream=None), **kw}[n] for n in (
        "x", "ldx", "w", "st", "snap", "n", "rows", "H", "D", "kc", "eps", "y", "ldy", "q32",
        "k32", "v32", "stream")])
    assert conv(kc=3) == E_UNSUP
    assert conv(y=A) == E_ALIAS
    assert conv(q32=Dp) == E_NULL
    assert conv(ldx=95) == E_SHAPE
    assert conv(rows=0, x=None) == OK
    # gate
    gate = lambda **kw: lib.kda_gate(*[{**dict(
        g=A, ldg=32, b=None, ldb=0, a=B, dt=C, T=5, H=2, D=16, gate=Dp, beta=None,
        stream=None), **kw}[n] for n in ("g", "ldg", "b", "ldb", "a", "dt", "T", "H", "D",
                                          "gate", "beta", "stream")])
    assert gate(D=32) == E_UNSUP
    assert gate(b=E) == E_NULL          # b_raw without beta
    assert gate(gate=A) == E_ALIAS
    assert gate(T=0, g=None) == OK
    # rmsnorm
    norm = lambda **kw: lib.gated_rmsnorm(*[{**dict(
        core=A, ldc=32, og=B, ldo=32, w=C, T=5, H=2, D=16, eps=1e-5, out=Dp, ldy=32,
        stream=None), **kw}[n] for n in ("core", "ldc", "og", "ldo", "w", "T", "H", "D", "eps",
                                          "out", "ldy", "stream")])
    assert norm(out=B) == E_ALIAS
    assert norm(w=None) == E_NULL
    assert norm(ldo=30) == E_SHAPE
    assert norm(T=0, core=None) == OK


def _block_args(lib):
    import gated_delta_rule_bounded_amd as kda
    L = kda._lib
    w = L.BlockWeights()
    for i, (n, _) in enumerate(L.BlockWeights._fields_):
        setattr(w, n, (i + 1) << 36)                 # distinct, far apart, 256-aligned
    b = L.BlockBuffers()
    for i, (n, _) in enumerate(L.BlockBuffers._fields_):
        if not n.endswith("_bytes"):
            setattr(b, n, (i + 20) << 36)
    b.prefill_ws_bytes = lib.kda_prefill_workspace_bytes(128, 2, 16, 16)
    b.gemm_ws_bytes = 1 << 20
    return w, b


def test_block_validation(lib):
    w, b = _block_args(lib)
    ref = ctypes.byref
    H, Dh, hid, rank = 2, 16, 64, 16

    def call(w_=w, b_=b, T=100, T_pad=128, head_dim=Dh, chunk=16, hidden=hid, rk=rank,
             state=60 << 36, out=61 << 36, conv=62 << 36, x=63 << 36):
        return lib.kda_block_prefill(x, ref(w_) if w_ is not None else None, state, conv,
                                     ref(b_) if b_ is not None else None, out, T, T_pad,
                                     hidden, H, head_dim, rk, chunk, 0.25, 1e-6, 1e-5, None)

    assert call(T=0) == OK                                   # no-op before any pointer is used
    assert call(head_dim=64) == E_UNSUP
    assert call(chunk=32) == E_UNSUP
    assert call(T_pad=120) == E_SHAPE                        # T_pad % chunk
    assert call(T=129) == E_SHAPE                            # T_pad < T
    assert call(hidden=60) == E_SHAPE                        # hidden % 8
    assert call(rk=12) == E_SHAPE                            # rank % 8
    assert call(w_=None) == E_NULL
    assert call(b_=None) == E_NULL
    assert call(out=0) == E_NULL
    w2, b2 = _block_args(lib)
    w2.o_proj = None
    assert call(w_=w2) == E_NULL
    w2, b2 = _block_args(lib)
    b2.prefill_ws_bytes -= 1
    assert call(b_=b2) == E_WS
    w2, b2 = _block_args(lib)
    b2.out_gate = b2.g_raw                                   # the pages forbid this alias
    assert call(b_=b2) == E_ALIAS
    w2, b2 = _block_args(lib)
    assert call(out=w2.q_proj) == E_ALIAS                    # writing over a weight
    assert call(state=b2.core + 64) == E_ALIAS
    assert call(x=b2.qkv_proj) == E_ALIAS                    # a buffer over the input
    # the block's conv launch takes T rows as 8-row tiles in grid y
    w3, b3 = _block_args(lib)
    b3.prefill_ws_bytes = lib.kda_prefill_workspace_bytes(65535 * 8 + 16, H, Dh, 16)
    assert call(b_=b3, T=65535 * 8 + 1, T_pad=65535 * 8 + 16) == E_SHAPE


def test_gemv_validation(lib):
    def call(x=A, ldx=256, w=B, M=4, N=48, Kd=256, y=C, ldy=48):
        return lib.dense_gemv_bf16_batchm(x, ldx, w, M, N, Kd, y, ldy, None)

    assert call(M=0) == OK                                   # no-op
    assert call(Kd=100) == E_SHAPE                           # Kd % 32
    assert call(N=0) == E_SHAPE
    assert call(M=-1) == E_SHAPE
    assert call(ldx=128) == E_SHAPE                          # ldx < Kd
    assert call(ldy=40) == E_SHAPE                           # ldy < N
    assert call(x=0) == E_NULL
    assert call(y=A + 64) == E_ALIAS                         # y over x
    assert call(y=B) == E_ALIAS                              # y over the weights
    assert call(x=A + 2) == E_SHAPE                          # misaligned
    assert call(ldx=(1 << 22) + 8) == E_SHAPE                # beyond the 32-bit x offsets


def _decode_bufs():
    import gated_delta_rule_bounded_amd as kda
    b = kda._lib.BlockDecodeBuffers()
    for i, (n, _) in enumerate(kda._lib.BlockDecodeBuffers._fields_):
        setattr(b, n, (i + 20) << 36)
    return b


def test_block_decode_validation(lib):
    w, _ = _block_args(lib)
    b = _decode_bufs()
    ref = ctypes.byref
    H, Dh, hid, rank = 2, 16, 64, 32

    def call(w_=w, b_=b, Bn=3, K=4, head_dim=Dh, hidden=hid, rk=rank, state=60 << 36,
             conv=61 << 36, snap=None, csnap=None, out=62 << 36, x=63 << 36):
        return lib.kda_block_decode_k(x, ref(w_) if w_ is not None else None, state, conv, snap,
                                      csnap, ref(b_) if b_ is not None else None, out, Bn, K,
                                      hidden, H, head_dim, rk, 0.25, 1e-6, 1e-5, None)

    assert call(K=0) == OK and call(Bn=0) == OK
    assert call(head_dim=64) == E_UNSUP
    assert call(hidden=48) == E_SHAPE                        # hidden % 32
    assert call(rk=16) == E_SHAPE                            # rank % 32
    assert call(K=-1) == E_SHAPE
    assert call(w_=None) == E_NULL
    assert call(b_=None) == E_NULL
    assert call(state=0) == E_NULL
    b2 = _decode_bufs()
    b2.core = None
    assert call(b_=b2) == E_NULL
    b2 = _decode_bufs()
    b2.out_gate = b2.g_raw
    assert call(b_=b2) == E_ALIAS
    assert call(out=w.o_proj) == E_ALIAS                     # writing over a weight
    assert call(x=b.qkv_proj) == E_ALIAS
    assert call(snap=60 << 36) == E_ALIAS                    # snapshot table = state table
    assert call(csnap=61 << 36) == E_ALIAS
    # the one-token form is the K = 1 case of the same checks
    assert lib.kda_block_decode(63 << 36, ref(w), 60 << 36, 61 << 36, ref(b), 62 << 36, 3,
                                hid, H, 64, rank, 0.25, 1e-6, 1e-5, None) == E_UNSUP
    assert lib.kda_block_decode(63 << 36, ref(w), 60 << 36, 61 << 36, ref(b), 62 << 36, 0,
                                hid, H, Dh, rank, 0.25, 1e-6, 1e-5, None) == OK


def test_varlen_validation(lib):
    H, Dh, C = 2, 16, 16
    ws = lib.kda_prefill_varlen_workspace_bytes(3, 10, H, Dh, C)

    def call(q=A, core=B, cu=C, state=Dp, wsp=E, ws_bytes=ws, Bn=3, rows=100, mx=4, tot=10,
             head_dim=Dh, chunk=C, status=None):
        return lib.kda_prefill_varlen(q, q + (1 << 30), q + (2 << 30), q + (3 << 30),
                                      q + (4 << 30), state, core, cu, Bn, rows, mx, tot, H,
                                      head_dim, chunk, 0.25, wsp, ws_bytes, status, None)

    assert call(Bn=0) == OK and call(tot=0) == OK and call(rows=0) == OK
    assert call(head_dim=64) == E_UNSUP
    assert call(chunk=32) == E_UNSUP
    assert call(Bn=-1) == E_SHAPE
    assert call(mx=70000) == E_SHAPE
    assert call(cu=0) == E_NULL
    assert call(state=0) == E_NULL
    assert call(ws_bytes=ws - 1) == E_WS
    assert call(core=A + 64) == E_ALIAS                        # core over q
    assert call(wsp=B + 256) == E_ALIAS                        # workspace over core
    assert call(q=A + 4) == E_SHAPE                            # misaligned
    assert call(status=F + 2) == E_SHAPE                       # report word not 4-byte aligned


def test_varlen_workspace_bytes(lib):
    # the operand blocks of every chunk, then (total_chunks + 3B + 1) int32 of
    # sequence tables rounded up to 256 bytes
    blocks = lib.kda_prefill_workspace_bytes(10 * 64, 32, 128, 64)
    assert lib.kda_prefill_varlen_workspace_bytes(3, 10, 32, 128, 64) == blocks + 256
    assert lib.kda_prefill_varlen_workspace_bytes(1000, 10, 32, 128, 64) == blocks + 12288
    assert lib.kda_prefill_varlen_workspace_bytes(1000, 0, 32, 128, 64) == 12032
    for bad in ((-1, 10, 32, 128, 64), (65536, 10, 32, 128, 64), (3, -1, 32, 128, 64),
                (3, 10, 32, 128, 32), (3, 10, 0, 128, 64), (3, (1 << 24) + 1, 32, 128, 64)):
        assert lib.kda_prefill_varlen_workspace_bytes(*bad) == 0, bad


def test_write_on_accept_validation(lib):
    def verify(qkv=A, ld=3 * 32, core=B, Bn=2, K=4, head_dim=16, state=C):
        return lib.kda_verify_k(qkv, ld, Dp, E, state, core, Bn, K, 2, head_dim, 0.25, None)

    def fold(qkv=A, ld=3 * 32, na=F, Bn=2, K=4, head_dim=16, state=C, status=None):
        return lib.kda_fold_accepted(qkv, ld, Dp, E, state, na, Bn, K, 2, head_dim, status, None)

    assert verify(K=0) == OK and fold(Bn=0) == OK
    assert verify(head_dim=64) == E_UNSUP and fold(head_dim=64) == E_UNSUP
    assert verify(K=-1) == E_SHAPE and fold(K=-1) == E_SHAPE
    assert verify(ld=90) == E_SHAPE and fold(ld=90) == E_SHAPE
    assert verify(state=0) == E_NULL and fold(na=0) == E_NULL
    assert verify(core=A + 64) == E_ALIAS                     # core over the qkv rows
    assert fold(status=F + 2) == E_SHAPE                      # report word not 4-byte aligned


def test_write_on_accept_table_validation(lib):
    def verify(qkv=A, ld=3 * 32, core=B, Bn=2, K=4, head_dim=16, state=C, wy=Dp):
        return lib.kda_verify_wy_k(qkv, ld, Dp + 4096, E, state, wy, core, Bn, K, 2, head_dim,
                                   0.25, None)

    def fold(qkv=A, ld=3 * 32, na=F, Bn=2, K=4, head_dim=16, state=C, wy=Dp, status=None):
        return lib.kda_fold_wy(qkv, ld, Dp + 4096, state, wy, na, Bn, K, 2, head_dim, status,
                               None)

    assert verify(K=0) == OK and fold(Bn=0) == OK
    assert verify(head_dim=64) == E_UNSUP and fold(head_dim=64) == E_UNSUP
    assert verify(K=-1) == E_SHAPE and fold(K=-1) == E_SHAPE
    assert verify(ld=90) == E_SHAPE and fold(ld=90) == E_SHAPE
    assert verify(wy=0) == E_NULL and fold(wy=0) == E_NULL and fold(na=0) == E_NULL
    assert verify(wy=C) == E_ALIAS and fold(wy=C) == E_ALIAS   # u-row table is the state table
    assert verify(core=A + 64) == E_ALIAS                        # core over the qkv rows
    assert fold(status=F + 2) == E_SHAPE                         # report word not 4-byte aligned


def test_prefill_split_validation(lib):
    H, Dh, C = 2, 16, 16
    ws = lib.kda_prefill_workspace_bytes(128, H, Dh, C)

    def call(T=100, cap=37, T_pad=128, cap_state=E + (1 << 30), state=Dp, chunk=C):
        return lib.kda_prefill_split(A, A + (1 << 30), A + (2 << 30), A + (3 << 30),
                                     A + (4 << 30), state, B, cap_state, T, cap, T_pad, H, Dh,
                                     chunk, 0.25, E, ws, None)

    assert call(T=0, cap=0) == OK
    assert call(cap=101) == E_SHAPE                            # cap > T
    assert call(cap=-1) == E_SHAPE
    assert call(T=120, cap=1) == E_SHAPE                       # tail chunks end past T_pad
    assert call(chunk=32) == E_UNSUP
    assert call(cap_state=0) == E_NULL
    assert call(cap_state=Dp + 64) == E_ALIAS                  # over the state
    assert call(cap_state=E + 256) == E_ALIAS                  # over the workspace
    assert call(cap_state=A + 4096) == E_ALIAS                 # over q


def test_block_write_on_accept_validation(lib):
    w, _ = _block_args(lib)
    b = _decode_bufs()
    ref = ctypes.byref
    assert lib.kda_block_verify_k(63 << 36, ref(w), 60 << 36, 61 << 36, ref(b), 62 << 36, 3, 0,
                                  64, 2, 16, 32, 0.25, 1e-6, 1e-5, None) == OK
    assert lib.kda_block_verify_k(63 << 36, ref(w), 60 << 36, 61 << 36, ref(b), 62 << 36, 3, 4,
                                  64, 2, 64, 32, 0.25, 1e-6, 1e-5, None) == E_UNSUP
    assert lib.kda_block_verify_k(63 << 36, ref(w), 60 << 36, 61 << 36, ref(b), w.q_proj, 3, 4,
                                  64, 2, 16, 32, 0.25, 1e-6, 1e-5, None) == E_ALIAS
    assert lib.kda_block_fold_accepted(ref(b), 60 << 36, 61 << 36, 64 << 36, 0, 4, 2, 16,
                                       None, None) == OK
    assert lib.kda_block_fold_accepted(ref(b), 60 << 36, 61 << 36, 64 << 36, 3, 4, 2, 64,
                                       None, None) == E_UNSUP
    assert lib.kda_block_fold_accepted(ref(b), 60 << 36, 61 << 36, 0, 3, 4, 2, 16, None,
                                       None) == E_NULL
    assert lib.kda_block_fold_accepted(None, 60 << 36, 61 << 36, 64 << 36, 3, 4, 2, 16,
                                       None, None) == E_NULL
    assert lib.kda_block_fold_accepted(ref(b), 60 << 36, 61 << 36, 64 << 36, 3, -1, 2, 16,
                                       None, None) == E_SHAPE
    assert lib.kda_block_fold_accepted(ref(b), 60 << 36, 61 << 36, 64 << 36, 3, 4, 2, 16,
                                       (65 << 36) + 1, None) == E_SHAPE
    # the table form: the same checks, plus the table of u rows
    wy = 66 << 36
    assert lib.kda_block_verify_wy_k(63 << 36, ref(w), 60 << 36, 61 << 36, wy, ref(b), 62 << 36,
                                     3, 0, 64, 2, 16, 32, 0.25, 1e-6, 1e-5, None) == OK
    assert lib.kda_block_verify_wy_k(63 << 36, ref(w), 60 << 36, 61 << 36, 0, ref(b), 62 << 36,
                                     3, 4, 64, 2, 16, 32, 0.25, 1e-6, 1e-5, None) == E_NULL
    assert lib.kda_block_verify_wy_k(63 << 36, ref(w), 60 << 36, 61 << 36, 60 << 36, ref(b),
                                     62 << 36, 3, 4, 64, 2, 16, 32, 0.25, 1e-6, 1e-5,
                                     None) == E_ALIAS
    assert lib.kda_block_verify_wy_k(63 << 36, ref(w), 60 << 36, 61 << 36, wy, ref(b), 62 << 36,
                                     3, 4, 64, 2, 64, 32, 0.25, 1e-6, 1e-5, None) == E_UNSUP
    assert lib.kda_block_fold_wy(ref(b), 60 << 36, 61 << 36, wy, 64 << 36, 0, 4, 2, 16,
                                 None, None) == OK
    assert lib.kda_block_fold_wy(ref(b), 60 << 36, 61 << 36, 0, 64 << 36, 3, 4, 2, 16,
                                 None, None) == E_NULL
    assert lib.kda_block_fold_wy(ref(b), 60 << 36, 61 << 36, 61 << 36, 64 << 36, 3, 4, 2, 16,
                                 None, None) == E_ALIAS
    assert lib.kda_block_fold_wy(ref(b), 60 << 36, 61 << 36, wy, 64 << 36, 3, 4, 2, 64,
                                 None, None) == E_UNSUP
    assert lib.kda_block_fold_wy(ref(b), 60 << 36, 61 << 36, wy, 64 << 36, 3, 4, 2, 16,
                                 (65 << 36) + 1, None) == E_SHAPE


def test_grid_limits_are_shape_errors(lib):
    # batches past the launch grid's y extent are refused before any launch
    assert lib.kda_decode(A, 96, B, C, Dp, E, 70000, 2, 16, 0.25, None) == E_SHAPE
    assert lib.kda_decode_k(A, 96, B, C, Dp, 0, E, 70000, 2, 2, 16, 0.25, None) == E_SHAPE
    assert lib.kda_verify_k(A, 96, B, C, Dp, E, 70000, 2, 2, 16, 0.25, None) == E_SHAPE
    assert lib.kda_fold_accepted(A, 96, B, C, Dp, E, 70000, 2, 2, 16, None, None) == E_SHAPE
    assert lib.conv_silu_l2(A, 96, B, None, None, 70000, 1, 2, 16, 4, 1e-6, C, 96,
                            None, None, None, None) == E_SHAPE
    # a sequence of conv rows is at most 65535 row tiles of 8 rows (grid y)
    assert lib.conv_silu_l2(A, 96, B, None, None, 1, 65535 * 8 + 1, 2, 16, 4, 1e-6, C, 96,
                            None, None, None, None) == E_SHAPE
    assert "rows=524281" in lib.kda_last_error().decode()
    assert lib.dense_gemv_bf16_batchm(A, 256, B, 65535 * 64 + 1, 48, 256, C, 48, None) == E_SHAPE


def test_block_fold_alignment(lib):
    b = _decode_bufs()
    b.conv_out += 2
    assert lib.kda_block_fold_accepted(ctypes.byref(b), 60 << 36, 61 << 36, 64 << 36, 3, 4, 2, 16,
                                       None, None) == E_SHAPE


def test_prefill_bf16_validation(lib):
    H, Dh, C = 2, 16, 16
    ws = lib.kda_prefill_workspace_bytes(64, H, Dh, C)

    def call(qkv=A, ld=96, gate=B, beta=C, state=Dp, core=E, wsp=F, ws_bytes=ws, T=57, T_pad=64):
        return lib.kda_prefill_bf16(qkv, ld, gate, beta, state, core, T, T_pad, H, Dh, C, 0.25,
                                    wsp, ws_bytes, None)

    assert call(T=0) == OK
    assert call(ld=90) == E_SHAPE and call(ld=98) == E_SHAPE       # < 3*H*D, not % 4
    assert call(qkv=A + 4) == E_SHAPE                              # 8-byte alignment
    assert call(ws_bytes=ws - 1) == E_WS
    assert call(core=A + 64) == E_ALIAS                            # core over the rows
    assert call(wsp=B) == E_ALIAS                                  # workspace over the gate
    assert call(state=C) == E_ALIAS                                # state over beta


def test_bind_records_then_replays(monkeypatch):
    # kda.bind runs the wrapper once against a recorder (no library call is
    # made), then each call of the returned function repeats the recorded C
    # calls in order with the same arguments, and a failing status raises
    import gated_delta_rule_bounded_amd as kda
    made = []

    class FakeLib:
        rc = 0

        def kda_first(self, *a):
            made.append(("first",) + a)
            return self.rc

        def kda_second(self, *a):
            made.append(("second",) + a)
            return self.rc

        def kda_last_error(self):
            return b"fake failure"

    fake = FakeLib()
    monkeypatch.setattr(kda._lib, "lib", fake)

    def two_calls(v, *, w):
        kda._check(kda._lib.lib.kda_first(v, w))
        kda._check(kda._lib.lib.kda_second(w))

    again = kda.bind(two_calls, 7, w=3)
    assert made == []
    assert kda._lib.lib is fake
    again()
    again()
    assert made == [("first", 7, 3), ("second", 3)] * 2
    fake.rc = -2
    with pytest.raises(kda.KdaError, match="fake failure"):
        again()
    with pytest.raises(ValueError):
        kda.bind(lambda: None)
