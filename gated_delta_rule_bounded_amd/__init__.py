"""KDA core for AMD MI355X (gfx950): thin Python binding over ``libkda.so``.

Each function here has the name of a C entry point in ``include/kda.h`` and
only marshals arguments (device pointers, sizes, row strides, the current
torch stream); every step of the computation runs in the library's HIP
kernels.  There is no CPU or PyTorch fallback: if ``libkda.so`` is missing or
fails to load, importing this package raises.

PyTorch supplies device memory and the stream.  Pointer tables (per-sequence
state, snapshots, conv states) are device int64 tensors of addresses; build
them with :func:`ptr_table`.
"""
import ctypes
import os

import torch  # loads the HIP runtime that libkda then shares

from . import _lib
from ._lib import KdaError, last_error  # noqa: F401

__all__ = ["conv_silu_l2", "kda_gate", "kda_prefill", "kda_prefill_noalloc", "kda_prefill_prepare",
           "kda_prefill_forward", "kda_decode", "kda_decode_k",
           "gated_rmsnorm", "kda_prefill_workspace_bytes", "kda_prefill_segment_chunks",
           "kda_prefill_varlen_workspace_bytes",
           "kda_block_prefill", "block_buffers", "BLOCK_WEIGHT_NAMES",
           "dense_gemv_bf16_batchm", "kda_prefill_varlen", "varlen_chunks",
           "kda_verify_k", "kda_fold_accepted", "kda_verify_wy_k", "kda_fold_wy",
           "kda_prefill_split",
           "kda_block_verify_k", "kda_block_fold_accepted", "kda_block_verify_wy_k",
           "kda_block_fold_wy", "kda_prefill_bf16", "kda_block_decode", "kda_block_decode_k",
           "block_decode_buffers",
           "ptr_table", "bind", "KdaError",
           "last_error", "library_path"]


def library_path() -> str:
    return _lib.LIB_PATH


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t, dtype=None, name="tensor"):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _rowstride(t, name):
    if t.dim() < 2 or t.stride(-1) != 1:
        raise ValueError(f"{name} must be 2-D (or more) with unit innermost stride")
    return int(t.stride(0)) if t.dim() == 2 else int(t.stride(-2))


# Size checks.  The library sees only device pointers, so a tensor smaller
# than the call implies would be read or written past its end; every wrapper
# checks its tensors against the sizes of the call first and raises
# ValueError (TypeError for a wrong dtype) before anything reaches the GPU.
def _tensor(t, name, dtype):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _dense(t, name, dtype, numel):
    """A whole-buffer argument: contiguous, at least ``numel`` elements."""
    _tensor(t, name, dtype)
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements; the call needs {numel}")


def _rows(t, name, dtype, rows, width):
    """A row-strided argument: 2-D with unit inner stride, at least ``rows``
    rows of at least ``width`` elements."""
    _tensor(t, name, dtype)
    if t.dim() != 2 or (t.numel() and t.stride(1) != 1):
        raise ValueError(f"{name} must be 2-D with unit innermost stride")
    if t.shape[0] < rows or t.shape[1] < width:
        raise ValueError(f"{name} is {tuple(t.shape)}; the call needs at least ({rows}, {width})")


def _table(t, name, count):
    """A pointer table: contiguous int64 with at least ``count`` entries."""
    _dense(t, name, torch.int64, count)


def _nbytes(t):
    return t.numel() * t.element_size()


def _status(t):
    """Optional run-time report word: a device int32 tensor of >= 1 element."""
    if t is not None:
        _dense(t, "status", torch.int32, 1)
    return _ptr(t, torch.int32, "status")


def _check(rc):
    if rc != 0:
        raise KdaError(rc, _lib.last_error())


class _Recorder:
    """Stands in for the loaded library while :func:`bind` runs a call: each
    C entry point the call reaches is recorded with its arguments, not run."""

    def __init__(self, real):
        self._real, self.calls = real, []

    def __getattr__(self, name):
        fn = getattr(self._real, name)

        def record(*args):
            self.calls.append((fn, args))
            return 0
        return record


def bind(fn, *args, **kwargs):
    """One of this module's launching calls (``fn``) with its arguments,
    checked and marshalled once, returned as a function of no arguments that
    makes the same C call(s) again: the same pointers, sizes and stream (the
    stream current at bind time).  For loops that re-run one call on tensors
    refilled in place, where the per-call checks would cost more host time
    than the GPU work; the tensors must outlive the returned function.
    Nothing is launched by ``bind`` itself.  Not for the size queries, whose
    results it would drop; not thread-safe with other calls of this module."""
    real = _lib.lib
    rec = _Recorder(real)
    _lib.lib = rec
    try:
        fn(*args, **kwargs)
    finally:
        _lib.lib = real
    calls = tuple(rec.calls)
    if not calls:
        raise ValueError(f"bind: {getattr(fn, '__name__', fn)} made no library call")

    def call():
        for f, a in calls:
            _check(f(*a))
    return call


def ptr_table(tensors, device=None):
    """Device int64 tensor of base addresses.

    ``tensors`` is a list of CUDA tensors (one per entry), or one CUDA tensor
    whose leading dimension indexes the entries (entry i = tensors[i])."""
    if isinstance(tensors, torch.Tensor):
        base = tensors.data_ptr()
        step = tensors.stride(0) * tensors.element_size()
        addrs = [base + i * step for i in range(tensors.shape[0])]
        device = device or tensors.device
    else:
        addrs = [t.data_ptr() for t in tensors]
        device = device or (tensors[0].device if tensors else torch.device("cuda"))
    return torch.tensor(addrs, dtype=torch.int64, device=device)


def conv_silu_l2(x, w, y, *, n_seq, rows, heads, head_dim, conv_state=None, conv_snap=None,
                 eps_l2=1e-6, q32=None, k32=None, v32=None, kc=4):
    """Causal depthwise conv + SiLU + q/k L2 (bf16 in/out).  ``conv_state`` and
    ``conv_snap`` are pointer tables from :func:`ptr_table` (or None)."""
    bf = torch.bfloat16
    n = n_seq * rows
    cd = 3 * heads * head_dim
    _rows(x, "x", bf, n, cd)
    _rows(y, "y", bf, n, cd)
    _dense(w, "w", bf, cd * kc)
    if conv_state is not None:
        _table(conv_state, "conv_state", n_seq)
    if conv_snap is not None:
        _table(conv_snap, "conv_snap", n_seq * max(rows - 1, 0))
    for name, t in (("q32", q32), ("k32", k32), ("v32", v32)):
        if t is not None:
            _dense(t, name, torch.float32, n * heads * head_dim)
    _check(_lib.lib.conv_silu_l2(
        _ptr(x, bf, "x"), _rowstride(x, "x"), _ptr(w, bf, "w"),
        _ptr(conv_state, torch.int64, "conv_state"), _ptr(conv_snap, torch.int64, "conv_snap"),
        n_seq, rows, heads, head_dim, kc, float(eps_l2), _ptr(y, bf, "y"), _rowstride(y, "y"),
        _ptr(q32, torch.float32, "q32"), _ptr(k32, torch.float32, "k32"),
        _ptr(v32, torch.float32, "v32"), _stream()))


def kda_gate(g_raw, a_log, dt_bias, gate, *, T, heads, head_dim, b_raw=None, beta=None):
    """gate = -exp(a_log[h]) softplus(g_raw + dt_bias[c]); beta = sigmoid(b_raw)."""
    bf = torch.bfloat16
    qkv = heads * head_dim
    _rows(g_raw, "g_raw", bf, T, qkv)
    _dense(a_log, "a_log", torch.float32, heads)
    _dense(dt_bias, "dt_bias", torch.float32, qkv)
    _dense(gate, "gate", torch.float32, T * qkv)
    if b_raw is not None:
        _rows(b_raw, "b_raw", bf, T, heads)
        if beta is None:
            raise ValueError("beta is required with b_raw")
        _dense(beta, "beta", torch.float32, T * heads)
    ldb = _rowstride(b_raw, "b_raw") if b_raw is not None else 0
    _check(_lib.lib.kda_gate(
        _ptr(g_raw, bf, "g_raw"), _rowstride(g_raw, "g_raw"), _ptr(b_raw, bf, "b_raw"), ldb,
        _ptr(a_log, torch.float32, "a_log"), _ptr(dt_bias, torch.float32, "dt_bias"),
        T, heads, head_dim, _ptr(gate, torch.float32, "gate"),
        _ptr(beta, torch.float32, "beta"), _stream()))


def kda_prefill_workspace_bytes(T_pad, heads, head_dim, chunk):
    return int(_lib.lib.kda_prefill_workspace_bytes(T_pad, heads, head_dim, chunk))


def kda_prefill_varlen_workspace_bytes(B, total_chunks, heads, head_dim, chunk):
    """Workspace of kda_prefill_varlen: the operand blocks of all chunks and
    the call's sequence tables."""
    return int(_lib.lib.kda_prefill_varlen_workspace_bytes(B, total_chunks, heads, head_dim,
                                                           chunk))


def kda_prefill_segment_chunks(T, heads, head_dim, chunk):
    """Chunks per segment that kda_prefill walks at a time."""
    return int(_lib.lib.kda_prefill_segment_chunks(T, heads, head_dim, chunk))


def _prefill_sizes(T_pad, heads, head_dim, rows=None, **ts):
    """Check the fp32 [T_pad, heads, head_dim] row arrays, beta [T_pad, heads],
    the [heads, head_dim, head_dim] state and the workspace of a prefill."""
    f = torch.float32
    rows = T_pad if rows is None else rows
    for name, t in ts.items():
        if name == "workspace":
            _tensor(t, name, None)
            if not t.is_contiguous():
                raise ValueError("workspace must be contiguous")
        elif name == "beta":
            _dense(t, name, f, rows * heads)
        elif name in ("state", "cap_state"):
            _dense(t, name, f, heads * head_dim * head_dim)
        else:
            _dense(t, name, f, rows * heads * head_dim)


def kda_prefill(q, k, v, gate, beta, state, core, workspace, *, T, T_pad, heads, head_dim,
                chunk, scale):
    """Chunked prefill from the carried ``state`` (updated in place)."""
    f = torch.float32
    _prefill_sizes(T_pad, heads, head_dim, q=q, k=k, v=v, gate=gate, beta=beta, state=state,
                   core=core, workspace=workspace)
    _check(_lib.lib.kda_prefill(
        _ptr(q, f, "q"), _ptr(k, f, "k"), _ptr(v, f, "v"), _ptr(gate, f, "gate"),
        _ptr(beta, f, "beta"), _ptr(state, f, "state"), _ptr(core, f, "core"),
        T, T_pad, heads, head_dim, chunk, float(scale), _ptr(workspace, None, "workspace"),
        _nbytes(workspace), _stream()))


def kda_prefill_noalloc(q, k, v, gate, beta, state, core, *, T, T_pad, heads, head_dim, chunk,
                        scale):
    """kda_prefill without a workspace argument: the operand blocks go to the
    library's own 64 MiB device array (see include/kda.h for sharing)."""
    f = torch.float32
    _prefill_sizes(T_pad, heads, head_dim, q=q, k=k, v=v, gate=gate, beta=beta, state=state,
                   core=core)
    _check(_lib.lib.kda_prefill_noalloc(
        _ptr(q, f, "q"), _ptr(k, f, "k"), _ptr(v, f, "v"), _ptr(gate, f, "gate"),
        _ptr(beta, f, "beta"), _ptr(state, f, "state"), _ptr(core, f, "core"),
        T, T_pad, heads, head_dim, chunk, float(scale), _stream()))


def kda_prefill_prepare(q, k, v, gate, beta, workspace, *, T, T_pad, heads, head_dim, chunk):
    """Phase 1 of kda_prefill: every per-chunk operand of the state walk into
    the workspace (reads no state)."""
    f = torch.float32
    _prefill_sizes(T_pad, heads, head_dim, q=q, k=k, v=v, gate=gate, beta=beta,
                   workspace=workspace)
    _check(_lib.lib.kda_prefill_prepare(
        _ptr(q, f, "q"), _ptr(k, f, "k"), _ptr(v, f, "v"), _ptr(gate, f, "gate"),
        _ptr(beta, f, "beta"), T, T_pad, heads, head_dim, chunk,
        _ptr(workspace, None, "workspace"), workspace.numel() * workspace.element_size(),
        _stream()))


def kda_prefill_forward(state, core, workspace, *, T, T_pad, heads, head_dim, chunk, scale):
    """Phase 2 of kda_prefill: walk the chunks from the carried state."""
    f = torch.float32
    _prefill_sizes(T_pad, heads, head_dim, state=state, core=core, workspace=workspace)
    _check(_lib.lib.kda_prefill_forward(
        _ptr(state, f, "state"), _ptr(core, f, "core"), T, T_pad, heads, head_dim, chunk,
        float(scale), _ptr(workspace, None, "workspace"),
        _nbytes(workspace), _stream()))


def _decode_sizes(qkv, gate, beta, state, core, B, K, heads, head_dim, snap=None):
    """Check the [B*K] rows of a decode-family call and its pointer tables."""
    f = torch.float32
    n, qw = B * K, heads * head_dim
    _rows(qkv, "qkv", torch.bfloat16, n, 3 * qw)
    _dense(gate, "gate", f, n * qw)
    _dense(beta, "beta", f, n * heads)
    _table(state, "state", B)
    if core is not None:
        _dense(core, "core", f, n * qw)
    if snap is not None:
        _table(snap, "snap", B * max(K - 1, 0))


def kda_decode(qkv, gate, beta, state, core, *, B, heads, head_dim, scale):
    """One token per sequence; ``state`` is a pointer table (see ptr_table)."""
    f = torch.float32
    _decode_sizes(qkv, gate, beta, state, core, B, 1, heads, head_dim)
    _check(_lib.lib.kda_decode(
        _ptr(qkv, torch.bfloat16, "qkv"), _rowstride(qkv, "qkv"), _ptr(gate, f, "gate"),
        _ptr(beta, f, "beta"), _ptr(state, torch.int64, "state"), _ptr(core, f, "core"),
        B, heads, head_dim, float(scale), _stream()))


def kda_decode_k(qkv, gate, beta, state, core, *, B, K, heads, head_dim, scale, snap=None):
    """K tokens per sequence, bit-identical to K kda_decode calls; ``snap`` is
    a pointer table of B*(K-1) snapshot buffers or None."""
    f = torch.float32
    _decode_sizes(qkv, gate, beta, state, core, B, K, heads, head_dim, snap)
    _check(_lib.lib.kda_decode_k(
        _ptr(qkv, torch.bfloat16, "qkv"), _rowstride(qkv, "qkv"), _ptr(gate, f, "gate"),
        _ptr(beta, f, "beta"), _ptr(state, torch.int64, "state"),
        _ptr(snap, torch.int64, "snap"), _ptr(core, f, "core"), B, K, heads, head_dim,
        float(scale), _stream()))


def gated_rmsnorm(core, out_gate, w, out, *, T, heads, head_dim, eps=1e-5):
    """out = bf16(x / sqrt(mean x^2 + eps) * w * sigmoid(out_gate)) per head."""
    bf = torch.bfloat16
    qw = heads * head_dim
    _tensor(core, "core", torch.float32)
    c2 = core.reshape(core.shape[0], -1) if core.dim() == 3 else core
    _rows(c2, "core", torch.float32, T, qw)
    _rows(out_gate, "out_gate", bf, T, qw)
    _rows(out, "out", bf, T, qw)
    _dense(w, "w", bf, head_dim)
    _check(_lib.lib.gated_rmsnorm(
        _ptr(c2, torch.float32, "core"), _rowstride(c2, "core"), _ptr(out_gate, bf, "out_gate"),
        _rowstride(out_gate, "out_gate"), _ptr(w, bf, "w"), T, heads, head_dim, float(eps),
        _ptr(out, bf, "out"), _rowstride(out, "out"), _stream()))


# weight names of struct kda_block_weights, in order
BLOCK_WEIGHT_NAMES = ("q_proj", "k_proj", "v_proj", "conv", "f_a", "f_b", "dt_bias", "a_log",
                      "b_proj", "g_a", "g_b", "o_norm", "o_proj")


def block_buffers(T_pad, *, heads, head_dim, rank, chunk, device, gemm_ws_bytes=32 << 20,
                  f32_copies=False):
    """Allocate the stage buffers of kda_block_prefill as torch tensors (a
    dict keyed by the fields of struct kda_block_buffers); the optional fp32
    copies q32/k32/v32 only with ``f32_copies``."""
    qkv = heads * head_dim
    bf, f = torch.bfloat16, torch.float32
    e = lambda shape, dt: torch.empty(shape, dtype=dt, device=device)  # noqa: E731
    return dict(
        qkv_proj=e((T_pad, 3 * qkv), bf), conv_out=e((T_pad, 3 * qkv), bf),
        q32=e((T_pad, heads, head_dim), f) if f32_copies else None,
        k32=e((T_pad, heads, head_dim), f) if f32_copies else None,
        v32=e((T_pad, heads, head_dim), f) if f32_copies else None,
        fa=e((T_pad, rank), bf), g_raw=e((T_pad, qkv), bf),
        b_raw=e((T_pad, heads), bf), gate=e((T_pad, heads, head_dim), f),
        beta=e((T_pad, heads), f), core=e((T_pad, heads, head_dim), f), ga=e((T_pad, rank), bf),
        out_gate=e((T_pad, qkv), bf), o_norm_out=e((T_pad, qkv), bf),
        prefill_ws=e((kda_prefill_workspace_bytes(T_pad, heads, head_dim, chunk),), torch.uint8),
        gemm_ws=e((gemm_ws_bytes,), torch.uint8) if gemm_ws_bytes else None)


def _weight_numel(hidden_size, heads, head_dim, rank):
    """Elements of each block weight (layouts of struct kda_block_weights)."""
    qkv = heads * head_dim
    return dict(q_proj=qkv * hidden_size, k_proj=qkv * hidden_size, v_proj=qkv * hidden_size,
                conv=3 * qkv * 4, f_a=rank * hidden_size, f_b=qkv * rank, dt_bias=qkv,
                a_log=heads, b_proj=heads * hidden_size, g_a=rank * hidden_size, g_b=qkv * rank,
                o_norm=head_dim, o_proj=hidden_size * qkv)


def _weight_dtype(n):
    return torch.float32 if n in ("a_log", "dt_bias") else torch.bfloat16


def _check_weights(weights, hidden_size, heads, head_dim, rank):
    need = _weight_numel(hidden_size, heads, head_dim, rank)
    for n in BLOCK_WEIGHT_NAMES:
        _dense(weights[n], f"weight {n}", _weight_dtype(n), need[n])


def _block_weights(weights):
    wts = _lib.BlockWeights()
    for n in BLOCK_WEIGHT_NAMES:
        setattr(wts, n, _ptr(weights[n], _weight_dtype(n), n).value)
    return wts


def kda_block_prefill(hidden, weights, state, conv_state, buffers, out, *, T, T_pad, hidden_size,
                      heads, head_dim, rank, chunk, scale, eps_l2=1e-6, eps_rms=1e-5):
    """One KDA block over T tokens (see include/kda.h).  ``weights`` maps
    BLOCK_WEIGHT_NAMES to device tensors (bf16, a_log and dt_bias fp32);
    ``buffers`` is a dict from :func:`block_buffers`; ``conv_state`` is a
    pointer table (:func:`ptr_table`) of one conv state."""
    bf, f = torch.bfloat16, torch.float32
    _check_weights(weights, hidden_size, heads, head_dim, rank)
    qkv = heads * head_dim
    need = dict(qkv_proj=(bf, 3 * qkv), conv_out=(bf, 3 * qkv), q32=(f, qkv), k32=(f, qkv),
                v32=(f, qkv), fa=(bf, rank), g_raw=(bf, qkv), b_raw=(bf, heads), gate=(f, qkv),
                beta=(f, heads), core=(f, qkv), ga=(bf, rank), out_gate=(bf, qkv),
                o_norm_out=(bf, qkv))
    names = [n for n, _ in _lib.BlockBuffers._fields_ if not n.endswith("_bytes")]
    for n in names:
        t = buffers.get(n)
        if t is not None:
            if n in need:
                _dense(t, f"buffer {n}", need[n][0], T_pad * need[n][1])
            else:
                _dense(t, f"buffer {n}", None, 0)
    _dense(hidden, "hidden", bf, T * hidden_size)
    _dense(out, "out", bf, T * hidden_size)
    _dense(state, "state", f, heads * head_dim * head_dim)
    _table(conv_state, "conv_state", 1)
    wts = _block_weights(weights)
    bufs = _lib.BlockBuffers()
    for n in names:
        t = buffers.get(n)
        setattr(bufs, n, _ptr(t, None, n).value if t is not None else None)
    bufs.prefill_ws_bytes = _nbytes(buffers["prefill_ws"])
    g = buffers.get("gemm_ws")
    bufs.gemm_ws_bytes = _nbytes(g) if g is not None else 0
    _check(_lib.lib.kda_block_prefill(
        _ptr(hidden, bf, "hidden"), ctypes.byref(wts), _ptr(state, torch.float32, "state"),
        _ptr(conv_state, torch.int64, "conv_state"), ctypes.byref(bufs), _ptr(out, bf, "out"),
        T, T_pad, hidden_size, heads, head_dim, rank, chunk, float(scale), float(eps_l2),
        float(eps_rms), _stream()))


def dense_gemv_bf16_batchm(x, w, y, *, M, N, Kd):
    """y[:M] = bf16(x[:M] w^T), each row exactly as it would come out alone."""
    bf = torch.bfloat16
    _rows(x, "x", bf, M, Kd)
    _dense(w, "w", bf, N * Kd)
    _rows(y, "y", bf, M, N)
    _check(_lib.lib.dense_gemv_bf16_batchm(
        _ptr(x, bf, "x"), _rowstride(x, "x"), _ptr(w, bf, "w"), M, N, Kd, _ptr(y, bf, "y"),
        _rowstride(y, "y"), _stream()))


def block_decode_buffers(rows, *, heads, head_dim, rank, device):
    """Allocate the stage buffers of kda_block_decode(_k) for ``rows`` = B*K
    rows (a dict keyed by the fields of struct kda_block_decode_buffers)."""
    qkv = heads * head_dim
    bf, f = torch.bfloat16, torch.float32
    e = lambda shape, dt: torch.empty(shape, dtype=dt, device=device)  # noqa: E731
    return dict(
        qkv_proj=e((rows, 3 * qkv), bf), conv_out=e((rows, 3 * qkv), bf),
        fa=e((rows, rank), bf), g_raw=e((rows, qkv), bf), b_raw=e((rows, heads), bf),
        gate=e((rows, heads, head_dim), f), beta=e((rows, heads), f),
        core=e((rows, heads, head_dim), f), ga=e((rows, rank), bf),
        out_gate=e((rows, qkv), bf), o_norm_out=e((rows, qkv), bf))


def _decode_buffers(buffers, rows, heads, head_dim, rank=None):
    """Struct of the block-decode stage buffers, each checked for ``rows``
    rows (rank=None: the fold, which reads no rank-sized buffer)."""
    bf, f = torch.bfloat16, torch.float32
    qkv = heads * head_dim
    need = dict(qkv_proj=(bf, 3 * qkv), conv_out=(bf, 3 * qkv), fa=(bf, rank or 0),
                g_raw=(bf, qkv), b_raw=(bf, heads), gate=(f, qkv), beta=(f, heads),
                core=(f, qkv), ga=(bf, rank or 0), out_gate=(bf, qkv), o_norm_out=(bf, qkv))
    names = [n for n, _ in _lib.BlockDecodeBuffers._fields_]
    for n in names:
        _dense(buffers[n], f"buffer {n}", need[n][0], rows * need[n][1])

    def build():
        bufs = _lib.BlockDecodeBuffers()
        for n in names:
            setattr(bufs, n, _ptr(buffers[n], None, n).value)
        return bufs
    return build


def _block_decode_sizes(hidden, state, conv_state, out, B, K, hidden_size, snap=None,
                        conv_snap=None):
    bf = torch.bfloat16
    _dense(hidden, "hidden", bf, B * K * hidden_size)
    _dense(out, "out", bf, B * K * hidden_size)
    _table(state, "state", B)
    _table(conv_state, "conv_state", B)
    if snap is not None:
        _table(snap, "snap", B * max(K - 1, 0))
    if conv_snap is not None:
        _table(conv_snap, "conv_snap", B * max(K - 1, 0))


def kda_block_decode_k(hidden, weights, state, conv_state, buffers, out, *, B, K, hidden_size,
                       heads, head_dim, rank, scale, snap=None, conv_snap=None, eps_l2=1e-6,
                       eps_rms=1e-5):
    """K tokens of each of B sequences through the whole block, bit-identical
    to K kda_block_decode calls.  ``state`` / ``conv_state`` are pointer
    tables of B entries; ``snap`` / ``conv_snap`` tables of B*(K-1) or None."""
    bf = torch.bfloat16
    _check_weights(weights, hidden_size, heads, head_dim, rank)
    mk = _decode_buffers(buffers, B * K, heads, head_dim, rank)
    _block_decode_sizes(hidden, state, conv_state, out, B, K, hidden_size, snap, conv_snap)
    wts, bufs = _block_weights(weights), mk()
    _check(_lib.lib.kda_block_decode_k(
        _ptr(hidden, bf, "hidden"), ctypes.byref(wts), _ptr(state, torch.int64, "state"),
        _ptr(conv_state, torch.int64, "conv_state"), _ptr(snap, torch.int64, "snap"),
        _ptr(conv_snap, torch.int64, "conv_snap"), ctypes.byref(bufs), _ptr(out, bf, "out"),
        B, K, hidden_size, heads, head_dim, rank, float(scale), float(eps_l2), float(eps_rms),
        _stream()))


def kda_block_decode(hidden, weights, state, conv_state, buffers, out, *, B, hidden_size, heads,
                     head_dim, rank, scale, eps_l2=1e-6, eps_rms=1e-5):
    """One token of each of B sequences through the whole block."""
    bf = torch.bfloat16
    _check_weights(weights, hidden_size, heads, head_dim, rank)
    mk = _decode_buffers(buffers, B, heads, head_dim, rank)
    _block_decode_sizes(hidden, state, conv_state, out, B, 1, hidden_size)
    wts, bufs = _block_weights(weights), mk()
    _check(_lib.lib.kda_block_decode(
        _ptr(hidden, bf, "hidden"), ctypes.byref(wts), _ptr(state, torch.int64, "state"),
        _ptr(conv_state, torch.int64, "conv_state"), ctypes.byref(bufs), _ptr(out, bf, "out"),
        B, hidden_size, heads, head_dim, rank, float(scale), float(eps_l2), float(eps_rms),
        _stream()))


def varlen_chunks(lengths, chunk):
    """(max_chunks, total_chunks) of kda_prefill_varlen for host-known lengths."""
    n = [-(-int(t) // chunk) for t in lengths]
    return (max(n) if n else 0), sum(n)


def kda_prefill_varlen(q, k, v, gate, beta, state, core, cu_seqlens, workspace, *, B, rows,
                       max_chunks, total_chunks, heads, head_dim, chunk, scale, status=None):
    """B sequences back to back (rows [cu_seqlens[s], cu_seqlens[s+1])), one
    state pointer each (``state``: a :func:`ptr_table`); ``cu_seqlens`` a
    device int32 tensor of B+1 row offsets.  ``status``: an optional device
    int32 word the call ORs its run-time report bits into (a skipped
    sequence: 1; clamped offsets: 2); the caller zeroes it."""
    f = torch.float32
    _prefill_sizes(rows, heads, head_dim, q=q, k=k, v=v, gate=gate, beta=beta, core=core,
                   workspace=workspace)
    _table(state, "state", B)
    _dense(cu_seqlens, "cu_seqlens", torch.int32, B + 1)
    st = _status(status)
    _check(_lib.lib.kda_prefill_varlen(
        _ptr(q, f, "q"), _ptr(k, f, "k"), _ptr(v, f, "v"), _ptr(gate, f, "gate"),
        _ptr(beta, f, "beta"), _ptr(state, torch.int64, "state"), _ptr(core, f, "core"),
        _ptr(cu_seqlens, torch.int32, "cu_seqlens"), B, rows, max_chunks, total_chunks, heads,
        head_dim, chunk, float(scale), _ptr(workspace, None, "workspace"), _nbytes(workspace),
        st, _stream()))


def kda_verify_k(qkv, gate, beta, state, core, *, B, K, heads, head_dim, scale):
    """Outputs of K rows per sequence (bitwise those of kda_decode_k); the
    states are left as they are."""
    f = torch.float32
    _decode_sizes(qkv, gate, beta, state, core, B, K, heads, head_dim)
    _check(_lib.lib.kda_verify_k(
        _ptr(qkv, torch.bfloat16, "qkv"), _rowstride(qkv, "qkv"), _ptr(gate, f, "gate"),
        _ptr(beta, f, "beta"), _ptr(state, torch.int64, "state"), _ptr(core, f, "core"), B, K,
        heads, head_dim, float(scale), _stream()))


def kda_fold_accepted(qkv, gate, beta, state, n_accept, *, B, K, heads, head_dim, status=None):
    """Fold the first n_accept[b] verified rows into each state (``n_accept``
    a device int32 tensor of B counts).  ``status``: an optional device int32
    word that gets bit 4 when a count outside [0, K] was clamped."""
    f = torch.float32
    _decode_sizes(qkv, gate, beta, state, None, B, K, heads, head_dim)
    _dense(n_accept, "n_accept", torch.int32, B)
    st = _status(status)
    _check(_lib.lib.kda_fold_accepted(
        _ptr(qkv, torch.bfloat16, "qkv"), _rowstride(qkv, "qkv"), _ptr(gate, f, "gate"),
        _ptr(beta, f, "beta"), _ptr(state, torch.int64, "state"),
        _ptr(n_accept, torch.int32, "n_accept"), B, K, heads, head_dim, st, _stream()))


def kda_verify_wy_k(qkv, gate, beta, state, wy, core, *, B, K, heads, head_dim, scale):
    """kda_verify_k that also writes each row's u to the WY tables ``wy`` (a
    pointer table of B entries, each fp32 [heads, K, head_dim])."""
    f = torch.float32
    _decode_sizes(qkv, gate, beta, state, core, B, K, heads, head_dim)
    _table(wy, "wy", B)
    _check(_lib.lib.kda_verify_wy_k(
        _ptr(qkv, torch.bfloat16, "qkv"), _rowstride(qkv, "qkv"), _ptr(gate, f, "gate"),
        _ptr(beta, f, "beta"), _ptr(state, torch.int64, "state"), _ptr(wy, torch.int64, "wy"),
        _ptr(core, f, "core"), B, K, heads, head_dim, float(scale), _stream()))


def kda_fold_wy(qkv, gate, state, wy, n_accept, *, B, K, heads, head_dim, status=None):
    """Fold the first n_accept[b] verified rows into each state in one pass
    from the WY tables kda_verify_wy_k wrote (equal to kda_fold_accepted up
    to rounding).  ``status`` as kda_fold_accepted."""
    f = torch.float32
    n, qw = B * K, heads * head_dim
    _rows(qkv, "qkv", torch.bfloat16, n, 3 * qw)
    _dense(gate, "gate", f, n * qw)
    _table(state, "state", B)
    _table(wy, "wy", B)
    _dense(n_accept, "n_accept", torch.int32, B)
    st = _status(status)
    _check(_lib.lib.kda_fold_wy(
        _ptr(qkv, torch.bfloat16, "qkv"), _rowstride(qkv, "qkv"), _ptr(gate, f, "gate"),
        _ptr(state, torch.int64, "state"), _ptr(wy, torch.int64, "wy"),
        _ptr(n_accept, torch.int32, "n_accept"), B, K, heads, head_dim, st, _stream()))


def kda_prefill_split(q, k, v, gate, beta, state, core, cap_state, workspace, *, T, cap, T_pad,
                      heads, head_dim, chunk, scale):
    """Prefill rows [0, cap), copy the state to ``cap_state``, then rows
    [cap, T) on chunks starting at cap (bitwise two kda_prefill calls)."""
    f = torch.float32
    _prefill_sizes(T_pad, heads, head_dim, q=q, k=k, v=v, gate=gate, beta=beta, state=state,
                   core=core, cap_state=cap_state, workspace=workspace)
    _check(_lib.lib.kda_prefill_split(
        _ptr(q, f, "q"), _ptr(k, f, "k"), _ptr(v, f, "v"), _ptr(gate, f, "gate"),
        _ptr(beta, f, "beta"), _ptr(state, f, "state"), _ptr(core, f, "core"),
        _ptr(cap_state, f, "cap_state"), T, cap, T_pad, heads, head_dim, chunk, float(scale),
        _ptr(workspace, None, "workspace"), _nbytes(workspace), _stream()))


def kda_block_verify_k(hidden, weights, state, conv_state, buffers, out, *, B, K, hidden_size,
                       heads, head_dim, rank, scale, eps_l2=1e-6, eps_rms=1e-5):
    """The block over K rows of B sequences, bitwise as kda_block_decode_k,
    with the recurrent and conv states left unwritten."""
    bf = torch.bfloat16
    _check_weights(weights, hidden_size, heads, head_dim, rank)
    mk = _decode_buffers(buffers, B * K, heads, head_dim, rank)
    _block_decode_sizes(hidden, state, conv_state, out, B, K, hidden_size)
    wts, bufs = _block_weights(weights), mk()
    _check(_lib.lib.kda_block_verify_k(
        _ptr(hidden, bf, "hidden"), ctypes.byref(wts), _ptr(state, torch.int64, "state"),
        _ptr(conv_state, torch.int64, "conv_state"), ctypes.byref(bufs), _ptr(out, bf, "out"),
        B, K, hidden_size, heads, head_dim, rank, float(scale), float(eps_l2), float(eps_rms),
        _stream()))


def kda_block_fold_accepted(buffers, state, conv_state, n_accept, *, B, K, heads, head_dim,
                            status=None):
    """Fold the first n_accept[b] verified rows into each recurrent and conv
    state (``buffers`` those of the verify); ``status`` as kda_fold_accepted."""
    mk = _decode_buffers(buffers, B * K, heads, head_dim)
    _table(state, "state", B)
    _table(conv_state, "conv_state", B)
    _dense(n_accept, "n_accept", torch.int32, B)
    st, bufs = _status(status), mk()
    _check(_lib.lib.kda_block_fold_accepted(
        ctypes.byref(bufs), _ptr(state, torch.int64, "state"),
        _ptr(conv_state, torch.int64, "conv_state"), _ptr(n_accept, torch.int32, "n_accept"), B,
        K, heads, head_dim, st, _stream()))


def kda_block_verify_wy_k(hidden, weights, state, conv_state, wy, buffers, out, *, B, K,
                          hidden_size, heads, head_dim, rank, scale, eps_l2=1e-6, eps_rms=1e-5):
    """kda_block_verify_k that also writes the recurrent rows' u values to the
    WY tables ``wy`` (a pointer table of B entries, each fp32 [heads, K,
    head_dim])."""
    bf = torch.bfloat16
    _check_weights(weights, hidden_size, heads, head_dim, rank)
    mk = _decode_buffers(buffers, B * K, heads, head_dim, rank)
    _block_decode_sizes(hidden, state, conv_state, out, B, K, hidden_size)
    _table(wy, "wy", B)
    wts, bufs = _block_weights(weights), mk()
    _check(_lib.lib.kda_block_verify_wy_k(
        _ptr(hidden, bf, "hidden"), ctypes.byref(wts), _ptr(state, torch.int64, "state"),
        _ptr(conv_state, torch.int64, "conv_state"), _ptr(wy, torch.int64, "wy"),
        ctypes.byref(bufs), _ptr(out, bf, "out"), B, K, hidden_size, heads, head_dim, rank,
        float(scale), float(eps_l2), float(eps_rms), _stream()))


def kda_block_fold_wy(buffers, state, conv_state, wy, n_accept, *, B, K, heads, head_dim,
                      status=None):
    """Fold the first n_accept[b] verified rows into each recurrent state in
    one pass from the verify's WY tables, and into each conv state as
    kda_block_fold_accepted does; ``status`` as kda_fold_accepted."""
    mk = _decode_buffers(buffers, B * K, heads, head_dim)
    _table(state, "state", B)
    _table(conv_state, "conv_state", B)
    _table(wy, "wy", B)
    _dense(n_accept, "n_accept", torch.int32, B)
    st, bufs = _status(status), mk()
    _check(_lib.lib.kda_block_fold_wy(
        ctypes.byref(bufs), _ptr(state, torch.int64, "state"),
        _ptr(conv_state, torch.int64, "conv_state"), _ptr(wy, torch.int64, "wy"),
        _ptr(n_accept, torch.int32, "n_accept"), B, K, heads, head_dim, st, _stream()))


def kda_prefill_bf16(qkv, gate, beta, state, core, workspace, *, T, T_pad, heads, head_dim, chunk,
                     scale):
    """kda_prefill reading q | k | v from bf16 rows (``qkv`` [T_pad, >= 3*H*D])."""
    f = torch.float32
    _rows(qkv, "qkv", torch.bfloat16, T_pad, 3 * heads * head_dim)
    _prefill_sizes(T_pad, heads, head_dim, gate=gate, beta=beta, state=state, core=core,
                   workspace=workspace)
    _check(_lib.lib.kda_prefill_bf16(
        _ptr(qkv, torch.bfloat16, "qkv"), _rowstride(qkv, "qkv"), _ptr(gate, f, "gate"),
        _ptr(beta, f, "beta"), _ptr(state, f, "state"), _ptr(core, f, "core"), T, T_pad, heads,
        head_dim, chunk, float(scale), _ptr(workspace, None, "workspace"), _nbytes(workspace),
        _stream()))
