"""ctypes declarations of the libkda C ABI (include/kda.h).

The library is built in-tree by ``build.py``; loading it never compiles and
never falls back to anything else: a missing or unloadable library raises.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkda.so")

# exported C symbols, as declared in include/kda.h
SYMBOLS = ("kda_last_error", "conv_silu_l2", "kda_gate", "kda_prefill_workspace_bytes",
           "kda_prefill_segment_chunks", "kda_prefill", "kda_prefill_prepare",
           "kda_prefill_forward", "kda_decode", "kda_decode_k", "gated_rmsnorm",
           "kda_block_prefill", "dense_gemv_bf16_batchm", "kda_block_decode_k",
           "kda_block_decode", "kda_prefill_varlen", "kda_verify_k", "kda_fold_accepted",
           "kda_prefill_split", "kda_block_verify_k", "kda_block_fold_accepted",
           "kda_prefill_bf16", "kda_prefill_noalloc", "kda_prefill_varlen_workspace_bytes",
           "kda_verify_wy_k", "kda_fold_wy", "kda_block_verify_wy_k", "kda_block_fold_wy")


class BlockWeights(ctypes.Structure):
    """struct kda_block_weights (include/kda.h)."""
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "q_proj", "k_proj", "v_proj", "conv", "f_a", "f_b", "dt_bias", "a_log", "b_proj",
        "g_a", "g_b", "o_norm", "o_proj")]


class BlockBuffers(ctypes.Structure):
    """struct kda_block_buffers (include/kda.h)."""
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "qkv_proj", "conv_out", "q32", "k32", "v32", "fa", "g_raw", "b_raw", "gate", "beta",
        "core", "ga", "out_gate", "o_norm_out", "prefill_ws")] + [
        ("prefill_ws_bytes", ctypes.c_size_t), ("gemm_ws", ctypes.c_void_p),
        ("gemm_ws_bytes", ctypes.c_size_t)]


class BlockDecodeBuffers(ctypes.Structure):
    """struct kda_block_decode_buffers (include/kda.h)."""
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "qkv_proj", "conv_out", "fa", "g_raw", "b_raw", "gate", "beta", "core", "ga",
        "out_gate", "o_norm_out")]


class KdaError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"libkda error {code}: {msg}")
        self.code = code


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libkda.so not built at {LIB_PATH}; run "
                          "`python gated_delta_rule_bounded_amd/build.py` (or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    i32, i64, f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    lib.kda_last_error.restype = ctypes.c_char_p
    lib.kda_last_error.argtypes = []
    lib.conv_silu_l2.restype = ctypes.c_int
    lib.conv_silu_l2.argtypes = [P, i64, P, P, P, i32, i32, i32, i32, i32, f32, P, i64, P, P, P, P]
    lib.kda_gate.restype = ctypes.c_int
    lib.kda_gate.argtypes = [P, i64, P, i64, P, P, i32, i32, i32, P, P, P]
    lib.kda_prefill_workspace_bytes.restype = ctypes.c_size_t
    lib.kda_prefill_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.kda_prefill_segment_chunks.restype = ctypes.c_int32
    lib.kda_prefill_segment_chunks.argtypes = [i32, i32, i32, i32]
    lib.kda_prefill_varlen_workspace_bytes.restype = ctypes.c_size_t
    lib.kda_prefill_varlen_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.kda_prefill.restype = ctypes.c_int
    lib.kda_prefill.argtypes = [P, P, P, P, P, P, P, i32, i32, i32, i32, i32, f32, P,
                                ctypes.c_size_t, P]
    lib.kda_prefill_noalloc.restype = ctypes.c_int
    lib.kda_prefill_noalloc.argtypes = [P, P, P, P, P, P, P, i32, i32, i32, i32, i32, f32, P]
    lib.kda_prefill_prepare.restype = ctypes.c_int
    lib.kda_prefill_prepare.argtypes = [P, P, P, P, P, i32, i32, i32, i32, i32, P,
                                        ctypes.c_size_t, P]
    lib.kda_prefill_forward.restype = ctypes.c_int
    lib.kda_prefill_forward.argtypes = [P, P, i32, i32, i32, i32, i32, f32, P, ctypes.c_size_t, P]
    lib.kda_decode.restype = ctypes.c_int
    lib.kda_decode.argtypes = [P, i64, P, P, P, P, i32, i32, i32, f32, P]
    lib.kda_decode_k.restype = ctypes.c_int
    lib.kda_decode_k.argtypes = [P, i64, P, P, P, P, P, i32, i32, i32, i32, f32, P]
    lib.gated_rmsnorm.restype = ctypes.c_int
    lib.gated_rmsnorm.argtypes = [P, i64, P, i64, P, i32, i32, i32, f32, P, i64, P]
    lib.kda_block_prefill.restype = ctypes.c_int
    lib.kda_block_prefill.argtypes = [P, ctypes.POINTER(BlockWeights), P, P,
                                      ctypes.POINTER(BlockBuffers), P] + [i32] * 7 + [f32] * 3 + [P]
    lib.kda_prefill_bf16.restype = ctypes.c_int
    lib.kda_prefill_bf16.argtypes = [P, i64, P, P, P, P, i32, i32, i32, i32, i32, f32, P,
                                     ctypes.c_size_t, P]
    lib.kda_prefill_split.restype = ctypes.c_int
    lib.kda_prefill_split.argtypes = [P, P, P, P, P, P, P, P, i32, i32, i32, i32, i32, i32, f32,
                                      P, ctypes.c_size_t, P]
    lib.kda_verify_k.restype = ctypes.c_int
    lib.kda_verify_k.argtypes = [P, i64, P, P, P, P, i32, i32, i32, i32, f32, P]
    lib.kda_fold_accepted.restype = ctypes.c_int
    lib.kda_fold_accepted.argtypes = [P, i64, P, P, P, P, i32, i32, i32, i32, P, P]
    lib.kda_verify_wy_k.restype = ctypes.c_int
    lib.kda_verify_wy_k.argtypes = [P, i64, P, P, P, P, P, i32, i32, i32, i32, f32, P]
    lib.kda_fold_wy.restype = ctypes.c_int
    lib.kda_fold_wy.argtypes = [P, i64, P, P, P, P, i32, i32, i32, i32, P, P]
    lib.kda_prefill_varlen.restype = ctypes.c_int
    lib.kda_prefill_varlen.argtypes = [P, P, P, P, P, P, P, P, i32, i32, i32, i32, i32, i32, i32,
                                       f32, P, ctypes.c_size_t, P, P]
    lib.dense_gemv_bf16_batchm.restype = ctypes.c_int
    lib.dense_gemv_bf16_batchm.argtypes = [P, i64, P, i32, i32, i32, P, i64, P]
    lib.kda_block_decode_k.restype = ctypes.c_int
    lib.kda_block_decode_k.argtypes = [P, ctypes.POINTER(BlockWeights), P, P, P, P,
                                       ctypes.POINTER(BlockDecodeBuffers), P] + [i32] * 6 + \
        [f32] * 3 + [P]
    lib.kda_block_verify_k.restype = ctypes.c_int
    lib.kda_block_verify_k.argtypes = [P, ctypes.POINTER(BlockWeights), P, P,
                                       ctypes.POINTER(BlockDecodeBuffers), P] + [i32] * 6 + \
        [f32] * 3 + [P]
    lib.kda_block_fold_accepted.restype = ctypes.c_int
    lib.kda_block_fold_accepted.argtypes = [ctypes.POINTER(BlockDecodeBuffers), P, P, P, i32, i32,
                                            i32, i32, P, P]
    lib.kda_block_verify_wy_k.restype = ctypes.c_int
    lib.kda_block_verify_wy_k.argtypes = [P, ctypes.POINTER(BlockWeights), P, P, P,
                                          ctypes.POINTER(BlockDecodeBuffers), P] + [i32] * 6 + \
        [f32] * 3 + [P]
    lib.kda_block_fold_wy.restype = ctypes.c_int
    lib.kda_block_fold_wy.argtypes = [ctypes.POINTER(BlockDecodeBuffers), P, P, P, P, i32, i32,
                                      i32, i32, P, P]
    lib.kda_block_decode.restype = ctypes.c_int
    lib.kda_block_decode.argtypes = [P, ctypes.POINTER(BlockWeights), P, P,
                                     ctypes.POINTER(BlockDecodeBuffers), P] + [i32] * 5 + \
        [f32] * 3 + [P]
    return lib


lib = _load()


def last_error() -> str:
    return lib.kda_last_error().decode()
