"""Thin ctypes binding of libua.so (the C ABI in include/ua.h).

Argument marshalling only: every step of the attention runs in the library's
HIP kernels.  torch supplies device memory and the current stream.  If the
library is not built this module raises on import of any entry point; there is
no fallback path.
"""

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libua.so")

UA_F16, UA_BF16, UA_FP8_E4M3FN, UA_FP8_E4M3FNUZ = 0, 1, 2, 3
UA_PATH_AUTO, UA_PATH_2D, UA_PATH_SPLITKV = 0, 1, 2
UA_CHECK_BITS = {1: "cu_seqlens_q", 2: "q_len", 4: "kv_len", 8: "block_table"}
UA_OK = 0
UA_EPLAN = -5


class UaError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed: {status} ({msg})")
        self.status = status


class UaProblem(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32), ("total_q", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("block_size", ctypes.c_int32),
        ("num_blocks", ctypes.c_int64), ("max_blocks_per_seq", ctypes.c_int32),
        ("max_seqlen_q", ctypes.c_int32), ("max_seqlen_k", ctypes.c_int32),
        ("q_dtype", ctypes.c_int32), ("kv_dtype", ctypes.c_int32), ("o_dtype", ctypes.c_int32),
        ("scale", ctypes.c_float), ("softcap", ctypes.c_float), ("window", ctypes.c_int32),
        ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float),
        ("has_alibi", ctypes.c_int32), ("has_sinks", ctypes.c_int32),
        ("q_stride_tok", ctypes.c_int64), ("q_stride_head", ctypes.c_int64),
        ("o_stride_tok", ctypes.c_int64), ("o_stride_head", ctypes.c_int64),
        ("kv_stride_block", ctypes.c_int64), ("kv_stride_slot", ctypes.c_int64),
        ("kv_stride_head", ctypes.c_int64),
        ("has_qq_bias", ctypes.c_int32), ("qq_bias_stride", ctypes.c_int32),
        ("has_kv_token_scales", ctypes.c_int32), ("reserved0", ctypes.c_int32),
        ("ks_stride_block", ctypes.c_int64), ("ks_stride_slot", ctypes.c_int64),
        ("ks_stride_head", ctypes.c_int64),
        ("vs_stride_block", ctypes.c_int64), ("vs_stride_slot", ctypes.c_int64),
        ("vs_stride_head", ctypes.c_int64),
    ]


class UaPlan(ctypes.Structure):
    _fields_ = [
        ("path", ctypes.c_int32), ("kernel", ctypes.c_int32), ("block_q", ctypes.c_int32),
        ("n_part", ctypes.c_int32), ("grid_x", ctypes.c_int32), ("grid_y", ctypes.c_int32),
        ("grid_z", ctypes.c_int32), ("flags", ctypes.c_int32),
        ("workspace_bytes", ctypes.c_uint64), ("problem_hash", ctypes.c_uint64),
    ]


class UaArgs(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p), ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p), ("cu_seqlens_q", ctypes.c_void_p),
        ("seq_lens", ctypes.c_void_p), ("alibi_slopes", ctypes.c_void_p),
        ("sinks", ctypes.c_void_p), ("out", ctypes.c_void_p), ("lse", ctypes.c_void_p),
        ("qq_bias", ctypes.c_void_p),
        ("k_token_scales", ctypes.c_void_p), ("v_token_scales", ctypes.c_void_p),
    ]


_lib = None
_lib_lock = threading.Lock()

EXPORTS = ["ua_plan", "ua_forward_2d", "ua_forward_splitkv", "ua_reduce", "ua_forward",
           "ua_workspace_acc_offset", "ua_status_string", "ua_check_inputs", "ua_abi_version",
           "ua_forward_noalloc"]
UA_ESCRATCH = -6
# Bytes of the library's static split-KV scratch per GPU (ua_forward_noalloc).
UA_NOALLOC_SCRATCH_BYTES = 64 << 20


def lib():
    """Load libua.so once; raise if it has not been built."""
    global _lib
    with _lib_lock:
        if _lib is None:
            # torch first: the library must bind to the HIP runtime torch loaded
            # (a second runtime loaded before torch's sees no device).
            import torch  # noqa: F401
            if not os.path.exists(LIB_PATH):
                raise ImportError(
                    f"{LIB_PATH} is missing: build it with "
                    "`python -m paged_varlen_attention_ua_amd.build` (no fallback exists)")
            L = ctypes.CDLL(LIB_PATH)
            P = ctypes.POINTER
            L.ua_plan.argtypes = [P(UaProblem), ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                  P(UaPlan)]
            L.ua_plan.restype = ctypes.c_int32
            for fn in ("ua_forward_2d",):
                getattr(L, fn).argtypes = [P(UaProblem), P(UaPlan), P(UaArgs), ctypes.c_void_p]
                getattr(L, fn).restype = ctypes.c_int32
            for fn in ("ua_forward_splitkv", "ua_forward"):
                getattr(L, fn).argtypes = [P(UaProblem), P(UaPlan), P(UaArgs), ctypes.c_void_p,
                                           ctypes.c_size_t, ctypes.c_void_p]
                getattr(L, fn).restype = ctypes.c_int32
            L.ua_reduce.argtypes = [P(UaProblem), P(UaPlan), P(UaArgs), ctypes.c_void_p,
                                    ctypes.c_size_t, ctypes.c_void_p]
            L.ua_reduce.restype = ctypes.c_int32
            L.ua_workspace_acc_offset.argtypes = [P(UaProblem), P(UaPlan)]
            L.ua_workspace_acc_offset.restype = ctypes.c_uint64
            L.ua_status_string.argtypes = [ctypes.c_int32]
            L.ua_status_string.restype = ctypes.c_char_p
            L.ua_check_inputs.argtypes = [P(UaProblem), P(UaArgs), ctypes.c_void_p,
                                          ctypes.c_void_p]
            L.ua_check_inputs.restype = ctypes.c_int32
            L.ua_forward_noalloc.argtypes = [P(UaProblem), P(UaPlan), P(UaArgs),
                                             ctypes.c_void_p]
            L.ua_forward_noalloc.restype = ctypes.c_int32
            L.ua_abi_version.argtypes = []
            L.ua_abi_version.restype = ctypes.c_int32
            _lib = L
    return _lib


def _check(fn, status):
    if status != UA_OK:
        raise UaError(fn, status, lib().ua_status_string(status).decode())


# ----------------------------------------------------------------------------- C entry points

def ua_plan(problem, num_cus=0, force_path=UA_PATH_AUTO, force_n_part=0):
    plan = UaPlan()
    _check("ua_plan", lib().ua_plan(ctypes.byref(problem), num_cus, force_path, force_n_part,
                                    ctypes.byref(plan)))
    return plan


def ua_forward_2d(problem, plan, args, stream=None):
    _check("ua_forward_2d", lib().ua_forward_2d(ctypes.byref(problem), ctypes.byref(plan),
                                                ctypes.byref(args), stream))


def ua_forward_splitkv(problem, plan, args, workspace_ptr, workspace_bytes, stream=None):
    _check("ua_forward_splitkv", lib().ua_forward_splitkv(
        ctypes.byref(problem), ctypes.byref(plan), ctypes.byref(args), workspace_ptr,
        workspace_bytes, stream))


def ua_check_inputs(problem, args, flags_ptr, stream=None):
    _check("ua_check_inputs", lib().ua_check_inputs(ctypes.byref(problem), ctypes.byref(args),
                                                    flags_ptr, stream))


def ua_forward_noalloc(problem, plan, args, stream=None):
    """The planned path with the library's static split-KV scratch (no workspace)."""
    _check("ua_forward_noalloc", lib().ua_forward_noalloc(
        ctypes.byref(problem), ctypes.byref(plan), ctypes.byref(args), stream))


def ua_reduce(problem, plan, args, workspace_ptr, workspace_bytes, stream=None):
    _check("ua_reduce", lib().ua_reduce(ctypes.byref(problem), ctypes.byref(plan),
                                        ctypes.byref(args), workspace_ptr, workspace_bytes,
                                        stream))


def ua_workspace_acc_offset(problem, plan):
    return int(lib().ua_workspace_acc_offset(ctypes.byref(problem), ctypes.byref(plan)))


def ua_abi_version():
    return int(lib().ua_abi_version())
