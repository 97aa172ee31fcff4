"""Python binding of libkvd.so (include/kvd.h): argument marshalling only.

Every function has the name and argument order of its C entry point.  Tensor
arguments may be torch tensors on a ROCm device (their data pointers are
passed), raw device addresses (int) or None for NULL; ``stream`` may be a
``torch.cuda.Stream``, a raw hipStream_t (int) or None for torch's current
stream.  A nonzero status raises KvdError carrying the status and the
library's message.  All computation happens in the library's HIP kernels;
this module never computes a result itself.

torch is imported before the library is loaded so that libkvd.so binds to the
HIP runtime torch already uses (both resolve the soname libamdhip64.so.7).
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvd.so")

KVD_OK, KVD_ERR_INVALID, KVD_ERR_UNSUPPORTED, KVD_ERR_HIP = 0, 1, 2, 3
KVD_F32, KVD_BF16, KVD_FP8_E4M3, KVD_MXFP4 = 0, 1, 2, 3
DTYPE_CODES = {"f32": KVD_F32, "bf16": KVD_BF16, "fp8": KVD_FP8_E4M3, "mxfp4": KVD_MXFP4}
KVD_LAYOUT_CONTIGUOUS, KVD_LAYOUT_STRIPED, KVD_LAYOUT_STAGGERED16, KVD_LAYOUT_PAGED = 0, 1, 2, 3
LAYOUT_CODES = {"contiguous": KVD_LAYOUT_CONTIGUOUS, "striped": KVD_LAYOUT_STRIPED,
                "staggered16": KVD_LAYOUT_STAGGERED16, "paged": KVD_LAYOUT_PAGED}

# Every symbol include/kvd.h declares.
EXPORTED = ("kvd_decode_partial", "kvd_lse_merge", "kvd_decode_workspace_bytes", "kvd_decode",
            "kvd_decode_noalloc",
            "kvd_append_kv", "kvd_status_string", "kvd_last_error", "kvd_abi_version")
ABI_VERSION = 5
# KVD_NOALLOC_SCRATCH_BYTES of kvd.h: the static partials of kvd_decode_noalloc
NOALLOC_SCRATCH_BYTES = 96 * 1024 * 1024


class KvdProblem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
                ("Dqk", ctypes.c_int32), ("Dv", ctypes.c_int32), ("S_max", ctypes.c_int64),
                ("kvp", ctypes.c_int32), ("q_dtype", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
                ("sm_scale", ctypes.c_float), ("v_aliases_k", ctypes.c_int32), ("layout", ctypes.c_int32),
                ("block_len", ctypes.c_int32), ("max_blocks", ctypes.c_int32), ("num_blocks", ctypes.c_int64),
                ("block_table", ctypes.c_void_p), ("q_tokens", ctypes.c_int32)]


class KvdKV(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("scale", ctypes.c_void_p)]


class KvdError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s (%s)" % (message, _status_name(status)))
        self.status = status
        self.message = message


_lib = None


def _status_name(status):
    return {0: "KVD_OK", 1: "KVD_ERR_INVALID", 2: "KVD_ERR_UNSUPPORTED", 3: "KVD_ERR_HIP"}.get(status, str(status))


def lib() -> ctypes.CDLL:
    """The loaded libkvd.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libkvd.so is not built (%s); run __graft_entry__.build() or "
                               "python -m long_context_decode_split_amd.build" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        P = ctypes.POINTER(KvdProblem)
        L.kvd_decode_partial.argtypes = [P, vp, KvdKV, KvdKV, vp, vp, vp, vp]
        L.kvd_decode_partial.restype = ctypes.c_int
        L.kvd_lse_merge.argtypes = [i32, i64, i32, vp, vp, vp, vp, vp]
        L.kvd_lse_merge.restype = ctypes.c_int
        L.kvd_decode_workspace_bytes.argtypes = [P]
        L.kvd_decode_workspace_bytes.restype = ctypes.c_size_t
        L.kvd_decode.argtypes = [P, vp, KvdKV, KvdKV, vp, vp, vp, vp, vp]
        L.kvd_decode.restype = ctypes.c_int
        L.kvd_decode_noalloc.argtypes = [P, vp, KvdKV, KvdKV, vp, vp, vp, vp]
        L.kvd_decode_noalloc.restype = ctypes.c_int
        L.kvd_append_kv.argtypes = [P, vp, vp, vp, KvdKV, KvdKV, vp]
        L.kvd_append_kv.restype = ctypes.c_int
        L.kvd_status_string.argtypes = [ctypes.c_int]
        L.kvd_status_string.restype = ctypes.c_char_p
        L.kvd_last_error.argtypes = []
        L.kvd_last_error.restype = ctypes.c_char_p
        L.kvd_abi_version.argtypes = []
        L.kvd_abi_version.restype = ctypes.c_int
        if L.kvd_abi_version() != ABI_VERSION:
            raise RuntimeError("libkvd.so ABI version %d, binding expects %d" % (L.kvd_abi_version(), ABI_VERSION))
        _lib = L
    return _lib


def problem(B, Hq, Hkv, Dqk, Dv, S_max, kvp, q_dtype, kv_dtype, sm_scale=0.0, v_aliases_k=False,
            layout="contiguous", block_len=0, max_blocks=0, num_blocks=0, block_table=None,
            q_tokens=1) -> KvdProblem:
    """A kvd_problem; dtypes may be KVD_* codes or 'f32' / 'bf16' / 'fp8' / 'mxfp4', the layout a
    KVD_LAYOUT_* code or 'contiguous' / 'striped' / 'staggered16' / 'paged' (then block_len,
    max_blocks, num_blocks and the device block_table [B,max_blocks] int32 describe the pool);
    q_tokens is T, the query (and appended) tokens per request.
    The problem holds block_table's address: keep the tensor alive while it is used."""
    qd = DTYPE_CODES.get(q_dtype, q_dtype)
    kd = DTYPE_CODES.get(kv_dtype, kv_dtype)
    lay = LAYOUT_CODES.get(layout, layout)
    return KvdProblem(B, Hq, Hkv, Dqk, Dv, S_max, kvp, qd, kd, float(sm_scale), int(bool(v_aliases_k)),
                      int(lay), int(block_len), int(max_blocks), int(num_blocks), _ptr(block_table),
                      int(q_tokens))


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if isinstance(x, torch.Tensor):
        if x.device.type != "cuda":
            raise ValueError("tensor arguments must live on the GPU (got %s)" % x.device)
        if not x.is_contiguous():
            raise ValueError("tensor arguments must be contiguous")
        return x.data_ptr()
    raise TypeError("expected a torch tensor, an int address or None, got %r" % type(x))


def _kv(x) -> KvdKV:
    if x is None:
        return KvdKV(None, None)
    if isinstance(x, KvdKV):
        return x
    data, scale = x
    return KvdKV(_ptr(data), _ptr(scale))


def _stream(s):
    if s is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(status: int):
    if status != KVD_OK:
        raise KvdError(status, lib().kvd_last_error().decode())


def kvd_decode_partial(p: KvdProblem, q, k, v, seq_lens, o_part, lse_part, stream=None) -> None:
    _check(lib().kvd_decode_partial(ctypes.byref(p), _ptr(q), _kv(k), _kv(v), _ptr(seq_lens),
                                    _ptr(o_part), _ptr(lse_part), _stream(stream)))


def kvd_lse_merge(kvp: int, rows: int, Dv: int, o_part, lse_part, o, lse, stream=None) -> None:
    _check(lib().kvd_lse_merge(kvp, rows, Dv, _ptr(o_part), _ptr(lse_part), _ptr(o), _ptr(lse),
                               _stream(stream)))


def kvd_decode_workspace_bytes(p: KvdProblem) -> int:
    return int(lib().kvd_decode_workspace_bytes(ctypes.byref(p)))


def kvd_decode(p: KvdProblem, q, k, v, seq_lens, workspace, o, lse, stream=None) -> None:
    _check(lib().kvd_decode(ctypes.byref(p), _ptr(q), _kv(k), _kv(v), _ptr(seq_lens), _ptr(workspace),
                            _ptr(o), _ptr(lse), _stream(stream)))


def kvd_decode_noalloc(p: KvdProblem, q, k, v, seq_lens, o, lse, stream=None) -> None:
    _check(lib().kvd_decode_noalloc(ctypes.byref(p), _ptr(q), _kv(k), _kv(v), _ptr(seq_lens), _ptr(o),
                                    _ptr(lse), _stream(stream)))


def kvd_append_kv(p: KvdProblem, k_new, v_new, positions, k, v, stream=None) -> None:
    _check(lib().kvd_append_kv(ctypes.byref(p), _ptr(k_new), _ptr(v_new), _ptr(positions), _kv(k), _kv(v),
                               _stream(stream)))


def kvd_status_string(status: int) -> str:
    return lib().kvd_status_string(status).decode()


def kvd_last_error() -> str:
    return lib().kvd_last_error().decode()


def kvd_abi_version() -> int:
    return int(lib().kvd_abi_version())
