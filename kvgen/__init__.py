"""Seeded synthetic inputs for split-KV decode attention.

This module is shared by the GPU tests, the benchmark and the CPU oracle's
tests.  It only *produces* inputs (random values and their encodings into the
cache formats); it contains none of the attention arithmetic and none of the
decoding that either side performs.  The generator itself is C++
(``gen.cpp``, built into ``libkvgen.so``) so that multi-gigabyte caches can be
produced in seconds and any slab can be regenerated on its own.

Streams: element ``i`` of stream ``s`` under seed ``seed`` is a fixed function
of ``(seed, s, i)``; the query uses stream 0, K stream 1, V stream 2 and the
sequence lengths stream 3.  Tensors are generated in the flat order of their
canonical layout (``q [B,Hq,Dqk]``, ``k/v [B,Hkv,S_max,D]``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field, replace
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gen.cpp")
_LIB_PATH = os.path.join(_HERE, "libkvgen.so")

STREAM_Q, STREAM_K, STREAM_V, STREAM_SEQLEN = 0, 1, 2, 3

KV_DTYPES = ("f32", "bf16", "fp8", "mxfp4")
Q_DTYPES = ("f32", "bf16")


def build(force: bool = False) -> str:
    """Compile libkvgen.so with g++ (host code only)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["g++", "-O3", "-fPIC", "-shared", "-pthread", "-ffp-contract=off",
                               _SRC, "-o", tmp])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib_handle = None


def _lib():
    global _lib_handle
    if _lib_handle is None:
        build()
        L = ctypes.CDLL(_LIB_PATH)
        u64, i64, i32, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        L.kvgen_normal_f64.argtypes = [u64, u64, u64, u64, vp, i32]
        L.kvgen_f32.argtypes = [u64, u64, u64, u64, vp, i32]
        L.kvgen_bf16.argtypes = [u64, u64, u64, u64, vp, i32]
        L.kvgen_fp8_slabs.argtypes = [u64, u64, u64, u64, u64, vp, vp, i32]
        L.kvgen_mxfp4.argtypes = [u64, u64, u64, u64, ctypes.c_uint32, vp, vp, i32]
        L.kvgen_uniform_int.argtypes = [u64, u64, u64, i64, i64, vp]
        L.kvgen_encode_e4m3.argtypes = [vp, u64, vp]
        L.kvgen_encode_e2m1.argtypes = [vp, u64, vp]
        for f in ("kvgen_normal_f64", "kvgen_f32", "kvgen_bf16", "kvgen_fp8_slabs", "kvgen_mxfp4",
                  "kvgen_uniform_int", "kvgen_encode_e4m3", "kvgen_encode_e2m1"):
            getattr(L, f).restype = None
        _lib_handle = L
    return _lib_handle


def default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def _out(out, shape, dtype):
    if out is None:
        return np.empty(shape, dtype=dtype)
    assert out.dtype == np.dtype(dtype) and out.size == int(np.prod(shape)), (out.dtype, out.shape, shape)
    return out.reshape(shape)


# ---------------------------------------------------------------- raw streams
def normals_f64(seed: int, stream: int, start: int, count: int, threads: Optional[int] = None) -> np.ndarray:
    out = np.empty(count, dtype=np.float64)
    _lib().kvgen_normal_f64(seed, stream, start, count, _ptr(out), threads or default_threads())
    return out


def normals_f32(seed, stream, start, count, threads=None, out=None) -> np.ndarray:
    out = _out(out, (count,), np.float32)
    _lib().kvgen_f32(seed, stream, start, count, _ptr(out), threads or default_threads())
    return out


def normals_bf16(seed, stream, start, count, threads=None, out=None) -> np.ndarray:
    """bf16 bit patterns (uint16) of the N(0,1) stream, RNE via fp32."""
    out = _out(out, (count,), np.uint16)
    _lib().kvgen_bf16(seed, stream, start, count, _ptr(out), threads or default_threads())
    return out


def fp8_slabs(seed, stream, first_slab, nslabs, slab_len, threads=None, out=None, out_scale=None):
    codes = _out(out, (nslabs * slab_len,), np.uint8)
    scales = _out(out_scale, (nslabs,), np.float32)
    _lib().kvgen_fp8_slabs(seed, stream, first_slab, nslabs, slab_len, _ptr(codes), _ptr(scales),
                           threads or default_threads())
    return codes, scales


def mxfp4_rows(seed, stream, start_row, nrows, D, threads=None, out=None, out_scale=None):
    assert D % 32 == 0
    data = _out(out, (nrows * D // 2,), np.uint8)
    scales = _out(out_scale, (nrows * D // 32,), np.uint8)
    _lib().kvgen_mxfp4(seed, stream, start_row, nrows, D, _ptr(data), _ptr(scales),
                       threads or default_threads())
    return data, scales


def uniform_int(seed, stream, count, lo, hi) -> np.ndarray:
    out = np.empty(count, dtype=np.int32)
    _lib().kvgen_uniform_int(seed, stream, count, lo, hi, _ptr(out))
    return out


def encode_e4m3(values) -> np.ndarray:
    v = np.ascontiguousarray(values, dtype=np.float32).ravel()
    out = np.empty(v.size, dtype=np.uint8)
    _lib().kvgen_encode_e4m3(_ptr(v), v.size, _ptr(out))
    return out


def encode_e2m1(values) -> np.ndarray:
    v = np.ascontiguousarray(values, dtype=np.float64).ravel()
    out = np.empty(v.size, dtype=np.uint8)
    _lib().kvgen_encode_e2m1(_ptr(v), v.size, _ptr(out))
    return out


# ------------------------------------------------ encoding given values
# Planted test inputs (values chosen by a test rather than drawn from a
# stream) are encoded by the same rules as the generated tensors.
def encode_fp8_slab(values):
    """(codes, scale) of one (request, KV head) slab of given values: scale =
    amax / 448 in fp32 (1 for an all-zero slab), each code the nearest E4M3 of
    x / scale (fp32 division), ties to even, saturated to +-448."""
    x = np.ascontiguousarray(values, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0.0)
    scale = np.float32(amax / np.float32(448.0)) if amax > 0 else np.float32(1.0)
    codes = encode_e4m3(x / scale).reshape(x.shape)
    return codes, scale


def pack_mxfp4(codes, exponents):
    """MXFP4 bytes from E2M1 codes [..., D] (4-bit, sign in bit 3) and E8M0
    exponents [..., D/32]: (data [..., D/2] with element 2i in the low nibble,
    scales [..., D/32])."""
    c = np.asarray(codes, dtype=np.uint8)
    data = (c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)
    return (np.ascontiguousarray(data, dtype=np.uint8),
            np.ascontiguousarray(np.asarray(exponents), dtype=np.uint8))


def encode_mxfp4(values):
    """MXFP4 rows of given values [..., D] (D % 32 == 0) by the generated rows'
    rule: per 32-element block E = clamp(floor(log2 amax) - 2 + 127, 0, 254)
    (127 for an all-zero block) and elements the nearest E2M1 of
    x 2^(127 - E), ties to even, saturated to +-6."""
    x = np.asarray(values, dtype=np.float32).astype(np.float64)
    D = x.shape[-1]
    assert D % 32 == 0
    blocks = x.reshape(x.shape[:-1] + (D // 32, 32))
    amax = np.abs(blocks).max(axis=-1)
    _, e2 = np.frexp(amax)                       # amax = m 2^e2, m in [0.5, 1)
    E = np.where(amax > 0, np.clip(e2 - 1 - 2 + 127, 0, 254), 127).astype(np.int64)
    scaled = blocks * np.ldexp(1.0, (127 - E))[..., None]
    codes = encode_e2m1(scaled).reshape(x.shape)
    return pack_mxfp4(codes, E)


# -------------------------------------------------------------- workloads
@dataclass(frozen=True)
class Workload:
    """Shape, formats and seed of one synthetic decode-attention problem.

    ``seq_lens`` is either None (every request uses ``S_max`` tokens), a tuple
    of explicit lengths, or ``("uniform", lo, hi)`` (integers drawn uniformly
    in [lo, hi] from stream 3).
    """
    name: str
    B: int
    Hq: int
    Hkv: int
    Dqk: int
    Dv: int
    S_max: int
    kvp: tuple
    q_dtype: str
    kv_dtype: str
    seed: int
    seq_lens: object = None
    v_aliases_k: bool = False
    q_tokens: int = 1          # new query tokens per request (T)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    # MQA decode, fp32 throughout; KVP=4.
    "mqa_f32": Workload("mqa_f32", B=1, Hq=8, Hkv=1, Dqk=64, Dv=64, S_max=4096, kvp=(4,),
                        q_dtype="f32", kv_dtype="f32", seed=1001),
    # GQA group 16, bf16 cache, per-request lengths uniform in [65536, 131072]; KVP=16.
    "gqa_bf16_varlen": Workload("gqa_bf16_varlen", B=8, Hq=128, Hkv=8, Dqk=128, Dv=128,
                                S_max=131072, kvp=(16,), q_dtype="bf16", kv_dtype="bf16",
                                seed=1002, seq_lens=("uniform", 65536, 131072)),
    # Helix Figure-1 dense shape, one layer: B=8, 128/8 heads, Hsz=128, S=2^20, fp8 E4M3 cache.
    "helix_fp8": Workload("helix_fp8", B=8, Hq=128, Hkv=8, Dqk=128, Dv=128, S_max=1 << 20,
                          kvp=(8, 32, 128), q_dtype="bf16", kv_dtype="fp8", seed=1003),
    # Same shape with an MXFP4 cache.
    "helix_mxfp4": Workload("helix_mxfp4", B=8, Hq=128, Hkv=8, Dqk=128, Dv=128, S_max=1 << 20,
                            kvp=(8, 32, 128), q_dtype="bf16", kv_dtype="mxfp4", seed=1004),
    # MXFP4 batch sweep at S=2^18.
    "mxfp4_b1_s256k": Workload("mxfp4_b1_s256k", B=1, Hq=128, Hkv=8, Dqk=128, Dv=128,
                               S_max=1 << 18, kvp=(8, 32, 128), q_dtype="bf16", kv_dtype="mxfp4",
                               seed=1004),
    "mxfp4_b32_s256k": Workload("mxfp4_b32_s256k", B=32, Hq=128, Hkv=8, Dqk=128, Dv=128,
                                S_max=1 << 18, kvp=(8, 32, 128), q_dtype="bf16",
                                kv_dtype="mxfp4", seed=1004),
    # One GPU's share of the Helix shape at TPA=8, KVP=8 (one KV head of 16 query
    # heads, S/8 = 131072 resident tokens per request), split further over the
    # GPU's own compute units; the whole cache fits the 256 MB last-level cache.
    "helix_shard_fp8": Workload("helix_shard_fp8", B=8, Hq=16, Hkv=1, Dqk=128, Dv=128,
                                S_max=1 << 17, kvp=(64, 16, 128), q_dtype="bf16", kv_dtype="fp8",
                                seed=1006),
    "helix_shard_mxfp4": Workload("helix_shard_mxfp4", B=8, Hq=16, Hkv=1, Dqk=128, Dv=128,
                                  S_max=1 << 17, kvp=(64, 16, 128), q_dtype="bf16",
                                  kv_dtype="mxfp4", seed=1007),
    # A group of 8 query heads per KV head at the Helix length: B=8, 64/8 heads,
    # Hsz=128, S=2^20, fp8 E4M3 cache.
    "gqa8_fp8": Workload("gqa8_fp8", B=8, Hq=64, Hkv=8, Dqk=128, Dv=128, S_max=1 << 20,
                         kvp=(32, 8, 128), q_dtype="bf16", kv_dtype="fp8", seed=1008),
    # MLA-style: 128 query heads on one 576-wide latent head; V = first 512 dims of K.
    "mla_bf16": Workload("mla_bf16", B=8, Hq=128, Hkv=1, Dqk=576, Dv=512, S_max=1 << 19,
                         kvp=(32,), q_dtype="bf16", kv_dtype="bf16", seed=1005,
                         v_aliases_k=True),
}


@dataclass
class Inputs:
    """Encoded host-side inputs in the library's layouts.

    q        [B,Hq,Dqk] ([B,T,Hq,Dqk] for T > 1 query tokens) float32, or
             uint16 bf16 bit patterns
    k_data   [B,Hkv,S_max,D]  float32 / uint16 (bf16) / uint8 (fp8 codes);
             MXFP4: uint8 [B,Hkv,S_max,D/2], element 2i in the low nibble
    k_scale  fp8: float32 [B,Hkv]; MXFP4: uint8 E8M0 [B,Hkv,S_max,D/32]; else None
    v_*      the same for V (None when V aliases K)
    seq_lens int32 [B]
    """
    workload: Workload
    q: np.ndarray
    k_data: np.ndarray
    k_scale: Optional[np.ndarray]
    v_data: Optional[np.ndarray]
    v_scale: Optional[np.ndarray]
    seq_lens: np.ndarray


def gen_seq_lens(w: Workload) -> np.ndarray:
    if w.seq_lens is None:
        return np.full(w.B, w.S_max, dtype=np.int32)
    if isinstance(w.seq_lens, tuple) and len(w.seq_lens) == 3 and w.seq_lens[0] == "uniform":
        _, lo, hi = w.seq_lens
        return uniform_int(w.seed, STREAM_SEQLEN, w.B, lo, hi)
    sl = np.asarray(w.seq_lens, dtype=np.int32)
    assert sl.shape == (w.B,)
    return sl


def gen_q(w: Workload, threads=None) -> np.ndarray:
    """q [B,Hq,Dqk] for one query token, [B,T,Hq,Dqk] for T = q_tokens > 1
    (the same flat stream, so a T = 1 query is the first token's)."""
    T = w.q_tokens
    shape = (w.B, w.Hq, w.Dqk) if T == 1 else (w.B, T, w.Hq, w.Dqk)
    n = w.B * T * w.Hq * w.Dqk
    if w.q_dtype == "f32":
        return normals_f32(w.seed, STREAM_Q, 0, n, threads).reshape(shape)
    if w.q_dtype == "bf16":
        return normals_bf16(w.seed, STREAM_Q, 0, n, threads).reshape(shape)
    raise ValueError(w.q_dtype)


def _kv_shape(w: Workload, D: int):
    return (w.B, w.Hkv, w.S_max, D)


def gen_kv_slab(w: Workload, which: str, b: int, h: int, threads=None):
    """(data, scale) of one (request, KV head) slab of K or V, shaped [S_max, ...]."""
    stream = STREAM_K if which == "k" else STREAM_V
    D = w.Dqk if which == "k" else w.Dv
    slab = b * w.Hkv + h
    S = w.S_max
    if w.kv_dtype == "f32":
        return normals_f32(w.seed, stream, slab * S * D, S * D, threads).reshape(S, D), None
    if w.kv_dtype == "bf16":
        return normals_bf16(w.seed, stream, slab * S * D, S * D, threads).reshape(S, D), None
    if w.kv_dtype == "fp8":
        codes, sc = fp8_slabs(w.seed, stream, slab, 1, S * D, threads)
        return codes.reshape(S, D), sc.reshape(())
    if w.kv_dtype == "mxfp4":
        data, sc = mxfp4_rows(w.seed, stream, slab * S, S, D, threads)
        return data.reshape(S, D // 2), sc.reshape(S, D // 32)
    raise ValueError(w.kv_dtype)


def gen_kv(w: Workload, which: str, threads=None, out_data=None, out_scale=None):
    """(data, scale) of the whole K or V cache in the library layout."""
    stream = STREAM_K if which == "k" else STREAM_V
    D = w.Dqk if which == "k" else w.Dv
    nslab = w.B * w.Hkv
    S = w.S_max
    if w.kv_dtype == "f32":
        d = normals_f32(w.seed, stream, 0, nslab * S * D, threads, out=out_data)
        return d.reshape(_kv_shape(w, D)), None
    if w.kv_dtype == "bf16":
        d = normals_bf16(w.seed, stream, 0, nslab * S * D, threads, out=out_data)
        return d.reshape(_kv_shape(w, D)), None
    if w.kv_dtype == "fp8":
        c, s = fp8_slabs(w.seed, stream, 0, nslab, S * D, threads, out=out_data, out_scale=out_scale)
        return c.reshape(_kv_shape(w, D)), s.reshape(w.B, w.Hkv)
    if w.kv_dtype == "mxfp4":
        d, s = mxfp4_rows(w.seed, stream, 0, nslab * S, D, threads, out=out_data, out_scale=out_scale)
        return d.reshape(w.B, w.Hkv, S, D // 2), s.reshape(w.B, w.Hkv, S, D // 32)
    raise ValueError(w.kv_dtype)


def make_inputs(w: Workload, threads=None) -> Inputs:
    q = gen_q(w, threads)
    kd, ks = gen_kv(w, "k", threads)
    if w.v_aliases_k:
        vd, vs = None, None
    else:
        vd, vs = gen_kv(w, "v", threads)
    return Inputs(w, q, kd, ks, vd, vs, gen_seq_lens(w))


# Bit patterns that decode to NaN in each cache format (E2M1 has no NaN, so the
# MXFP4 block exponent 0xFF, which is NaN in E8M0, is used instead).
NAN_PATTERN = {"f32": np.uint32(0x7FC00000), "bf16": np.uint16(0x7FC0), "fp8": np.uint8(0x7F)}


def poison_tail(inp: Inputs) -> Inputs:
    """Overwrite every cached token at or beyond seq_lens[b] with NaN codes.

    A kernel that reads a token past a request's length then produces NaN,
    which the parity tests see.
    """
    w = inp.workload
    for arr_name, sc_name in (("k_data", "k_scale"), ("v_data", "v_scale")):
        arr = getattr(inp, arr_name)
        if arr is None:
            continue
        sc = getattr(inp, sc_name)
        for b in range(w.B):
            L = int(inp.seq_lens[b])
            if w.kv_dtype == "f32":
                arr.view(np.uint32)[b, :, L:, :] = NAN_PATTERN["f32"]
            elif w.kv_dtype == "bf16":
                arr[b, :, L:, :] = NAN_PATTERN["bf16"]
            elif w.kv_dtype == "fp8":
                arr[b, :, L:, :] = NAN_PATTERN["fp8"]
            else:
                sc[b, :, L:, :] = 0xFF
    return inp
