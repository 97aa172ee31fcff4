"""Float64 CPU oracle for exact split-KV decode attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the GPU
library (kernels, host code, tables or helpers); it reads the same encoded
input bytes, which come from the separate ``kvgen`` generator.

What is computed (the plain definition, in float64, no online softmax):

* One new query token per request attends to all of that request's cached
  tokens.  Per query head h of request b, with KV head kvh = floor(h / G)
  (G = Hq / Hkv consecutive query heads share one KV head: the GQA grouping
  described in the Helix article, "The ceiling, in algebra", and in the
  inference-parallelism survey's tensor-parallel attention section), and L =
  seq_len[b]:

      x_s = sm_scale * sum_d q[b,h,d] * k[b,kvh,s,d]        s = 0 .. L-1
      m   = max_s x_s
      l   = sum_s exp(x_s - m)
      o   = sum_s exp(x_s - m) * v[b,kvh,s,:] / l
      lse = m + ln l

  with sm_scale = 1/sqrt(Dqk) unless given.  This is softmax(q K^T / sqrt(d)) V
  for a single query row.

* Shards (split-KV / KV parallelism): the sequence of each request is cut
  into KVP contiguous pieces and each piece yields a normalized partial output
  and the log-sum-exp of its own logits (Helix article, "Sharding the sequence
  instead": every KV-parallel rank returns a partial attention output plus one
  log-sum-exp value per token).  Shard j of a request with L tokens covers
  [j*C, min(L, (j+1)*C)) with C = roundup(ceil(L / KVP), 16); a shard that
  starts at or past L is empty and yields o = 0, lse = -inf.

* Merge (Helix article, "Sharding the sequence instead", the per-token merge
  sketch; Context Parallelism knowledge note, "Pass-KV keeps queries local
  and circulates keys and values", the exact merge equation): with M the
  largest shard lse, each shard is weighted by exp(lse_j - M); the merged
  output is the weighted sum of the shard outputs divided by the sum of the
  weights, and the merged lse is M + ln(sum of weights).

Cache formats (decoded exactly: every code and scale is exact in float64):

* bf16: the upper 16 bits of an IEEE fp32.
* fp8 E4M3 ("fn" variant of the OCP 8-bit floating point spec): bias 7, 3
  mantissa bits, subnormals, no infinities, S.1111.111 is NaN; one fp32 scale
  per (request, KV head) multiplies every code of that slab.
* MXFP4 (OCP Microscaling spec): E2M1 elements (bias 1, 1 mantissa bit, no
  inf/NaN) packed two per byte, element 2i in bits [3:0] of byte i; every
  32 contiguous elements of a row share one E8M0 scale 2^(E-127) (E = 255 is
  NaN).

Parity: pinned by tests/test_oracle.py against brute force, closed forms,
invariances, library decoders and format fixtures.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence, Tuple

import numpy as np

# ------------------------------------------------------------------ formats


def e4m3_value(code: int) -> float:
    """Value of one OCP E4M3 ("fn") byte."""
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return s * (m / 8.0) * 2.0 ** (1 - 7)
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def e2m1_value(nibble: int) -> float:
    """Value of one OCP E2M1 nibble."""
    s = -1.0 if nibble & 0x8 else 1.0
    e = (nibble >> 1) & 0x3
    m = nibble & 0x1
    if e == 0:
        return s * (m / 2.0) * 2.0 ** (1 - 1)
    return s * (1.0 + m / 2.0) * 2.0 ** (e - 1)


def e8m0_value(code: int) -> float:
    """Value of one E8M0 scale byte: 2^(code - 127); 255 is NaN."""
    if code == 255:
        return math.nan
    return math.ldexp(1.0, code - 127)


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
E8M0_TABLE = np.array([e8m0_value(c) for c in range(256)], dtype=np.float64)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64 (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def q_to_f64(q: np.ndarray, q_dtype: str) -> np.ndarray:
    if q_dtype == "f32":
        return np.asarray(q, dtype=np.float32).astype(np.float64)
    if q_dtype == "bf16":
        return bf16_to_f64(q)
    raise ValueError(q_dtype)


def dequant(kv_dtype: str, data: np.ndarray, scale, D: int) -> np.ndarray:
    """Decode cache rows to float64.

    data: [..., S, D] elements (MXFP4: [..., S, D/2] bytes); scale: a scalar
    fp32 for fp8 (one slab), [..., S, D/32] E8M0 bytes for MXFP4, else None.
    Returns float64 [..., S, D].
    """
    if kv_dtype == "f32":
        return np.asarray(data, dtype=np.float32).astype(np.float64)
    if kv_dtype == "bf16":
        return bf16_to_f64(data)
    if kv_dtype == "fp8":
        return E4M3_TABLE[np.asarray(data, dtype=np.uint8)] * float(np.float32(scale))
    if kv_dtype == "mxfp4":
        raw = np.asarray(data, dtype=np.uint8)
        lo = raw & 0x0F
        hi = raw >> 4
        nib = np.stack([lo, hi], axis=-1).reshape(raw.shape[:-1] + (raw.shape[-1] * 2,))
        assert nib.shape[-1] == D
        vals = E2M1_TABLE[nib]
        sc = E8M0_TABLE[np.asarray(scale, dtype=np.uint8)]          # [..., S, D/32]
        return vals * np.repeat(sc, 32, axis=-1)
    raise ValueError(kv_dtype)


# ------------------------------------------------------------------- shards


def split_ranges(L: int, kvp: int) -> list:
    """Token range [start, end) of each of the kvp shards of an L-token request."""
    if kvp < 1:
        raise ValueError("kvp must be >= 1")
    if L <= 0:
        return [(0, 0)] * kvp
    per = -(-L // kvp)                 # ceil(L / kvp)
    C = -(-per // 16) * 16             # rounded up to a multiple of 16 tokens
    out = []
    for j in range(kvp):
        s = j * C
        e = min(L, (j + 1) * C)
        out.append((s, e) if s < L else (L, L))
    return out


# ---------------------------------------------------------------- attention


def default_scale(Dqk: int) -> float:
    return 1.0 / math.sqrt(Dqk)


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, sm_scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Attention of G query rows over L cached rows, plain definition.

    q [G, Dqk], k [L, Dqk], v [L, Dv] (float64).  Returns o [G, Dv] and lse [G];
    an empty range (L = 0) gives o = 0 and lse = -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    G = q.shape[0]
    Dv = v.shape[1]
    if k.shape[0] == 0:
        return np.zeros((G, Dv)), np.full(G, -np.inf)
    x = sm_scale * (q @ k.T)                       # [G, L]
    m = x.max(axis=1)
    w = np.exp(x - m[:, None])
    l = w.sum(axis=1)
    o = (w @ v) / l[:, None]
    lse = m + np.log(l)
    return o, lse


def merge(o_parts: np.ndarray, lse_parts: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Exact merge of shard partials.

    o_parts [J, ..., Dv], lse_parts [J, ...] -> o [..., Dv], lse [...].
    Entries whose shards are all empty (every lse = -inf) give o = 0, lse = -inf.
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    M = lse_parts.max(axis=0)
    any_tokens = np.isfinite(M)
    Msafe = np.where(any_tokens, M, 0.0)
    w = np.where(np.isfinite(lse_parts), np.exp(lse_parts - Msafe), 0.0)   # [J, ...]
    den = w.sum(axis=0)
    num = (w[..., None] * o_parts).sum(axis=0)
    with np.errstate(invalid="ignore", divide="ignore"):
        o = np.where(any_tokens[..., None], num / np.where(any_tokens, den, 1.0)[..., None], 0.0)
        lse = np.where(any_tokens, Msafe + np.log(np.where(any_tokens, den, 1.0)), -np.inf)
    return o, lse


# --------------------------------------------------------- whole problems


class Problem:
    """Shapes and formats of one decode step (mirrors the inputs' layouts).

    q [B,Hq,Dqk]; k/v [B,Hkv,S_max,D] (MXFP4: [B,Hkv,S_max,D/2] bytes and
    [B,Hkv,S_max,D/32] scales; fp8: [B,Hkv] fp32 scales); V may alias the first
    Dv columns of K (v_aliases_k).
    """

    def __init__(self, B, Hq, Hkv, Dqk, Dv, S_max, q_dtype, kv_dtype, v_aliases_k=False,
                 sm_scale: Optional[float] = None):
        assert Hq % Hkv == 0
        self.B, self.Hq, self.Hkv, self.Dqk, self.Dv = B, Hq, Hkv, Dqk, Dv
        self.S_max, self.q_dtype, self.kv_dtype = S_max, q_dtype, kv_dtype
        self.v_aliases_k = bool(v_aliases_k)
        self.sm_scale = default_scale(Dqk) if not sm_scale else float(sm_scale)

    @property
    def G(self):
        return self.Hq // self.Hkv

    @classmethod
    def from_workload(cls, w):
        return cls(w.B, w.Hq, w.Hkv, w.Dqk, w.Dv, w.S_max, w.q_dtype, w.kv_dtype, w.v_aliases_k)


def slab_kv(p: Problem, k_data, k_scale, v_data, v_scale, b: int, kvh: int, lo: int, hi: int):
    """Decoded K [hi-lo, Dqk] and V [hi-lo, Dv] rows of one (request, KV head)."""
    def part(data, scale, D):
        d = data[b, kvh, lo:hi]
        if p.kv_dtype == "fp8":
            s = scale[b, kvh]
        elif p.kv_dtype == "mxfp4":
            s = scale[b, kvh, lo:hi]
        else:
            s = None
        return dequant(p.kv_dtype, d, s, D)

    k = part(k_data, k_scale, p.Dqk)
    if p.v_aliases_k:
        v = k[:, :p.Dv]
    else:
        v = part(v_data, v_scale, p.Dv)
    return k, v


def decode(p: Problem, q, k_data, k_scale, v_data, v_scale, seq_lens,
           pairs: Optional[Sequence[Tuple[int, int]]] = None):
    """Full-context o [B,Hq,Dv] and lse [B,Hq] (float64).

    pairs: optional list of (b, kvh) to compute; other entries are NaN.
    """
    qf = q_to_f64(q, p.q_dtype)
    o = np.full((p.B, p.Hq, p.Dv), np.nan)
    lse = np.full((p.B, p.Hq), np.nan)
    todo = pairs if pairs is not None else [(b, h) for b in range(p.B) for h in range(p.Hkv)]
    for b, kvh in todo:
        L = int(seq_lens[b])
        k, v = slab_kv(p, k_data, k_scale, v_data, v_scale, b, kvh, 0, L)
        heads = slice(kvh * p.G, (kvh + 1) * p.G)
        o[b, heads], lse[b, heads] = attend(qf[b, heads], k, v, p.sm_scale)
    return o, lse


def decode_partials(p: Problem, kvp: int, q, k_data, k_scale, v_data, v_scale, seq_lens,
                    pairs: Optional[Sequence[Tuple[int, int]]] = None):
    """Shard partials o_part [kvp,B,Hq,Dv] and lse_part [kvp,B,Hq] (float64)."""
    qf = q_to_f64(q, p.q_dtype)
    o = np.full((kvp, p.B, p.Hq, p.Dv), np.nan)
    lse = np.full((kvp, p.B, p.Hq), np.nan)
    todo = pairs if pairs is not None else [(b, h) for b in range(p.B) for h in range(p.Hkv)]
    for b, kvh in todo:
        L = int(seq_lens[b])
        heads = slice(kvh * p.G, (kvh + 1) * p.G)
        for j, (s, e) in enumerate(split_ranges(L, kvp)):
            k, v = slab_kv(p, k_data, k_scale, v_data, v_scale, b, kvh, s, e)
            o[j, b, heads], lse[j, b, heads] = attend(qf[b, heads], k, v, p.sm_scale)
    return o, lse
