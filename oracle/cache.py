"""Float64 CPU oracle for the growing KV cache: shard layouts, the encoding
of a new token, and decode over a sharded cache.

TEST INFRASTRUCTURE ONLY, like oracle.py: only ``tests/``,
``__graft_entry__.smoke()`` and bench.py's ``cpu_baseline`` leg may use it.
It shares no code with the GPU library.

Shard layouts (which shard stores global token position i of a request, and
at which local row):

* ``contiguous``: one cache [B,Hkv,S_max,D]; token i is row i; shards are cut
  at decode time by the split rule of oracle.split_ranges.
* ``striped``: token i belongs to shard i mod KVP and is that shard's
  (i div KVP)-th token (the inference-parallelism survey, sequence layouts
  section, "Striped": rank = position mod CP, each rank storing its tokens
  compactly).
* ``staggered16``: tokens are dealt to shards in runs of 16: token i belongs
  to shard (i div 16) mod KVP, and is that shard's
  16 * (i div (16 KVP)) + (i mod 16)-th token (the Helix article, section
  "Then reconfigure the same GPUs", staggered KV concatenation: new tokens go
  to one KV-parallel rank for 16 decode steps, then to the next, round-robin).

* ``paged``: a pool of blocks [num_blocks,Hkv,block_len,D]; the cache dict
  carries "block_table" [B,max_blocks] and "block_len", and token i of
  request b is row i mod block_len of block block_table[b, i div block_len]
  (the "Attention DP" design note, section "KV Cache": a per-rank block
  cache [num_blocks, kv heads, block_len, head dim]; the block table that
  lists a request's blocks in order is the usual companion of such a pool).
  Shards are cut by the split rule over positions, as for ``contiguous``.

A sharded cache is [KVP,B,Hkv,S_shard,D] (MXFP4 scales
[KVP,B,Hkv,S_shard,D/32]); shard j of request b holds its tokens, in
increasing position, at rows 0 .. L_j - 1.  Decode results do not depend on
the layout: a single new query attends to every cached token, and the merge
is exact.

Encoding a new token (the readings of the cache formats used by the
generator, written here from the format definitions):

* bf16: the fp32 value rounded to nearest, ties to even mantissa.
* fp8 E4M3 (OCP "fn"): y = x / scale computed in fp32 (one fp32 scale per
  (request, KV head), already set for the slab), then the E4M3 code nearest to
  y, ties to the even code, saturated to +-448.
* MXFP4 (OCP MX): per block of 32 elements, E = clamp(floor(log2(amax)) - 2
  + 127, 0, 254) (127 for an all-zero block); each element x * 2^(127 - E)
  goes to the nearest E2M1 value, ties to even, saturated to +-6.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence, Tuple

import numpy as np

from .oracle import E2M1_TABLE, E4M3_TABLE, Problem, attend, q_to_f64, slab_kv, split_ranges

LAYOUTS = ("contiguous", "striped", "staggered16")      # by position alone
PAGED = "paged"
RUN = 16  # tokens per run of the staggered layout


# ------------------------------------------------------------ shard maps


def owner(i: int, kvp: int, layout: str) -> Tuple[int, int]:
    """(shard, local row) of global token position i in a sharded layout."""
    if layout == "striped":
        return i % kvp, i // kvp
    if layout == "staggered16":
        return (i // RUN) % kvp, RUN * (i // (RUN * kvp)) + i % RUN
    raise ValueError("owner() is defined for the sharded layouts only")


def shard_tokens(L: int, kvp: int, layout: str) -> list:
    """Global positions held by each shard, in local-row order."""
    if layout == "contiguous":
        return [np.arange(s, e) for s, e in split_ranges(L, kvp)]
    out = [[] for _ in range(kvp)]
    for i in range(L):
        j, r = owner(i, kvp, layout)
        assert r == len(out[j])
        out[j].append(i)
    return [np.array(t, dtype=np.int64) for t in out]


def shard_lengths(L: int, kvp: int, layout: str) -> np.ndarray:
    return np.array([len(t) for t in shard_tokens(L, kvp, layout)], dtype=np.int64)


# ---------------------------------------------------------------- encoders


def _nearest_code(a: np.ndarray, values: np.ndarray, codes: np.ndarray) -> np.ndarray:
    """Code of the table value nearest to each a >= 0 (values ascending), ties
    to the even code; a above the largest value saturates to it."""
    a = np.asarray(a, dtype=np.float64)
    idx = np.searchsorted(values, a, side="left")           # values[idx-1] < a <= values[idx]
    hi = np.clip(idx, 0, len(values) - 1)
    lo = np.clip(idx - 1, 0, len(values) - 1)
    dlo = a - values[lo]
    dhi = values[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (codes[hi] % 2 == 0))
    out = np.where(pick_hi, codes[hi], codes[lo])
    out = np.where(a >= values[-1], codes[-1], out)
    return out.astype(np.uint8)


def _positive_table(table: np.ndarray, sign_bit: int):
    codes = np.array([c for c in range(sign_bit) if np.isfinite(table[c])], dtype=np.int64)
    vals = table[codes]
    order = np.argsort(vals, kind="stable")
    vals, codes = vals[order], codes[order]
    keep = np.concatenate([[True], np.diff(vals) > 0])       # +0 only once
    return vals[keep], codes[keep]


_E4M3_POS = _positive_table(E4M3_TABLE, 0x80)
_E2M1_POS = _positive_table(E2M1_TABLE, 0x8)


def encode_e4m3(y_f32: np.ndarray) -> np.ndarray:
    """E4M3 codes of fp32 values (already divided by the slab scale)."""
    y = np.asarray(y_f32, dtype=np.float32).astype(np.float64)
    mag = _nearest_code(np.abs(y), *_E4M3_POS)
    return (mag | np.where(np.signbit(y), 0x80, 0)).astype(np.uint8)


def encode_e2m1(y: np.ndarray) -> np.ndarray:
    """E2M1 nibbles of float64 values (already scaled by the block scale)."""
    y = np.asarray(y, dtype=np.float64)
    mag = _nearest_code(np.abs(y), *_E2M1_POS)
    return (mag | np.where(np.signbit(y), 0x8, 0)).astype(np.uint8)


def encode_bf16(x_f32: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) of fp32 values, nearest with ties to even."""
    x = np.asarray(x_f32, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    lo = bits & 0xFFFF0000
    hi = lo + 0x10000
    xv = x.astype(np.float64)
    vlo = (lo.astype(np.uint32)).view(np.float32).astype(np.float64)
    vhi = (hi.astype(np.uint32)).view(np.float32).astype(np.float64)
    dlo, dhi = np.abs(xv - vlo), np.abs(vhi - xv)
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (((lo >> 16) & 1) == 1))
    out = np.where(pick_hi, hi, lo) >> 16
    return out.astype(np.uint16)


def encode_fp8(x_f32: np.ndarray, scale: float) -> np.ndarray:
    y = np.asarray(x_f32, dtype=np.float32) / np.float32(scale)     # fp32 division
    return encode_e4m3(y)


def mxfp4_block_exponent(block_f32: np.ndarray) -> int:
    amax = float(np.max(np.abs(np.asarray(block_f32, dtype=np.float64))))
    if amax == 0.0:
        return 127
    fl = math.floor(math.log2(amax))
    # log2 of a float64 near a power of two is exact enough here: correct it
    if 2.0 ** fl > amax:
        fl -= 1
    elif 2.0 ** (fl + 1) <= amax:
        fl += 1
    return min(254, max(0, fl - 2 + 127))


def encode_mxfp4_row(x_f32: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """(D/2 packed bytes, D/32 E8M0 exponents) of one row of D fp32 values;
    element 2i in the low nibble of byte i."""
    x = np.asarray(x_f32, dtype=np.float32).astype(np.float64)
    D = x.shape[0]
    assert D % 32 == 0
    scales = np.empty(D // 32, dtype=np.uint8)
    nib = np.empty(D, dtype=np.uint8)
    for blk in range(D // 32):
        xb = x[32 * blk:32 * (blk + 1)]
        E = mxfp4_block_exponent(xb)
        scales[blk] = E
        nib[32 * blk:32 * (blk + 1)] = encode_e2m1(xb * 2.0 ** (127 - E))
    data = (nib[0::2] | (nib[1::2] << 4)).astype(np.uint8)
    return data, scales


def encode_row(kv_dtype: str, x_f32: np.ndarray, fp8_scale: Optional[float] = None):
    """Encoded (data, per-row scales or None) of one cache row."""
    if kv_dtype == "f32":
        return np.asarray(x_f32, dtype=np.float32).copy(), None
    if kv_dtype == "bf16":
        return encode_bf16(x_f32), None
    if kv_dtype == "fp8":
        return encode_fp8(x_f32, fp8_scale), None
    if kv_dtype == "mxfp4":
        return encode_mxfp4_row(x_f32)
    raise ValueError(kv_dtype)


# --------------------------------------------------- appending a token


def append(p: Problem, layout: str, kvp: int, cache: dict, positions: Sequence[int],
           k_new: np.ndarray, v_new: Optional[np.ndarray]) -> None:
    """Encode token rows k_new/v_new [B,Hkv,D] (fp32) and store them at global
    position positions[b] of each request, in place; a negative position, or
    one whose row falls outside the cache, is skipped.

    cache: {"k": data, "k_scale": scales or None, "v": ..., "v_scale": ...}
    laid out per `layout` (contiguous [B,Hkv,S_max,...]; sharded
    [kvp,B,Hkv,S_shard,...]).  fp8 slab scales are read, not changed.
    """
    for b in range(p.B):
        i = int(positions[b])
        for kvh in range(p.Hkv):
            for name, x, D in (("k", k_new, p.Dqk), ("v", v_new, p.Dv)):
                if name == "v" and p.v_aliases_k:
                    continue
                data, sc = cache[name], cache[name + "_scale"]
                fscale = float(sc[b, kvh]) if p.kv_dtype == "fp8" else None
                row, rsc = encode_row(p.kv_dtype, x[b, kvh, :D], fscale)
                if i < 0:
                    continue                      # positions outside the cache are skipped
                if layout == PAGED:
                    bl, table = cache["block_len"], cache["block_table"]
                    if i >= table.shape[1] * bl:
                        continue
                    pb = int(table[b, i // bl])
                    if pb < 0 or pb >= data.shape[0]:
                        continue
                    data[pb, kvh, i % bl] = row
                    if p.kv_dtype == "mxfp4":
                        sc[pb, kvh, i % bl] = rsc
                    continue
                if layout == "contiguous":
                    idx = (b, kvh, i)
                    cap = data.shape[2]
                else:
                    j, r = owner(i, kvp, layout)
                    idx = (j, b, kvh, r)
                    cap = data.shape[3]
                if idx[-1] >= cap:
                    continue
                data[idx] = row
                if p.kv_dtype == "mxfp4":
                    sc[idx] = rsc


# ------------------------------------------------------ decode, any layout


def gather_contiguous(p: Problem, layout: str, kvp: int, cache: dict, seq_lens) -> dict:
    """The same tokens as a contiguous cache [B,Hkv,S,...] in global order
    (S = max length), for the plain definition."""
    if layout == "contiguous":
        return cache
    S = max(1, int(max(seq_lens)))
    if layout == PAGED:
        bl, table = cache["block_len"], cache["block_table"]
        out = {}
        for name in ("k", "k_scale", "v", "v_scale"):
            a = cache.get(name)
            if a is None or (name.endswith("scale") and p.kv_dtype != "mxfp4"):
                out[name] = a
                continue
            g = np.zeros((p.B, p.Hkv, S) + a.shape[3:], dtype=a.dtype)
            for b in range(p.B):
                for i in range(int(seq_lens[b])):
                    g[b, :, i] = a[int(table[b, i // bl]), :, i % bl]
            out[name] = g
        return out
    out = {}
    for name in ("k", "k_scale", "v", "v_scale"):
        a = cache.get(name)
        if a is None or (name.endswith("scale") and p.kv_dtype != "mxfp4"):
            out[name] = a
            continue
        g = np.zeros((p.B, p.Hkv, S) + a.shape[4:], dtype=a.dtype)
        for b in range(p.B):
            for j, toks in enumerate(shard_tokens(int(seq_lens[b]), kvp, layout)):
                for kvh in range(p.Hkv):
                    g[b, kvh, toks] = a[j, b, kvh, :len(toks)]
        out[name] = g
    return out


def decode_layout(p: Problem, layout: str, kvp: int, q, cache: dict, seq_lens, pairs=None):
    """Full-context o [B,Hq,Dv], lse [B,Hq]: the plain definition over the
    request's tokens, whichever shard stores them."""
    from .oracle import decode
    c = gather_contiguous(p, layout, kvp, cache, seq_lens)
    S = c["k"].shape[2]
    pc = Problem(p.B, p.Hq, p.Hkv, p.Dqk, p.Dv, S, p.q_dtype, p.kv_dtype, p.v_aliases_k, p.sm_scale)
    return decode(pc, q, c["k"], c["k_scale"], c["v"], c["v_scale"], seq_lens, pairs)


def decode_partials_layout(p: Problem, layout: str, kvp: int, q, cache: dict, seq_lens, pairs=None):
    """Shard partials o_part [kvp,B,Hq,Dv], lse_part [kvp,B,Hq]: partial j is
    attention over the tokens shard j holds."""
    from .oracle import decode_partials
    if layout in ("contiguous", PAGED):
        c = gather_contiguous(p, layout, kvp, cache, seq_lens)
        pc = Problem(p.B, p.Hq, p.Hkv, p.Dqk, p.Dv, c["k"].shape[2], p.q_dtype, p.kv_dtype, p.v_aliases_k,
                     p.sm_scale)
        return decode_partials(pc, kvp, q, c["k"], c["k_scale"], c["v"], c["v_scale"], seq_lens, pairs)
    qf = q_to_f64(q, p.q_dtype)
    o = np.full((kvp, p.B, p.Hq, p.Dv), np.nan)
    lse = np.full((kvp, p.B, p.Hq), np.nan)
    todo = pairs if pairs is not None else [(b, h) for b in range(p.B) for h in range(p.Hkv)]
    for b, kvh in todo:
        lens = shard_lengths(int(seq_lens[b]), kvp, layout)
        heads = slice(kvh * p.G, (kvh + 1) * p.G)
        for j in range(kvp):
            sub = {n: (None if cache.get(n) is None else
                       (cache[n] if (n.endswith("scale") and p.kv_dtype != "mxfp4") else cache[n][j]))
                   for n in ("k", "k_scale", "v", "v_scale")}
            k, v = slab_kv(p, sub["k"], sub["k_scale"], sub["v"], sub["v_scale"], b, kvh, 0, int(lens[j]))
            o[j, b, heads], lse[j, b, heads] = attend(qf[b, heads], k, v, p.sm_scale)
    return o, lse
