"""Plant plausible mistakes in the cache oracle (on the CPU) and check that
one of its pins (tests/test_oracle_cache.py) catches each.

(Dividing by the fp8 slab scale through its fp32 reciprocal is not among
them: it changes the fp32 quotient by an ulp in about half the cases, but on
a million generated values it never moves an E4M3 code, so no output can
tell the two apart.)"""
import numpy as np
import pytest

import oracle.cache as oc
from tests import test_oracle_cache as pins

_REAL_E4M3 = oc.encode_e4m3
_REAL = {n: getattr(oc, n) for n in ("owner", "_nearest_code", "encode_bf16", "mxfp4_block_exponent",
                                     "encode_fp8", "encode_mxfp4_row", "decode_partials_layout",
                                     "gather_contiguous")}


def _owner_staggered_local_wrong(i, kvp, layout):
    j, r = _REAL["owner"](i, kvp, layout)
    return (j, i // kvp) if layout == "staggered16" else (j, r)


def _owner_striped_shard_wrong(i, kvp, layout):
    return ((i // kvp) % kvp, i // kvp) if layout == "striped" else _REAL["owner"](i, kvp, layout)


def _nearest_ties_up(a, values, codes):
    a = np.asarray(a, dtype=np.float64)
    idx = np.searchsorted(values, a, side="left")
    hi = np.clip(idx, 0, len(values) - 1)
    lo = np.clip(idx - 1, 0, len(values) - 1)
    out = np.where(values[hi] - a <= a - values[lo], codes[hi], codes[lo])
    return np.where(a >= values[-1], codes[-1], out).astype(np.uint8)


def _bf16_truncate(x):
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _mx_exponent_off_by_one(block):
    e = _REAL["mxfp4_block_exponent"](block)
    return e if e in (0, 127) and not np.any(block) else min(254, e + 1)


def _fp8_scale_ignored(x, scale):
    return oc.encode_e4m3(np.asarray(x, dtype=np.float32))


def _e4m3_overflow_to_nan(y):
    codes = _REAL_E4M3(y)
    big = np.abs(np.asarray(y, dtype=np.float32)) >= 448.0
    return np.where(big, codes | 0x7F, codes).astype(np.uint8)


def _mx_nibbles_swapped(x):
    d, s = _REAL["encode_mxfp4_row"](x)
    return (((d & 0x0F) << 4) | (d >> 4)).astype(np.uint8), s


def _partials_rotated(p, layout, kvp, q, cache, seq_lens, pairs=None):
    o, l = _REAL["decode_partials_layout"](p, layout, kvp, q, cache, seq_lens, pairs)
    if layout == "contiguous":
        return o, l
    return np.roll(o, 1, axis=0), np.roll(l, 1, axis=0)


def _gather_paged_row_block_swapped(p, layout, kvp, cache, seq_lens):
    if layout != "paged":
        return _REAL["gather_contiguous"](p, layout, kvp, cache, seq_lens)
    c = dict(cache)
    bl, table = cache["block_len"], cache["block_table"]
    S = max(1, int(max(seq_lens)))
    for name in ("k", "v"):
        a = cache[name]
        g = np.zeros((p.B, p.Hkv, S) + a.shape[3:], dtype=a.dtype)
        for b in range(p.B):
            for i in range(int(seq_lens[b])):
                g[b, :, i] = a[int(table[b, i % table.shape[1]]), :, (i // table.shape[1]) % bl]
        c[name] = g
    for name in ("k_scale", "v_scale"):
        c[name] = _REAL["gather_contiguous"](p, layout, kvp, cache, seq_lens)[name]
    return c


MUTATIONS = {
    "staggered: local row i div kvp": ("owner", _owner_staggered_local_wrong),
    "striped: shard (i div kvp) mod kvp": ("owner", _owner_striped_shard_wrong),
    "encoders: ties rounded up": ("_nearest_code", _nearest_ties_up),
    "bf16: truncation": ("encode_bf16", _bf16_truncate),
    "mxfp4: block exponent one too large": ("mxfp4_block_exponent", _mx_exponent_off_by_one),
    "fp8: slab scale ignored": ("encode_fp8", _fp8_scale_ignored),
    "fp8: overflow encodes NaN instead of saturating": ("encode_e4m3", _e4m3_overflow_to_nan),
    "mxfp4: nibbles swapped": ("encode_mxfp4_row", _mx_nibbles_swapped),
    "partials: shard outputs rotated": ("decode_partials_layout", _partials_rotated),
    "paged: block and row indices interleaved": ("gather_contiguous", _gather_paged_row_block_swapped),
}


def _pin_calls():
    calls = []
    for name in dir(pins):
        fn = getattr(pins, name)
        if not name.startswith("test_") or not callable(fn):
            continue
        marks = getattr(fn, "pytestmark", [])
        grids = [m.args for m in marks if m.name == "parametrize"]
        combos = [{}]
        for argnames, values in grids:
            names = [a.strip() for a in argnames.split(",")]
            combos = [dict(c, **dict(zip(names, v if len(names) > 1 else (v,)))) for c in combos for v in values]
        calls += [(name, fn, c) for c in combos]
    return calls


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    attr, bad = MUTATIONS[name]
    monkeypatch.setattr(oc, attr, bad)
    caught = []
    for pname, fn, kw in _pin_calls():
        try:
            with np.errstate(all="ignore"):
                fn(**kw)
        except Exception:  # noqa: BLE001 - any failure counts as caught
            caught.append(pname)
    assert caught, "no pin caught mutation %r" % name
