"""Plant plausible mistakes in the oracle (on the CPU) and check a pin catches each.

Every mutation below replaces one oracle function with a subtly wrong copy; the
test passes only if at least one pin then raises.  This is what makes the pins
a check of the oracle rather than a restatement of it.
"""
import math

import numpy as np
import pytest

import oracle.oracle as ora
from tests import oracle_pins


def _attend_no_scale(q, k, v, sm_scale):
    return _REAL["attend"](q, k, v, 1.0)


def _attend_uses_k_as_v(q, k, v, sm_scale):
    if k.shape[1] == v.shape[1]:
        return _REAL["attend"](q, k, k, sm_scale)
    return _REAL["attend"](q, k, v, sm_scale)


def _attend_lse_without_max(q, k, v, sm_scale):
    o, lse = _REAL["attend"](q, k, v, sm_scale)
    if k.shape[0] == 0:
        return o, lse
    x = sm_scale * (np.asarray(q) @ k.T)
    return o, lse - x.max(axis=1)


def _attend_no_max_shift(q, k, v, sm_scale):
    q = np.asarray(q, dtype=np.float64)
    if k.shape[0] == 0:
        return np.zeros((q.shape[0], v.shape[1])), np.full(q.shape[0], -np.inf)
    with np.errstate(over="ignore", invalid="ignore"):
        x = sm_scale * (q @ k.T)
        w = np.exp(x)
        l = w.sum(axis=1)
        return (w @ v) / l[:, None], np.log(l)


def _attend_drops_last_token(q, k, v, sm_scale):
    if k.shape[0] > 1:
        return _REAL["attend"](q, k[:-1], v[:-1], sm_scale)
    return _REAL["attend"](q, k, v, sm_scale)


def _merge_unnormalized(o_parts, lse_parts):
    o, lse = _REAL["merge"](o_parts, lse_parts)
    M = np.max(lse_parts, axis=0)
    w = np.where(np.isfinite(lse_parts), np.exp(lse_parts - np.where(np.isfinite(M), M, 0)), 0)
    return (w[..., None] * o_parts).sum(axis=0), lse


def _merge_plain_average(o_parts, lse_parts):
    o, lse = _REAL["merge"](o_parts, lse_parts)
    return np.asarray(o_parts).mean(axis=0), lse


def _split_no_rounding(L, kvp):
    if L <= 0:
        return [(0, 0)] * kvp
    C = -(-L // kvp)
    return [(j * C, min(L, (j + 1) * C)) if j * C < L else (L, L) for j in range(kvp)]


def _dequant_nibbles_swapped(kv_dtype, data, scale, D):
    if kv_dtype == "mxfp4":
        raw = np.asarray(data, dtype=np.uint8)
        swapped = ((raw & 0x0F) << 4) | (raw >> 4)
        return _REAL["dequant"](kv_dtype, swapped.astype(np.uint8), scale, D)
    return _REAL["dequant"](kv_dtype, data, scale, D)


def _dequant_fp8_ignores_scale(kv_dtype, data, scale, D):
    if kv_dtype == "fp8":
        return _REAL["dequant"](kv_dtype, data, np.float32(1.0), D)
    return _REAL["dequant"](kv_dtype, data, scale, D)


def _decode_gqa_modulo(p, q, k_data, k_scale, v_data, v_scale, seq_lens, pairs=None):
    qf = ora.q_to_f64(q, p.q_dtype)
    o = np.full((p.B, p.Hq, p.Dv), np.nan)
    lse = np.full((p.B, p.Hq), np.nan)
    for b in range(p.B):
        for h in range(p.Hq):
            kvh = h % p.Hkv
            k, v = ora.slab_kv(p, k_data, k_scale, v_data, v_scale, b, kvh, 0, int(seq_lens[b]))
            oo, ll = ora.attend(qf[b, h:h + 1], k, v, p.sm_scale)
            o[b, h], lse[b, h] = oo[0], ll[0]
    return o, lse


def _partials_shifted(p, kvp, q, k_data, k_scale, v_data, v_scale, seq_lens, pairs=None):
    real = _REAL["split_ranges"]
    try:
        ora.split_ranges = lambda L, n: [(max(0, s - 1), e) for (s, e) in real(L, n)]
        return _REAL["decode_partials"](p, kvp, q, k_data, k_scale, v_data, v_scale, seq_lens, pairs)
    finally:
        ora.split_ranges = real


def _e4m3_bias8():
    def val(code):
        s = -1.0 if code & 0x80 else 1.0
        e, m = (code >> 3) & 0xF, code & 7
        if e == 0xF and m == 7:
            return math.nan
        if e == 0:
            return s * (m / 8.0) * 2.0 ** (1 - 8)
        return s * (1 + m / 8.0) * 2.0 ** (e - 8)
    return np.array([val(c) for c in range(256)])


def _e2m1_no_subnormal():
    t = ora.E2M1_TABLE.copy()
    t[1], t[9] = 0.0, -0.0
    return t


_REAL = {n: getattr(ora, n) for n in ("attend", "merge", "split_ranges", "dequant", "decode",
                                      "decode_partials")}

MUTATIONS = {
    "attend: logits not scaled": ("attend", _attend_no_scale),
    "attend: K used in place of V": ("attend", _attend_uses_k_as_v),
    "attend: lse missing the max": ("attend", _attend_lse_without_max),
    "attend: no max shift (overflow)": ("attend", _attend_no_max_shift),
    "attend: last token dropped": ("attend", _attend_drops_last_token),
    "merge: weights not normalized": ("merge", _merge_unnormalized),
    "merge: plain average of shards": ("merge", _merge_plain_average),
    "split: not rounded to 16 tokens": ("split_ranges", _split_no_rounding),
    "dequant: MXFP4 nibbles swapped": ("dequant", _dequant_nibbles_swapped),
    "dequant: fp8 scale ignored": ("dequant", _dequant_fp8_ignores_scale),
    "decode: head h reads KV head h mod Hkv": ("decode", _decode_gqa_modulo),
    "decode_partials: shard starts one token early": ("decode_partials", _partials_shifted),
    "table: E4M3 bias 8": ("E4M3_TABLE", _e4m3_bias8()),
    "table: E2M1 subnormal flushed": ("E2M1_TABLE", _e2m1_no_subnormal()),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    attr, bad = MUTATIONS[name]
    monkeypatch.setattr(ora, attr, bad)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(ora)
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            caught.append(pin.__name__)
    assert caught, "no pin caught mutation %r" % name
