"""Pins for the float64 oracle: checks against things other than the oracle.

Each ``pin_*`` function takes the oracle module and raises AssertionError when
the oracle disagrees with:
  * brute force written separately in pure Python (math.fsum, scalar loops),
  * closed forms of softmax attention,
  * invariances the exact merge guarantees (split invariance, associativity,
    log-sum-exp additivity, token-order invariance),
  * library decoders (torch's float8_e4m3fn, float8_e8m0fnu, bfloat16),
  * format fixtures under tests/golden/ (OCP E2M1 values, MXFP4 byte layout).

tests/test_oracle.py runs them on the real oracle; tests/test_oracle_mutations.py
plants mistakes in the oracle and checks that some pin catches each one.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


# --------------------------------------------------------------- brute force
def brute_attend(q_rows, k_rows, v_rows, scale):
    """Pure-Python softmax attention: lists in, lists out, math.fsum sums."""
    outs, lses = [], []
    for qh in q_rows:
        xs = [scale * math.fsum(float(a) * float(b) for a, b in zip(qh, kr)) for kr in k_rows]
        m = max(xs)
        ws = [math.exp(x - m) for x in xs]
        l = math.fsum(ws)
        o = [math.fsum(w * float(vr[d]) for w, vr in zip(ws, v_rows)) / l for d in range(len(v_rows[0]))]
        outs.append(o)
        lses.append(m + math.log(l))
    return np.array(outs), np.array(lses)


def _close(a, b, rtol=1e-12, atol=1e-12, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    ok = np.isclose(a, b, rtol=rtol, atol=atol) | (np.isneginf(a) & np.isneginf(b))
    assert ok.all(), (what, np.max(np.abs(a - b)))


# ------------------------------------------------------------ attention core
def pin_brute_small(ora):
    rng = _rng(1)
    for L in (1, 2, 3, 7, 16, 33, 64):
        for D, Dv in ((4, 4), (8, 6)):
            for G in (1, 2, 4):
                q = rng.standard_normal((G, D))
                k = rng.standard_normal((L, D))
                v = rng.standard_normal((L, Dv))
                o, lse = ora.attend(q, k, v, ora.default_scale(D))
                bo, bl = brute_attend(q.tolist(), k.tolist(), v.tolist(), 1.0 / math.sqrt(D))
                _close(o, bo, what="o L=%d" % L)
                _close(lse, bl, what="lse L=%d" % L)


def pin_brute_problem(ora):
    """Whole tiny problems through ora.decode vs brute force per head."""
    rng = _rng(2)
    for (B, Hq, Hkv, Dqk, Dv, alias) in ((2, 4, 2, 8, 8, False), (1, 6, 1, 8, 4, True),
                                         (3, 2, 2, 4, 4, False)):
        S = 40
        seq = rng.integers(1, S + 1, size=B)
        q = rng.standard_normal((B, Hq, Dqk)).astype(np.float32)
        k = rng.standard_normal((B, Hkv, S, Dqk)).astype(np.float32)
        v = None if alias else rng.standard_normal((B, Hkv, S, Dv)).astype(np.float32)
        p = ora.Problem(B, Hq, Hkv, Dqk, Dv, S, "f32", "f32", v_aliases_k=alias)
        o, lse = ora.decode(p, q, k, None, v, None, seq)
        G = Hq // Hkv
        for b in range(B):
            for h in range(Hq):
                kv = h // G
                L = int(seq[b])
                kr = k[b, kv, :L].tolist()
                vr = (k[b, kv, :L, :Dv] if alias else v[b, kv, :L]).tolist()
                bo, bl = brute_attend([q[b, h].tolist()], kr, vr, 1.0 / math.sqrt(Dqk))
                _close(o[b, h], bo[0], what="decode o")
                _close(lse[b, h], bl[0], what="decode lse")


def pin_single_token(ora):
    """L = 1: the output is that token's value row and lse is its logit."""
    rng = _rng(3)
    q = rng.standard_normal((3, 5))
    k = rng.standard_normal((1, 5))
    v = rng.standard_normal((1, 7))
    o, lse = ora.attend(q, k, v, 0.5)
    _close(o, np.repeat(v, 3, axis=0), what="L=1 o")
    _close(lse, 0.5 * (q @ k[0]), what="L=1 lse")


def pin_two_tokens(ora):
    """L = 2: o = sigmoid(x0 - x1) v0 + sigmoid(x1 - x0) v1, lse = log(e^x0 + e^x1)."""
    rng = _rng(4)
    q = rng.standard_normal((4, 6))
    k = rng.standard_normal((2, 6))
    v = rng.standard_normal((2, 3))
    s = 1 / math.sqrt(6)
    o, lse = ora.attend(q, k, v, s)
    for g in range(4):
        x0, x1 = s * float(q[g] @ k[0]), s * float(q[g] @ k[1])
        a = 1.0 / (1.0 + math.exp(x1 - x0))
        _close(o[g], a * v[0] + (1 - a) * v[1], what="L=2 o")
        _close(lse[g], max(x0, x1) + math.log1p(math.exp(-abs(x0 - x1))), what="L=2 lse")


def pin_zero_query(ora):
    """q = 0: uniform weights, o = mean of V, lse = ln L."""
    rng = _rng(5)
    for L in (1, 5, 100):
        v = rng.standard_normal((L, 4)) + 3.0
        o, lse = ora.attend(np.zeros((2, 8)), rng.standard_normal((L, 8)), v, 0.3)
        _close(o, np.repeat(v.mean(axis=0)[None], 2, axis=0), what="q=0 o")
        _close(lse, np.full(2, math.log(L)), what="q=0 lse")


def pin_equal_keys(ora):
    """All keys equal: o = mean of V, lse = x + ln L."""
    rng = _rng(6)
    L, D = 37, 8
    krow = rng.standard_normal(D)
    k = np.repeat(krow[None], L, axis=0)
    v = rng.standard_normal((L, 5)) + 2.0
    q = rng.standard_normal((3, D))
    o, lse = ora.attend(q, k, v, 0.25)
    _close(o, np.repeat(v.mean(axis=0)[None], 3, axis=0), what="equal keys o")
    _close(lse, 0.25 * (q @ krow) + math.log(L), what="equal keys lse")


def pin_constant_values(ora):
    """Constant V rows: o equals that constant for any keys."""
    rng = _rng(7)
    c = rng.standard_normal(6)
    v = np.repeat(c[None], 50, axis=0)
    o, _ = ora.attend(rng.standard_normal((4, 8)) * 3, rng.standard_normal((50, 8)) * 3, v, 1.0)
    _close(o, np.repeat(c[None], 4, axis=0), what="constant V")


def pin_permutation(ora):
    """Reordering the cached tokens leaves o and lse unchanged."""
    rng = _rng(8)
    q, k, v = rng.standard_normal((4, 8)), rng.standard_normal((60, 8)), rng.standard_normal((60, 8))
    perm = rng.permutation(60)
    o1, l1 = ora.attend(q, k, v, 0.5)
    o2, l2 = ora.attend(q, k[perm], v[perm], 0.5)
    _close(o1, o2, what="perm o")
    _close(l1, l2, what="perm lse")


def pin_large_logits(ora):
    """Logits of magnitude ~1e3 stay finite and match brute force (max-shifted)."""
    rng = _rng(9)
    q = rng.standard_normal((2, 4)) * 40
    k = rng.standard_normal((20, 4)) * 40
    v = rng.standard_normal((20, 3))
    o, lse = ora.attend(q, k, v, 1.0)
    bo, bl = brute_attend(q.tolist(), k.tolist(), v.tolist(), 1.0)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    _close(o, bo, rtol=1e-10, atol=1e-12, what="large o")
    _close(lse, bl, rtol=1e-12, what="large lse")


def pin_empty_range(ora):
    o, lse = ora.attend(np.ones((2, 4)), np.zeros((0, 4)), np.zeros((0, 3)), 1.0)
    assert o.shape == (2, 3) and (o == 0).all()
    assert np.isneginf(lse).all()


# ------------------------------------------------------------- split + merge
def pin_split_rule(ora):
    """Shards tile [0, L) in order, boundaries on 16-token multiples, sizes <= ceil(L/kvp) rounded up to 16."""
    for L in list(range(0, 70)) + [100, 255, 256, 257, 4096, 65536, 65537, 131072, 1 << 20]:
        for kvp in (1, 2, 3, 4, 7, 8, 16, 32, 128):
            r = ora.split_ranges(L, kvp)
            assert len(r) == kvp
            covered = 0
            C = 16 * math.ceil(math.ceil(L / kvp) / 16) if L > 0 else 0
            for j, (s, e) in enumerate(r):
                assert 0 <= s <= e <= L
                if e > s:
                    assert s == covered, (L, kvp, j)
                    assert s % 16 == 0 and s == j * C
                    assert e - s <= C and (e == L or (e - s) == C)
                    covered = e
                else:
                    assert j * C >= L or L == 0, (L, kvp, j)
            assert covered == L, (L, kvp)


def _parts(ora, q, k, v, scale, ranges):
    os_, ls_ = [], []
    for (s, e) in ranges:
        o, l = ora.attend(q, k[s:e], v[s:e], scale)
        os_.append(o)
        ls_.append(l)
    return np.stack(os_), np.stack(ls_)


def pin_split_invariance(ora):
    """Merging the partials of any partition equals the unsplit result."""
    rng = _rng(10)
    L, D = 300, 8
    q, k, v = rng.standard_normal((4, D)), rng.standard_normal((L, D)), rng.standard_normal((L, 5))
    o_ref, l_ref = ora.attend(q, k, v, 0.35)
    # the library's contiguous rule, several split counts (incl. empty shards)
    for kvp in (1, 2, 3, 16, 128):
        po, pl = _parts(ora, q, k, v, 0.35, ora.split_ranges(L, kvp))
        o, l = ora.merge(po, pl)
        _close(o, o_ref, what="split kvp=%d" % kvp)
        _close(l, l_ref, what="split lse kvp=%d" % kvp)
    # uneven random cut points
    for trial in range(5):
        cuts = np.sort(rng.choice(np.arange(1, L), size=6, replace=False))
        edges = [0] + cuts.tolist() + [L]
        po, pl = _parts(ora, q, k, v, 0.35, list(zip(edges[:-1], edges[1:])))
        o, l = ora.merge(po, pl)
        _close(o, o_ref, what="uneven")
        _close(l, l_ref, what="uneven lse")
    # striped ownership: token i belongs to shard i mod 5 (plus two empty shards)
    os_, ls_ = [], []
    for j in range(7):
        idx = np.arange(j, L, 5) if j < 5 else np.arange(0)
        o, l = ora.attend(q, k[idx], v[idx], 0.35)
        os_.append(o)
        ls_.append(l)
    o, l = ora.merge(np.stack(os_), np.stack(ls_))
    _close(o, o_ref, what="striped")
    _close(l, l_ref, what="striped lse")


def pin_merge_algebra(ora):
    """merge(merge(A,B),C) = merge(A,B,C); exp(lse) = sum_j exp(lse_j); all-empty -> (0, -inf)."""
    rng = _rng(11)
    o = rng.standard_normal((3, 4, 6))
    l = rng.standard_normal((3, 4)) * 3
    oab, lab = ora.merge(o[:2], l[:2])
    o1, l1 = ora.merge(np.stack([oab, o[2]]), np.stack([lab, l[2]]))
    o2, l2 = ora.merge(o, l)
    _close(o1, o2, what="assoc o")
    _close(l1, l2, what="assoc lse")
    _close(np.exp(l2), np.exp(l).sum(axis=0), what="lse additivity")
    oe, le = ora.merge(np.zeros((2, 4, 6)), np.full((2, 4), -np.inf))
    assert (oe == 0).all() and np.isneginf(le).all()
    # one nonempty shard among empties returns it unchanged
    lone = np.full((3, 4), -np.inf)
    lone[1] = l[1]
    om, lm = ora.merge(o, lone)
    _close(om, o[1], what="lone o")
    _close(lm, l[1], what="lone lse")


def pin_partials_problem(ora):
    """decode_partials: each shard equals brute force on its range; merged equals decode."""
    rng = _rng(12)
    B, Hq, Hkv, D, S = 2, 4, 2, 4, 70
    seq = np.array([70, 33], dtype=np.int32)
    q = rng.standard_normal((B, Hq, D)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, S, D)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, S, D)).astype(np.float32)
    p = ora.Problem(B, Hq, Hkv, D, D, S, "f32", "f32")
    for kvp in (1, 3, 4):
        po, pl = ora.decode_partials(p, kvp, q, k, None, v, None, seq)
        assert po.shape == (kvp, B, Hq, D) and pl.shape == (kvp, B, Hq)
        for b in range(B):
            L = int(seq[b])
            C = 16 * math.ceil(math.ceil(L / kvp) / 16)
            for j in range(kvp):
                s, e = j * C, min(L, (j + 1) * C)
                for h in range(Hq):
                    kv = h // (Hq // Hkv)
                    if s >= L:
                        assert (po[j, b, h] == 0).all() and np.isneginf(pl[j, b, h])
                        continue
                    bo, bl = brute_attend([q[b, h].tolist()], k[b, kv, s:e].tolist(),
                                          v[b, kv, s:e].tolist(), 1 / math.sqrt(D))
                    _close(po[j, b, h], bo[0], what="partial o")
                    _close(pl[j, b, h], bl[0], what="partial lse")
        o, l = ora.decode(p, q, k, None, v, None, seq)
        mo, ml = ora.merge(po, pl)
        _close(mo, o, what="merged partials")
        _close(ml, l, what="merged lse")


def pin_gqa_mapping(ora):
    """Query head h reads KV head floor(h / G): give each KV head its own constant V."""
    B, Hq, Hkv, D, S = 1, 8, 4, 4, 9
    rng = _rng(13)
    q = rng.standard_normal((B, Hq, D)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, S, D)).astype(np.float32)
    v = np.zeros((B, Hkv, S, D), dtype=np.float32)
    for h in range(Hkv):
        v[0, h] = 10.0 * (h + 1)
    p = ora.Problem(B, Hq, Hkv, D, D, S, "f32", "f32")
    o, _ = ora.decode(p, q, k, None, v, None, np.array([S], dtype=np.int32))
    for h in range(Hq):
        _close(o[0, h], np.full(D, 10.0 * (h // 2 + 1)), what="gqa head %d" % h)


# ------------------------------------------------------------------- formats
def pin_e4m3_torch(ora):
    import torch
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    tab = np.asarray(ora.E4M3_TABLE)
    assert (np.isnan(ref) == np.isnan(tab)).all()
    m = ~np.isnan(ref)
    assert np.array_equal(ref[m], tab[m])


def pin_e4m3_spec(ora):
    """OCP 8-bit FP spec values: max normal 448 (0x7E), min normal 2^-6 (0x08),
    max subnormal 0.875 * 2^-6 (0x07), min subnormal 2^-9 (0x01), NaN only at 0x7F/0xFF."""
    with open(os.path.join(GOLDEN, "ocp_e4m3_values.json")) as f:
        fx = json.load(f)
    for code_hex, val in fx["values"].items():
        assert ora.E4M3_TABLE[int(code_hex, 16)] == float(val), code_hex
    nan_codes = [c for c in range(256) if math.isnan(ora.E4M3_TABLE[c])]
    assert nan_codes == [int(c, 16) for c in fx["nan_codes"]]


def pin_e8m0_torch(ora):
    import torch
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    tab = np.asarray(ora.E8M0_TABLE)
    assert np.isnan(tab[255]) and np.isnan(ref[255])
    assert np.array_equal(ref[:255], tab[:255])


def pin_e2m1_spec(ora):
    with open(os.path.join(GOLDEN, "ocp_e2m1_values.json")) as f:
        fx = json.load(f)
    for code, val in enumerate(fx["values"]):
        assert ora.E2M1_TABLE[code] == float(val), code


def pin_bf16_torch(ora):
    import torch
    rng = _rng(14)
    bits = rng.integers(0, 1 << 16, size=4096, dtype=np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]          # finite values only
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ora.bf16_to_f64(bits), ref)


def pin_mxfp4_layout(ora):
    """Hand-built MXFP4 rows (tests/golden/mxfp4_layout.json) decode to the listed values."""
    with open(os.path.join(GOLDEN, "mxfp4_layout.json")) as f:
        fx = json.load(f)
    for case in fx["cases"]:
        data = np.array(case["bytes"], dtype=np.uint8).reshape(1, -1)
        scale = np.array(case["scales"], dtype=np.uint8).reshape(1, -1)
        got = ora.dequant("mxfp4", data, scale, data.shape[1] * 2)[0]
        exp = np.array(case["values"], dtype=np.float64)
        assert np.array_equal(got, exp), case["name"]


def pin_fp8_scale(ora):
    """fp8 slab: value = E4M3(code) * fp32 scale, exactly."""
    codes = np.array([[0x38, 0xB8, 0x7E, 0x01, 0x00]], dtype=np.uint8)    # 1, -1, 448, 2^-9, 0
    got = ora.dequant("fp8", codes, np.float32(0.75), 5)
    assert np.array_equal(got, np.array([[0.75, -0.75, 336.0, 0.75 * 2.0 ** -9, 0.0]]))


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
