"""Plant plausible mistakes in the multi-token oracle (on the CPU) and check
that one of its pins (tests/test_oracle_passq.py) catches each."""
import numpy as np
import pytest

import oracle
import oracle.passq as op
from oracle import cache as oc
from tests import test_oracle_passq as pins

_REAL = {n: getattr(op, n) for n in ("visible", "_q4", "decode_partials_tokens", "append_tokens")}


def _visible_excludes_self(L, T, t):
    return max(0, min(L, L - T + t))


def _visible_top_left(L, T, t):
    return max(0, min(L, t + 1))


def _q_head_major(p, T, q):
    qf = oracle.q_to_f64(q, p.q_dtype)
    return qf.reshape(p.B, p.Hq, T, p.Dqk).transpose(0, 2, 1, 3)


def _partials_local_row_cut(p, T, layout, kvp, q, cache, seq_lens, pairs=None):
    """Sharded layouts: cut each shard at local row vis(t) instead of at the
    global position."""
    if layout in ("contiguous", oc.PAGED):
        return _REAL["decode_partials_tokens"](p, T, layout, kvp, q, cache, seq_lens, pairs)
    qf = _REAL["_q4"](p, T, q)
    o = np.full((kvp, p.B, T, p.Hq, p.Dv), np.nan)
    lse = np.full((kvp, p.B, T, p.Hq), np.nan)
    for b in range(p.B):
        L = int(seq_lens[b])
        held = oc.shard_tokens(L, kvp, layout)
        for kvh in range(p.Hkv):
            hs = slice(kvh * p.G, (kvh + 1) * p.G)
            for j in range(kvp):
                k = cache["k"][j, b, kvh].astype(np.float64)
                v = cache["v"][j, b, kvh].astype(np.float64)
                for t in range(T):
                    n = min(len(held[j]), op.visible(L, T, t))
                    o[j, b, t, hs], lse[j, b, t, hs] = oracle.attend(qf[b, t, hs], k[:n], v[:n], p.sm_scale)
    return o, lse


def _partials_uncut(p, T, layout, kvp, q, cache, seq_lens, pairs=None):
    """Shard partials that ignore the causal cut (every query sees the whole shard)."""
    qf = _REAL["_q4"](p, T, q)
    o = np.full((kvp, p.B, T, p.Hq, p.Dv), np.nan)
    lse = np.full((kvp, p.B, T, p.Hq), np.nan)
    for t in range(T):
        o[:, :, t], lse[:, :, t] = oc.decode_partials_layout(p, layout, kvp, qf[:, t].astype(np.float32),
                                                             cache, seq_lens, pairs)
    return o, lse


def _append_reversed(p, T, layout, kvp, cache, positions, k_new, v_new):
    k4 = np.asarray(k_new, dtype=np.float32).reshape(p.B, T, p.Hkv, p.Dqk)
    v4 = np.asarray(v_new, dtype=np.float32).reshape(p.B, T, p.Hkv, p.Dv)
    return _REAL["append_tokens"](p, T, layout, kvp, cache, positions, k4[:, ::-1], v4[:, ::-1])


def _append_negative_not_skipped(p, T, layout, kvp, cache, positions, k_new, v_new):
    k4 = np.asarray(k_new, dtype=np.float32).reshape(p.B, T, p.Hkv, p.Dqk)
    v4 = np.asarray(v_new, dtype=np.float32).reshape(p.B, T, p.Hkv, p.Dv)
    for t in range(T):
        oc.append(p, layout, kvp, cache, [int(x) + t for x in positions], k4[:, t], v4[:, t])


MUTATIONS = {
    "visibility excludes the query's own token": ("visible", _visible_excludes_self),
    "causal mask aligned top-left": ("visible", _visible_top_left),
    "q read as [B,Hq,T,D]": ("_q4", _q_head_major),
    "sharded partials cut at the local row": ("decode_partials_tokens", _partials_local_row_cut),
    "partials ignore the causal cut": ("decode_partials_tokens", _partials_uncut),
    "append: tokens in reverse order": ("append_tokens", _append_reversed),
    "append: negative start not skipped for t > 0": ("append_tokens", _append_negative_not_skipped),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    attr, bad = MUTATIONS[name]
    monkeypatch.setattr(op, attr, bad)
    caught = []
    for pname, fn, kw in _pin_calls():
        try:
            with np.errstate(all="ignore"):
                fn(**kw)
        except Exception:  # noqa: BLE001 - any failure counts as caught
            caught.append(pname)
    assert caught, "no pin caught mutation %r" % name


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
