"""Pins of the multi-token (pass-Q, T >= 1 new query tokens) oracle,
oracle/passq.py.  CPU only.

Each pin checks the oracle against something other than itself: explicit
loops over a causal score table, torch's own lower-right causal attention in
float64, the single-token oracle (pinned in tests/test_oracle.py) on every
query's visible prefix, closed forms, and the merge of shard partials over
every cache layout.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import cache as oc
from oracle import passq as op

LAYOUTS = ("contiguous", "striped", "staggered16", "paged")


def _problem(B=2, Hq=4, Hkv=2, D=16, kv="f32"):
    return oracle.Problem(B, Hq, Hkv, D, D, 0, "f32", kv)


def _contiguous(p, S, rng):
    """A contiguous f32 cache [B,Hkv,S,D] of N(0,1) rows."""
    return {"k": rng.standard_normal((p.B, p.Hkv, S, p.Dqk)).astype(np.float32), "k_scale": None,
            "v": rng.standard_normal((p.B, p.Hkv, S, p.Dv)).astype(np.float32), "v_scale": None}


def _as_layout(p, layout, kvp, co, seq, rng):
    """The tokens of contiguous cache `co` stored under `layout` (placed row by
    row from the layout's definition)."""
    if layout == "contiguous":
        return co
    S = co["k"].shape[2]
    if layout == "paged":
        bl = 16
        nb = -(-S // bl)
        num_blocks = p.B * nb + 2
        table = rng.permutation(num_blocks)[:p.B * nb].reshape(p.B, nb).astype(np.int32)
        out = {"k_scale": None, "v_scale": None, "block_len": bl, "block_table": table}
        for name in ("k", "v"):
            a = co[name]
            pool = np.full((num_blocks, p.Hkv, bl, a.shape[-1]), np.nan, np.float32)
            for b in range(p.B):
                for i in range(S):
                    pool[table[b, i // bl], :, i % bl] = a[b, :, i]
            out[name] = pool
        return out
    cap = S // kvp + 32
    out = {"k_scale": None, "v_scale": None}
    for name in ("k", "v"):
        a = co[name]
        sh = np.full((kvp, p.B, p.Hkv, cap, a.shape[-1]), np.nan, np.float32)
        for b in range(p.B):
            for i in range(int(seq[b])):
                if layout == "striped":
                    j, r = i % kvp, i // kvp
                else:
                    j, r = (i // 16) % kvp, 16 * (i // (16 * kvp)) + i % 16
                sh[j, b, :, r] = a[b, :, i]
        out[name] = sh
    return out


def _q(p, T, rng):
    return rng.standard_normal((p.B, T, p.Hq, p.Dqk)).astype(np.float32)


# ------------------------------------------------------------ brute force

def test_brute_force_causal_loops():
    """Every output against explicit loops: score table, causal cut at
    position L - T + t, softmax with math.exp (request 1 is shorter than T)."""
    p = _problem(B=2, Hq=4, Hkv=2, D=8)
    T = 3
    rng = np.random.default_rng(11)
    co = _contiguous(p, 6, rng)
    seq = np.array([6, 2], dtype=np.int32)
    q = _q(p, T, rng)
    o, lse = op.decode_tokens(p, T, "contiguous", 1, q, co, seq)
    sc = 1.0 / math.sqrt(p.Dqk)
    for b in range(p.B):
        L = int(seq[b])
        for t in range(T):
            last = L - T + t          # newest position query t may see
            for h in range(p.Hq):
                kvh = h // (p.Hq // p.Hkv)
                xs = []
                for s in range(L):
                    if s <= last:
                        xs.append(sc * sum(float(q[b, t, h, d]) * float(co["k"][b, kvh, s, d])
                                           for d in range(p.Dqk)))
                if not xs:
                    assert lse[b, t, h] == -np.inf
                    assert np.all(o[b, t, h] == 0.0)
                    continue
                m = max(xs)
                w = [math.exp(x - m) for x in xs]
                tot = sum(w)
                for d in range(p.Dv):
                    ref = sum(w[s] * float(co["v"][b, kvh, s, d]) for s in range(len(xs))) / tot
                    assert abs(o[b, t, h, d] - ref) < 1e-12
                assert abs(lse[b, t, h] - (m + math.log(tot))) < 1e-12


def test_matches_torch_lower_right_causal_attention():
    """torch's scaled_dot_product_attention with its lower-right causal bias
    (query t of T sees the keys up to L - T + t) in float64, GQA heads
    expanded by torch's repeat_interleave."""
    from torch.nn.attention.bias import causal_lower_right
    p = _problem(B=2, Hq=8, Hkv=2, D=32)
    rng = np.random.default_rng(12)
    for T, L in ((5, 37), (16, 16), (7, 100)):
        co = _contiguous(p, L, rng)
        seq = np.array([L, L], dtype=np.int32)
        q = _q(p, T, rng)
        o, _ = op.decode_tokens(p, T, "contiguous", 1, q, co, seq)
        G = p.Hq // p.Hkv
        qt = torch.from_numpy(q.astype(np.float64)).transpose(1, 2)                # [B,Hq,T,D]
        kt = torch.from_numpy(co["k"].astype(np.float64)).repeat_interleave(G, dim=1)
        vt = torch.from_numpy(co["v"].astype(np.float64)).repeat_interleave(G, dim=1)
        ref = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=causal_lower_right(T, L))
        np.testing.assert_allclose(o, ref.transpose(1, 2).numpy(), rtol=0, atol=1e-12)


# ---------------------------------------------- reductions and closed forms

@pytest.mark.parametrize("layout", LAYOUTS)
def test_one_token_is_the_single_token_oracle(layout):
    p = _problem()
    rng = np.random.default_rng(13)
    seq = np.array([70, 23], dtype=np.int32)
    kvp = 3
    cache = _as_layout(p, layout, kvp, _contiguous(p, 70, rng), seq, rng)
    q = _q(p, 1, rng)
    o, lse = op.decode_tokens(p, 1, layout, kvp, q, cache, seq)
    ro, rl = oc.decode_layout(p, layout, kvp, q[:, 0], cache, seq)
    np.testing.assert_array_equal(o[:, 0], ro)
    np.testing.assert_array_equal(lse[:, 0], rl)
    po, pl = op.decode_partials_tokens(p, 1, layout, kvp, q, cache, seq)
    rpo, rpl = oc.decode_partials_layout(p, layout, kvp, q[:, 0], cache, seq)
    np.testing.assert_array_equal(po[:, :, 0], rpo)
    np.testing.assert_array_equal(pl[:, :, 0], rpl)


def test_each_query_is_a_single_token_decode_of_its_prefix():
    """Query t equals one-token decode of the cache cut to its visible
    length L - T + 1 + t (the token itself is the last key it sees)."""
    p = _problem(Hq=6, Hkv=3)
    rng = np.random.default_rng(14)
    T = 9
    co = _contiguous(p, 50, rng)
    seq = np.array([50, 12], dtype=np.int32)
    q = _q(p, T, rng)
    o, lse = op.decode_tokens(p, T, "contiguous", 1, q, co, seq)
    pc = oracle.Problem(p.B, p.Hq, p.Hkv, p.Dqk, p.Dv, 50, "f32", "f32")
    for t in range(T):
        cut = seq - (T - 1 - t)
        ro, rl = oracle.decode(pc, q[:, t], co["k"], None, co["v"], None, cut)
        np.testing.assert_array_equal(o[:, t], ro)
        np.testing.assert_array_equal(lse[:, t], rl)


def test_equal_keys_give_the_mean_of_the_visible_values():
    """With every key zero each visible logit is 0: o is the plain mean of the
    first L - T + 1 + t value rows and lse = ln(L - T + 1 + t); a query with
    no visible key gives o = 0, lse = -inf; constant V returns the constant."""
    p = _problem(B=3, Hq=2, Hkv=1, D=8)
    rng = np.random.default_rng(15)
    T = 5
    seq = np.array([21, 5, 3], dtype=np.int32)
    co = _contiguous(p, 21, rng)
    co["k"][:] = 0.0
    q = _q(p, T, rng)
    o, lse = op.decode_tokens(p, T, "contiguous", 1, q, co, seq)
    for b in range(p.B):
        for t in range(T):
            n = int(seq[b]) - T + 1 + t
            if n <= 0:
                assert np.all(lse[b, t] == -np.inf) and np.all(o[b, t] == 0.0)
                continue
            mean = co["v"][b, 0, :n].astype(np.float64).mean(axis=0)
            np.testing.assert_allclose(o[b, t], np.broadcast_to(mean, o[b, t].shape), rtol=0, atol=1e-14)
            np.testing.assert_allclose(lse[b, t], math.log(n), rtol=0, atol=1e-14)
    co2 = _contiguous(p, 21, rng)
    co2["v"][:] = 0.625
    o2, _ = op.decode_tokens(p, T, "contiguous", 1, q, co2, seq)
    for b in range(p.B):
        for t in range(T):
            if int(seq[b]) - T + 1 + t > 0:
                np.testing.assert_allclose(o2[b, t], 0.625, rtol=0, atol=1e-15)


# ------------------------------------------------------- split invariance

@pytest.mark.parametrize("layout", LAYOUTS)
def test_merged_partials_equal_full_context(layout):
    """Merging the shard partials gives the full-context result for every
    query token, including shards none of whose tokens a query sees."""
    p = _problem(Hq=4, Hkv=2, D=16)
    rng = np.random.default_rng(16)
    for T, seq, kvp in ((7, (100, 3), 3), (16, (53, 16), 8), (2, (33, 1), 1), (5, (64, 40), 5)):
        seq = np.array(seq, dtype=np.int32)
        cache = _as_layout(p, layout, kvp, _contiguous(p, int(seq.max()), rng), seq, rng)
        q = _q(p, T, rng)
        o, lse = op.decode_tokens(p, T, layout, kvp, q, cache, seq)
        po, pl = op.decode_partials_tokens(p, T, layout, kvp, q, cache, seq)
        assert po.shape == (kvp, p.B, T, p.Hq, p.Dv) and pl.shape == (kvp, p.B, T, p.Hq)
        mo, ml = oracle.merge(po, pl)
        np.testing.assert_allclose(mo, o, rtol=0, atol=1e-12)
        np.testing.assert_allclose(ml, lse, rtol=0, atol=1e-12)
        empty = pl == -np.inf
        assert np.all(po[empty] == 0.0)


def test_contiguous_partials_cut_each_shard_at_the_query():
    """Contiguous split of a 100-token request over 4 shards (C = 32): the
    last shard holds positions 96..99; with T = 8 query t sees positions
    < 93 + t, so queries 0..3 see none of it and query 7 all four."""
    p = _problem(B=1, Hq=2, Hkv=1, D=8)
    rng = np.random.default_rng(17)
    co = _contiguous(p, 100, rng)
    seq = np.array([100], dtype=np.int32)
    q = _q(p, 8, rng)
    po, pl = op.decode_partials_tokens(p, 8, "contiguous", 4, q, co, seq)
    assert np.all(pl[3, 0, :4] == -np.inf)
    pc = oracle.Problem(1, 2, 1, 8, 8, 100, "f32", "f32")
    qf = q.astype(np.float64)
    for t in range(4, 8):
        k, v = oracle.slab_kv(pc, co["k"], None, co["v"], None, 0, 0, 96, 93 + t)
        ro, rl = oracle.attend(qf[0, t], k, v, p.sm_scale)
        np.testing.assert_array_equal(po[3, 0, t], ro)
        np.testing.assert_array_equal(pl[3, 0, t], rl)
    assert np.all(np.isfinite(pl[:3]))


# ------------------------------------------------------------------ append

@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("kv", ["bf16", "mxfp4"])
def test_append_tokens_is_t_single_appends(layout, kv):
    """Token t goes to positions[b] + t: the same as T one-token appends; a
    negative position skips the whole request; tokens past the end are
    skipped one by one."""
    D = 64
    p = oracle.Problem(3, 4, 2, D, D, 0, "f32", kv)
    kvp, T = 3, 6
    rng = np.random.default_rng(18)

    def empty():
        if layout == "paged":
            bl, nb = 16, 4
            nblk = p.B * nb
            table = np.arange(nblk, dtype=np.int32)[::-1].reshape(p.B, nb).copy()
            shape = (nblk, p.Hkv, bl)
            extra = {"block_len": bl, "block_table": table}
        elif layout == "contiguous":
            shape, extra = (p.B, p.Hkv, 64), {}
        else:
            shape, extra = (kvp, p.B, p.Hkv, 32), {}
        if kv == "bf16":
            c = {"k": np.zeros(shape + (D,), np.uint16), "v": np.zeros(shape + (D,), np.uint16),
                 "k_scale": None, "v_scale": None}
        else:
            c = {"k": np.zeros(shape + (D // 2,), np.uint8), "v": np.zeros(shape + (D // 2,), np.uint8),
                 "k_scale": np.zeros(shape + (D // 32,), np.uint8), "v_scale": np.zeros(shape + (D // 32,), np.uint8)}
        c.update(extra)
        return c

    a, b_ = empty(), empty()
    kn = rng.standard_normal((p.B, T, p.Hkv, D)).astype(np.float32)
    vn = rng.standard_normal((p.B, T, p.Hkv, D)).astype(np.float32)
    pos = [5, -1, 61]           # request 2 runs past a 64-token cache after 3 tokens
    op.append_tokens(p, T, layout, kvp, a, pos, kn, vn)
    for t in range(T):
        oc.append(p, layout, kvp, b_, [5 + t, -1, 61 + t], kn[:, t], vn[:, t])
    for name in ("k", "v", "k_scale", "v_scale"):
        if a[name] is not None:
            np.testing.assert_array_equal(a[name], b_[name])
    # request 1 (negative position) left untouched, and something was written
    g = oc.gather_contiguous(p, layout, kvp, a, [64, 64, 64]) if layout != "contiguous" else a
    assert not np.any(g["k"][1])
    assert np.any(g["k"][0, :, 5:11]) and not np.any(g["k"][0, :, 11:])
