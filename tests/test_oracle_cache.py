"""Pins of the cache oracle (oracle/cache.py): shard layouts, token encoders,
append and decode over sharded caches.  CPU only.

Each pin checks the oracle against something other than itself: a step by
step simulation of the dealing rules, library conversions (torch), the OCP
fixtures, the separately written C++ generator's encoders, and the plain
decode of the same tokens in contiguous order.
"""
import json
import os

import numpy as np
import pytest
import torch

import kvgen
import oracle
from oracle import cache as oc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- maps

def _simulate(L, kvp, run):
    """Deal tokens 0..L-1 to shards in runs of `run`, round-robin, keeping a
    row counter per shard (the dealing rule written as a process)."""
    rows = [0] * kvp
    owner, local = [], []
    shard, left = 0, run
    for _ in range(L):
        owner.append(shard)
        local.append(rows[shard])
        rows[shard] += 1
        left -= 1
        if left == 0:
            shard, left = (shard + 1) % kvp, run
    return owner, local


@pytest.mark.parametrize("layout,run", [("striped", 1), ("staggered16", 16)])
def test_owner_matches_dealing_process(layout, run):
    for kvp in (1, 2, 3, 5, 8):
        owner, local = _simulate(700, kvp, run)
        for i in range(700):
            assert oc.owner(i, kvp, layout) == (owner[i], local[i]), (layout, kvp, i)


@pytest.mark.parametrize("layout", oc.LAYOUTS)
def test_shard_tokens_partition(layout):
    for L in (0, 1, 15, 16, 17, 100, 257):
        for kvp in (1, 2, 3, 7, 16):
            toks = oc.shard_tokens(L, kvp, layout)
            assert len(toks) == kvp
            allt = np.concatenate(toks) if L else np.zeros(0, dtype=np.int64)
            assert sorted(allt.tolist()) == list(range(L))
            for t in toks:
                assert np.all(np.diff(t) > 0)
            lens = oc.shard_lengths(L, kvp, layout)
            assert lens.sum() == L
            if layout == "striped":
                assert lens.max() - lens.min() <= 1
            if layout == "staggered16":
                assert lens.max() - lens.min() <= 16


# ------------------------------------------------------------- encoders

def test_bf16_matches_torch():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(5000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 5000),
                        np.array([0.0, -0.0, 1.0, 65504.0, 3.0e38, 1e-40, -1e-42], dtype=np.float32)])
    x = x.astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oc.encode_bf16(x), ref)
    # exact ties: halfway between two bf16 values goes to the even one
    lo = np.float32(1.0).view(np.uint32)
    tie_even = np.array([lo + 0x8000], dtype=np.uint32).view(np.float32)      # 1 + 2^-8
    tie_odd = np.array([lo + 0x18000], dtype=np.uint32).view(np.float32)     # 1 + 3*2^-8
    assert oc.encode_bf16(tie_even)[0] == 0x3F80
    assert oc.encode_bf16(tie_odd)[0] == 0x3F82


def test_e4m3_matches_torch_in_range():
    rng = np.random.default_rng(2)
    y = (rng.standard_normal(20000) * 10.0 ** rng.uniform(-4, 2.6, 20000)).astype(np.float32)
    y = y[np.abs(y) < 448.0]
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oc.encode_e4m3(y), ref)


def test_e4m3_saturates_and_matches_generator():
    y = np.array([448.0, 449.0, 460.0, 479.9, 480.0, 1e6, -500.0, np.inf, -np.inf], dtype=np.float32)
    codes = oc.encode_e4m3(y)
    assert np.all((codes & 0x7F) == 0x7E)
    assert np.array_equal(codes >> 7, np.signbit(y).astype(np.uint8))
    rng = np.random.default_rng(3)
    z = (rng.standard_normal(50000) * 10.0 ** rng.uniform(-4, 3, 50000)).astype(np.float32)
    assert np.array_equal(oc.encode_e4m3(z), kvgen.encode_e4m3(z))


def test_e2m1_fixture_ties_and_generator():
    with open(os.path.join(GOLDEN, "ocp_e2m1_values.json")) as f:
        vals = np.array(json.load(f)["values"], dtype=np.float64)
    # every representable value encodes to its own code (signed zero included)
    assert np.array_equal(oc.encode_e2m1(vals), np.arange(16, dtype=np.uint8))
    ties = {0.25: 0.0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0, 5.0: 4.0, 7.0: 6.0, 100.0: 6.0}
    for x, want in ties.items():
        assert vals[oc.encode_e2m1(np.array([x]))[0]] == want, x
        assert vals[oc.encode_e2m1(np.array([-x]))[0]] == -want, x
    rng = np.random.default_rng(4)
    z = rng.standard_normal(50000) * 4.0
    assert np.array_equal(oc.encode_e2m1(z), kvgen.encode_e2m1(z))


def test_mxfp4_rows_match_generator():
    D, nrows = 128, 200
    x = kvgen.normals_f32(77, 2, 0, nrows * D).reshape(nrows, D)
    data, scales = kvgen.mxfp4_rows(77, 2, 0, nrows, D)
    data = np.asarray(data).reshape(nrows, D // 2)
    scales = np.asarray(scales).reshape(nrows, D // 32)
    for r in range(nrows):
        d, s = oc.encode_mxfp4_row(x[r])
        assert np.array_equal(d, data[r])
        assert np.array_equal(s, scales[r])


def test_mxfp4_block_exponent_edges():
    assert oc.mxfp4_block_exponent(np.zeros(32, np.float32)) == 127
    for e in (-126, -10, -1, 0, 1, 5, 100, 127):
        blk = np.zeros(32, np.float32)
        blk[3] = np.float32(2.0) ** e
        assert oc.mxfp4_block_exponent(blk) == min(254, max(0, e - 2 + 127)), e
        # largest fp32 below 2^(e+1)
        blk[3] = np.array([((e + 127) << 23) | 0x7FFFFF], dtype=np.uint32).view(np.float32)[0]
        assert oc.mxfp4_block_exponent(blk) == min(254, max(0, e - 2 + 127)), e
    tiny = np.zeros(32, np.float32)
    tiny[0] = np.float32(1e-45)       # subnormal fp32, floor(log2) = -149 -> E clamps to 0
    assert oc.mxfp4_block_exponent(tiny) == 0


def test_fp8_rows_match_generator_slab():
    slab = 4096
    codes, scales = kvgen.fp8_slabs(55, 1, 0, 1, slab)
    scales = np.asarray(scales).reshape(-1)
    x = kvgen.normals_f32(55, 1, 0, slab)
    assert np.array_equal(oc.encode_fp8(x, float(scales[0])), codes.reshape(-1))


# --------------------------------------------------- append and decode

def _problem(kv, Hq=8, Hkv=2, D=64, Dv=None, alias=False):
    Dv = D if Dv is None else Dv
    return oracle.Problem(2, Hq, Hkv, D, Dv, 0, "f32", kv, alias)


def _alloc(p, layout, kvp, S):
    shape = (p.B, p.Hkv, S) if layout == "contiguous" else (kvp, p.B, p.Hkv, S)
    def one(D):
        if p.kv_dtype == "f32":
            return np.zeros(shape + (D,), np.float32), None
        if p.kv_dtype == "bf16":
            return np.zeros(shape + (D,), np.uint16), None
        if p.kv_dtype == "fp8":
            return np.zeros(shape + (D,), np.uint8), np.full((p.B, p.Hkv), 0.05, np.float32)
        return np.zeros(shape + (D // 2,), np.uint8), np.zeros(shape + (D // 32,), np.uint8)
    k, ks = one(p.Dqk)
    v, vs = (None, None) if p.v_aliases_k else one(p.Dv)
    return {"k": k, "k_scale": ks, "v": v, "v_scale": vs}


@pytest.mark.parametrize("kv", ["f32", "bf16", "fp8", "mxfp4"])
@pytest.mark.parametrize("layout", ["striped", "staggered16"])
def test_appends_then_decode_equal_contiguous(kv, layout):
    """Appending the same token stream into a sharded and a contiguous cache
    stores the same encoded rows (permuted by the map), and the plain decode,
    the shard partials and their merge agree with the contiguous cache."""
    p = _problem(kv, D=64 if kv != "mxfp4" else 128)
    kvp, T = 3, 70
    rng = np.random.default_rng(5)
    sh = _alloc(p, layout, kvp, (T + kvp * 16) // kvp + 16)
    co = _alloc(p, "contiguous", kvp, T)
    if kv == "fp8":
        sh["v_scale"][:] = co["v_scale"][:] = 0.03
    for t in range(T):
        kn = rng.standard_normal((p.B, p.Hkv, p.Dqk)).astype(np.float32)
        vn = rng.standard_normal((p.B, p.Hkv, p.Dv)).astype(np.float32)
        pos = [t, t]
        oc.append(p, layout, kvp, sh, pos, kn, vn)
        oc.append(p, "contiguous", kvp, co, pos, kn, vn)
    seq = np.array([T, 41], dtype=np.int32)
    q = rng.standard_normal((p.B, p.Hq, p.Dqk)).astype(np.float32)
    # rows land where the map says
    for i in range(T):
        j, r = oc.owner(i, kvp, layout)
        assert np.array_equal(sh["k"][j, :, :, r], co["k"][:, :, i])
    full_c = oracle.decode(oracle.Problem(p.B, p.Hq, p.Hkv, p.Dqk, p.Dv, T, "f32", kv), q,
                           co["k"], co["k_scale"], co["v"], co["v_scale"], seq)
    full_s = oc.decode_layout(p, layout, kvp, q, sh, seq)
    np.testing.assert_allclose(full_s[0], full_c[0], rtol=0, atol=1e-13)
    np.testing.assert_allclose(full_s[1], full_c[1], rtol=0, atol=1e-13)
    po, pl = oc.decode_partials_layout(p, layout, kvp, q, sh, seq)
    mo, ml = oracle.merge(po, pl)
    np.testing.assert_allclose(mo, full_c[0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(ml, full_c[1], rtol=0, atol=1e-12)
    # each partial is attention over exactly the tokens its shard holds
    qf = oracle.q_to_f64(q, "f32")
    for b in range(p.B):
        for j, toks in enumerate(oc.shard_tokens(int(seq[b]), kvp, layout)):
            for kvh in range(p.Hkv):
                k, v = oracle.slab_kv(oracle.Problem(p.B, p.Hq, p.Hkv, p.Dqk, p.Dv, T, "f32", kv),
                                      co["k"], co["k_scale"], co["v"], co["v_scale"], b, kvh, 0, T)
                hs = slice(kvh * p.G, (kvh + 1) * p.G)
                o_ref, l_ref = oracle.attend(qf[b, hs], k[toks], v[toks], p.sm_scale)
                np.testing.assert_allclose(po[j, b, hs], o_ref, rtol=0, atol=1e-13)
                np.testing.assert_allclose(pl[j, b, hs], l_ref, rtol=0, atol=1e-13)


def test_append_latent_alias_writes_k_only():
    p = _problem("bf16", Hq=16, Hkv=1, D=64, Dv=32, alias=True)
    sh = _alloc(p, "striped", 2, 8)
    kn = np.ones((p.B, 1, 64), np.float32)
    oc.append(p, "striped", 2, sh, [3, 0], kn, None)
    assert sh["v"] is None
    assert np.all(sh["k"][1, 0, 0, 1] == 0x3F80)     # position 3 -> shard 1, row 1
    assert np.all(sh["k"][0, 1, 0, 0] == 0x3F80)     # position 0 -> shard 0, row 0


def _paged_cache(p, num_blocks, bl, table):
    def one(D):
        if p.kv_dtype == "f32":
            return np.zeros((num_blocks, p.Hkv, bl, D), np.float32), None
        if p.kv_dtype == "bf16":
            return np.zeros((num_blocks, p.Hkv, bl, D), np.uint16), None
        if p.kv_dtype == "fp8":
            return np.zeros((num_blocks, p.Hkv, bl, D), np.uint8), np.full((p.B, p.Hkv), 0.05, np.float32)
        return (np.zeros((num_blocks, p.Hkv, bl, D // 2), np.uint8),
                np.zeros((num_blocks, p.Hkv, bl, D // 32), np.uint8))
    k, ks = one(p.Dqk)
    v, vs = one(p.Dv)
    return {"k": k, "k_scale": ks, "v": v, "v_scale": vs, "block_len": bl, "block_table": table}


@pytest.mark.parametrize("kv", ["bf16", "fp8", "mxfp4"])
def test_paged_appends_then_decode_equal_contiguous(kv):
    """A paged pool with a scrambled block table holds, after the same appends,
    the rows of a contiguous cache at the blocks the table names; decode and
    shard partials agree; positions past the table and negative block ids are
    skipped."""
    p = _problem(kv, D=64 if kv != "mxfp4" else 128)
    bl, max_blocks, T, kvp = 16, 5, 75, 3
    rng = np.random.default_rng(8)
    num_blocks = p.B * max_blocks + 3
    table = rng.permutation(num_blocks)[:p.B * max_blocks].reshape(p.B, max_blocks).astype(np.int32)
    pg = _paged_cache(p, num_blocks, bl, table)
    co = _alloc(p, "contiguous", 1, max_blocks * bl)
    if kv == "fp8":
        pg["v_scale"][:] = co["v_scale"][:] = 0.03
    for t in range(T):
        kn = rng.standard_normal((p.B, p.Hkv, p.Dqk)).astype(np.float32)
        vn = rng.standard_normal((p.B, p.Hkv, p.Dv)).astype(np.float32)
        oc.append(p, "paged", kvp, pg, [t, t], kn, vn)
        oc.append(p, "contiguous", kvp, co, [t, t], kn, vn)
    for b in range(p.B):
        for i in range(T):
            assert np.array_equal(pg["k"][table[b, i // bl], :, i % bl], co["k"][b, :, i])
    seq = np.array([T, 33], dtype=np.int32)
    q = rng.standard_normal((p.B, p.Hq, p.Dqk)).astype(np.float32)
    pc = oracle.Problem(p.B, p.Hq, p.Hkv, p.Dqk, p.Dv, max_blocks * bl, "f32", kv)
    ref = oracle.decode(pc, q, co["k"], co["k_scale"], co["v"], co["v_scale"], seq)
    got = oc.decode_layout(p, "paged", kvp, q, pg, seq)
    np.testing.assert_allclose(got[0], ref[0], rtol=0, atol=1e-13)
    np.testing.assert_allclose(got[1], ref[1], rtol=0, atol=1e-13)
    rpo, rpl = oracle.decode_partials(pc, kvp, q, co["k"], co["k_scale"], co["v"], co["v_scale"], seq)
    po, pl = oc.decode_partials_layout(p, "paged", kvp, q, pg, seq)
    np.testing.assert_allclose(po, rpo, rtol=0, atol=1e-13)
    np.testing.assert_allclose(pl, rpl, rtol=0, atol=1e-13)
    # skipped writes: past the table, and through a negative block id
    before = pg["k"].copy()
    pg["block_table"] = table.copy()
    pg["block_table"][1, 0] = -1
    oc.append(p, "paged", kvp, pg, [max_blocks * bl, 3], np.ones((p.B, p.Hkv, p.Dqk), np.float32),
              np.ones((p.B, p.Hkv, p.Dv), np.float32))
    assert np.array_equal(pg["k"], before)
