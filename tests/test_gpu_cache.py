"""GPU parity of the growing cache: kvd_append_kv against the oracle's
encoder (bit-exact cache bytes), decode over striped and staggered caches
against the oracle, and a decode loop that appends one token per step."""
import numpy as np
import pytest

import kvgen
import oracle
from oracle import cache as oc
from tests import gpu_cases as gc

pytestmark = pytest.mark.gpu


def _wl(kv, B=2, Hq=32, Hkv=2, D=128, Dv=None, S=200, alias=False, seed=41, q_dtype="bf16"):
    Dv = D if Dv is None else Dv
    return kvgen.Workload("cache_%s" % kv, B=B, Hq=Hq, Hkv=Hkv, Dqk=D, Dv=Dv, S_max=S, kvp=(4,),
                          q_dtype=q_dtype, kv_dtype=kv, seed=seed, seq_lens=(S,) * B, v_aliases_k=alias)


def _sharded_inputs(w, kvp):
    """Generated caches for a sharded layout: kvp * B slabs of S rows, viewed
    as [kvp,B,Hkv,S,...]; fp8 scales [B,Hkv]; q of the B requests."""
    import dataclasses
    big = dataclasses.replace(w, name=w.name + "_sh", B=kvp * w.B, seq_lens=(w.S_max,) * (kvp * w.B))
    inp = kvgen.make_inputs(big)
    def shard(a):
        return None if a is None else a.reshape((kvp, w.B) + a.shape[1:])
    cache = {"k": shard(inp.k_data), "v": shard(inp.v_data)}
    if w.kv_dtype == "fp8":
        cache["k_scale"] = inp.k_scale[:w.B].copy()
        cache["v_scale"] = None if inp.v_scale is None else inp.v_scale[:w.B].copy()
    else:
        cache["k_scale"], cache["v_scale"] = shard(inp.k_scale), shard(inp.v_scale)
    q = kvgen.make_inputs(w).q
    return q, cache


def _dev(a):
    import torch
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def _host(t, like):
    a = t.cpu().numpy()
    return a.view(np.uint16) if like.dtype == np.uint16 else a


def _decode_both(w, layout, kvp, q, cache, seq):
    import torch
    from long_context_decode_split_amd import kvd
    p = kvd.problem(w.B, w.Hq, w.Hkv, w.Dqk, w.Dv, w.S_max, kvp, w.q_dtype, w.kv_dtype, 0.0, w.v_aliases_k,
                    layout=layout)
    k = (_dev(cache["k"]), _dev(cache["k_scale"]))
    v = None if w.v_aliases_k else (_dev(cache["v"]), _dev(cache["v_scale"]))
    f32 = dict(dtype=torch.float32, device="cuda")
    o_part = torch.full((kvp, w.B, w.Hq, w.Dv), float("nan"), **f32)
    lse_part = torch.full((kvp, w.B, w.Hq), float("nan"), **f32)
    seq_d = _dev(np.asarray(seq, dtype=np.int32))
    kvd.kvd_decode_partial(p, _dev(q), k, v, seq_d, o_part, lse_part)
    ws = torch.empty(kvd.kvd_decode_workspace_bytes(p), dtype=torch.uint8, device="cuda")
    o = torch.full((w.B, w.Hq, w.Dv), float("nan"), **f32)
    lse = torch.full((w.B, w.Hq), float("nan"), **f32)
    kvd.kvd_decode(p, _dev(q), k, v, seq_d, ws, o, lse)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in (o_part, lse_part, o, lse)]


SHAPES = {
    "g16": dict(Hq=32, Hkv=2, D=128),                          # matrix-core GQA kernel
    "g4": dict(Hq=8, Hkv=2, D=64),                             # vector-ALU kernel
    "mla": dict(B=2, Hq=128, Hkv=1, D=576, Dv=512, alias=True),
}
CASES = [(lay, kv, sh) for lay in ("striped", "staggered16") for kv in ("bf16", "fp8", "mxfp4")
         for sh in ("g16", "g4", "mla") if not (sh == "mla" and kv != "bf16") and not (sh == "g4" and kv == "mxfp4")]


@pytest.mark.parametrize("layout,kv,shape", CASES, ids=lambda x: str(x))
def test_decode_sharded_layout(layout, kv, shape):
    """Partials and merged output over a sharded cache, lengths with ragged
    runs, empty shards and a full cache."""
    kvp, S = 4, 80
    w = _wl(kv, S=S, **SHAPES[shape])
    q, cache = _sharded_inputs(w, kvp)
    p = oracle.Problem(w.B, w.Hq, w.Hkv, w.Dqk, w.Dv, S, w.q_dtype, w.kv_dtype, w.v_aliases_k)
    for seq in ((kvp * S, 3), (77, 150), (0, 16 * kvp + 5)):
        o_part, lse_part, o, lse = _decode_both(w, layout, kvp, q, cache, seq)
        ref_po, ref_pl = oc.decode_partials_layout(p, layout, kvp, q, cache, np.array(seq))
        ref_o, ref_l = oc.decode_layout(p, layout, kvp, q, cache, np.array(seq))
        what = "%s %s %s L=%s" % (layout, kv, shape, seq)
        gc.compare(o_part, lse_part, ref_po, ref_pl, kv, what + " partials")
        gc.compare(o, lse, ref_o, ref_l, kv, what + " merged")


def _zero_cache(w, layout, kvp, S):
    lead = (w.B, w.Hkv, S) if layout == "contiguous" else (kvp, w.B, w.Hkv, S)
    def one(D):
        if w.kv_dtype == "f32":
            return np.zeros(lead + (D,), np.float32), None
        if w.kv_dtype == "bf16":
            return np.zeros(lead + (D,), np.uint16), None
        if w.kv_dtype == "fp8":
            return np.zeros(lead + (D,), np.uint8), np.linspace(0.01, 0.05, w.B * w.Hkv,
                                                                dtype=np.float32).reshape(w.B, w.Hkv)
        return np.zeros(lead + (D // 2,), np.uint8), np.zeros(lead + (D // 32,), np.uint8)
    k, ks = one(w.Dqk)
    v, vs = (None, None) if w.v_aliases_k else one(w.Dv)
    return {"k": k, "k_scale": ks, "v": v, "v_scale": vs}


@pytest.mark.parametrize("layout", ["contiguous", "striped", "staggered16"])
@pytest.mark.parametrize("kv", ["f32", "bf16", "fp8", "mxfp4"])
def test_append_bitexact(layout, kv):
    """Cache bytes after a stream of appends equal the oracle encoder's, bit
    for bit; out-of-range and negative positions are skipped."""
    import torch
    from long_context_decode_split_amd import kvd
    kvp, S, T = 3, 40, 60
    w = _wl(kv, B=3, Hq=8, Hkv=2, D=64 if kv != "mxfp4" else 128, S=S)
    host = _zero_cache(w, layout, kvp, S)
    dev = {n: _dev(a) for n, a in host.items()}
    p = kvd.problem(w.B, w.Hq, w.Hkv, w.Dqk, w.Dv, S, kvp, w.q_dtype, w.kv_dtype, 0.0, False, layout=layout)
    po = oracle.Problem(w.B, w.Hq, w.Hkv, w.Dqk, w.Dv, S, w.q_dtype, w.kv_dtype)
    rng = np.random.default_rng(9)
    cap = S if layout == "contiguous" else kvp * S
    for t in range(T):
        kn = rng.standard_normal((w.B, w.Hkv, w.Dqk)).astype(np.float32)
        vn = rng.standard_normal((w.B, w.Hkv, w.Dv)).astype(np.float32)
        if t % 7 == 3:            # outliers: fp8 saturation, MXFP4 big blocks
            kn[0, 0, :5] *= 1e3
            vn[-1, -1, -3:] *= -1e4
        if t % 11 == 5:           # tiny values
            kn[1] *= 1e-6
        pos = np.array([t, (5 * t) % (cap + 8), -1 if t % 9 == 0 else t + 1], dtype=np.int32)
        oc.append(po, layout, kvp, host, pos, kn, vn)
        kvd.kvd_append_kv(p, _dev(kn), _dev(vn), _dev(pos), (dev["k"], dev["k_scale"]),
                          (dev["v"], dev["v_scale"]))
    torch.cuda.synchronize()
    for n in ("k", "v"):
        got = _host(dev[n], host[n])
        assert np.array_equal(got.view(np.uint8), host[n].view(np.uint8)), "%s %s %s data differs" % (layout, kv, n)
        if kv == "mxfp4":
            assert np.array_equal(_host(dev[n + "_scale"], host[n + "_scale"]), host[n + "_scale"]), n
    gc.log("  append %s %s: %d tokens bit-exact" % (layout, kv, T))


def test_append_latent_writes_k_only():
    import torch
    from long_context_decode_split_amd import kvd
    w = _wl("bf16", B=2, Hq=128, Hkv=1, D=576, Dv=512, S=32, alias=True)
    host = _zero_cache(w, "staggered16", 2, 32)
    dk = _dev(host["k"])
    p = kvd.problem(w.B, w.Hq, w.Hkv, 576, 512, 32, 2, "bf16", "bf16", 0.0, True, layout="staggered16")
    po = oracle.Problem(w.B, w.Hq, 1, 576, 512, 32, "bf16", "bf16", True)
    rng = np.random.default_rng(3)
    for t in range(40):
        kn = rng.standard_normal((w.B, 1, 576)).astype(np.float32)
        pos = np.array([t, 39 - t], dtype=np.int32)
        oc.append(po, "staggered16", 2, host, pos, kn, None)
        kvd.kvd_append_kv(p, _dev(kn), None, _dev(pos), (dk, None), None)
    torch.cuda.synchronize()
    assert np.array_equal(_host(dk, host["k"]), host["k"])


@pytest.mark.parametrize("layout", ["contiguous", "striped", "staggered16"])
def test_decode_loop_appends_one_token_per_step(layout):
    """A decode loop: each step appends the new token of every request, then
    decodes; every step matches the oracle on the same cache."""
    import torch
    from long_context_decode_split_amd import kvd
    kvp, S = 4, 96
    w = _wl("fp8", B=2, Hq=32, Hkv=2, D=128, S=S)
    cap = S if layout == "contiguous" else kvp * S
    if layout == "contiguous":
        inp = kvgen.make_inputs(w)
        host = {"k": inp.k_data.copy(), "k_scale": inp.k_scale, "v": inp.v_data.copy(), "v_scale": inp.v_scale}
        q = inp.q
    else:
        q, host = _sharded_inputs(w, kvp)
    dev = {n: _dev(a) for n, a in host.items()}
    p = kvd.problem(w.B, w.Hq, w.Hkv, 128, 128, S, kvp, "bf16", "fp8", 0.0, False, layout=layout)
    po = oracle.Problem(w.B, w.Hq, w.Hkv, 128, 128, S, "bf16", "fp8")
    L = np.array([min(cap - 12, 70), 17], dtype=np.int32)
    rng = np.random.default_rng(21)
    ws = torch.empty(kvd.kvd_decode_workspace_bytes(p), dtype=torch.uint8, device="cuda")
    o = torch.empty((w.B, w.Hq, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device="cuda")
    qd = _dev(q)
    for step in range(10):
        kn = rng.standard_normal((w.B, w.Hkv, 128)).astype(np.float32)
        vn = rng.standard_normal((w.B, w.Hkv, 128)).astype(np.float32)
        oc.append(po, layout, kvp, host, L, kn, vn)
        kvd.kvd_append_kv(p, _dev(kn), _dev(vn), _dev(L), (dev["k"], dev["k_scale"]), (dev["v"], dev["v_scale"]))
        L = L + 1
        kvd.kvd_decode(p, qd, (dev["k"], dev["k_scale"]), (dev["v"], dev["v_scale"]), _dev(L), ws, o, lse)
        torch.cuda.synchronize()
        ref_o, ref_l = oc.decode_layout(po, layout, kvp, q, host, L)
        gc.compare(o.cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, "fp8", "%s step %d" % (layout, step))


def _paged_from_contiguous(w, inp, bl, max_blocks, rng, spare=5):
    """Scatter a generated contiguous cache [B,Hkv,max_blocks*bl,...] into a
    pool of blocks through a scrambled block table."""
    num_blocks = w.B * max_blocks + spare
    table = rng.permutation(num_blocks)[:w.B * max_blocks].reshape(w.B, max_blocks).astype(np.int32)
    def scatter(a):
        if a is None:
            return None
        pool = np.zeros((num_blocks, w.Hkv, bl) + a.shape[3:], dtype=a.dtype)
        for b in range(w.B):
            for lb in range(max_blocks):
                pool[table[b, lb]] = a[b, :, lb * bl:(lb + 1) * bl]
        return pool
    cache = {"k": scatter(inp.k_data), "v": scatter(inp.v_data), "block_len": bl, "block_table": table}
    if w.kv_dtype == "mxfp4":
        cache["k_scale"], cache["v_scale"] = scatter(inp.k_scale), scatter(inp.v_scale)
    else:
        cache["k_scale"], cache["v_scale"] = inp.k_scale, inp.v_scale
    return cache, num_blocks


def _paged_problem(w, kvp, cache, num_blocks, table_dev):
    from long_context_decode_split_amd import kvd
    return kvd.problem(w.B, w.Hq, w.Hkv, w.Dqk, w.Dv, 1, kvp, w.q_dtype, w.kv_dtype, 0.0, w.v_aliases_k,
                       layout="paged", block_len=cache["block_len"], max_blocks=cache["block_table"].shape[1],
                       num_blocks=num_blocks, block_table=table_dev)


PAGED_CASES = [(kv, sh, bl) for kv in ("bf16", "fp8", "mxfp4") for sh in ("g16", "g4", "mla") for bl in (16, 64)
               if not (sh == "mla" and kv != "bf16") and not (sh == "g4" and kv == "mxfp4")]


@pytest.mark.parametrize("kv,shape,bl", PAGED_CASES, ids=lambda x: str(x))
def test_decode_paged(kv, shape, bl):
    """Partials and merged output over a paged pool with a scrambled block
    table, ragged lengths, an empty request and a full table."""
    import torch
    from long_context_decode_split_amd import kvd
    max_blocks = 192 // bl
    S = max_blocks * bl
    w = _wl(kv, S=S, **SHAPES[shape])
    inp = kvgen.make_inputs(w)
    rng = np.random.default_rng(bl)
    cache, num_blocks = _paged_from_contiguous(w, inp, bl, max_blocks, rng)
    table_dev = _dev(cache["block_table"])
    p = _paged_problem(w, 5, cache, num_blocks, table_dev)
    po = oracle.Problem(w.B, w.Hq, w.Hkv, w.Dqk, w.Dv, S, w.q_dtype, w.kv_dtype, w.v_aliases_k)
    k = (_dev(cache["k"]), _dev(cache["k_scale"]))
    v = None if w.v_aliases_k else (_dev(cache["v"]), _dev(cache["v_scale"]))
    f32 = dict(dtype=torch.float32, device="cuda")
    for seq in ((S, 0), (177, 31), (bl + 1, S - 3)):
        o_part = torch.full((5, w.B, w.Hq, w.Dv), float("nan"), **f32)
        lse_part = torch.full((5, w.B, w.Hq), float("nan"), **f32)
        seq_d = _dev(np.asarray(seq, dtype=np.int32))
        kvd.kvd_decode_partial(p, _dev(inp.q), k, v, seq_d, o_part, lse_part)
        torch.cuda.synchronize()
        ref_po, ref_pl = oc.decode_partials_layout(po, "paged", 5, inp.q, cache, np.array(seq))
        gc.compare(o_part.cpu().numpy(), lse_part.cpu().numpy(), ref_po, ref_pl, kv,
                   "paged bl=%d %s %s L=%s" % (bl, kv, shape, seq))


@pytest.mark.parametrize("kv", ["f32", "bf16", "fp8", "mxfp4"])
def test_append_paged_bitexact(kv):
    import torch
    from long_context_decode_split_amd import kvd
    bl, max_blocks, T = 16, 4, 70
    w = _wl(kv, B=3, Hq=8, Hkv=2, D=64 if kv != "mxfp4" else 128, S=bl * max_blocks)
    rng = np.random.default_rng(12)
    num_blocks = w.B * max_blocks + 2
    table = rng.permutation(num_blocks)[:w.B * max_blocks].reshape(w.B, max_blocks).astype(np.int32)
    table[2, 1] = -1                                   # writes through it are skipped
    zero = _zero_cache(w, "contiguous", 1, 1)
    def pool(a):
        return None if a is None else np.zeros((num_blocks, w.Hkv, bl) + a.shape[3:], a.dtype)
    host = {"k": pool(zero["k"]), "v": pool(zero["v"]), "block_len": bl, "block_table": table}
    if kv == "mxfp4":
        host["k_scale"], host["v_scale"] = pool(zero["k_scale"]), pool(zero["v_scale"])
    else:
        host["k_scale"], host["v_scale"] = zero["k_scale"], zero["v_scale"]
    dev = {n: _dev(host[n]) for n in ("k", "k_scale", "v", "v_scale")}
    table_dev = _dev(table)
    p = kvd.problem(w.B, w.Hq, w.Hkv, w.Dqk, w.Dv, 1, 2, w.q_dtype, w.kv_dtype, 0.0, False, layout="paged",
                    block_len=bl, max_blocks=max_blocks, num_blocks=num_blocks, block_table=table_dev)
    po = oracle.Problem(w.B, w.Hq, w.Hkv, w.Dqk, w.Dv, bl * max_blocks, w.q_dtype, w.kv_dtype)
    for t in range(T):
        kn = rng.standard_normal((w.B, w.Hkv, w.Dqk)).astype(np.float32)
        vn = rng.standard_normal((w.B, w.Hkv, w.Dv)).astype(np.float32)
        pos = np.array([t, (3 * t) % (bl * max_blocks + 5), t // 2], dtype=np.int32)
        oc.append(po, "paged", 2, host, pos, kn, vn)
        kvd.kvd_append_kv(p, _dev(kn), _dev(vn), _dev(pos), (dev["k"], dev["k_scale"]), (dev["v"], dev["v_scale"]))
    torch.cuda.synchronize()
    for n in ("k", "v"):
        assert np.array_equal(_host(dev[n], host[n]).view(np.uint8), host[n].view(np.uint8)), n
        if kv == "mxfp4":
            assert np.array_equal(_host(dev[n + "_scale"], host[n + "_scale"]), host[n + "_scale"]), n
