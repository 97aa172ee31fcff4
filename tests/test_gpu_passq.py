"""GPU parity for T > 1 query tokens per request (a pass-Q turn, causal among
the new tokens): shard partials and merged outputs of every kernel family
over every cache layout against the oracle (oracle/passq.py), and the
multi-token append bit for bit."""
import numpy as np
import pytest

import kvgen
import oracle
from oracle import cache as oc
from oracle import passq as op
from tests import gpu_cases as gc
from tests.test_gpu_cache import SHAPES, _dev, _host, _paged_from_contiguous, _sharded_inputs, _wl, _zero_cache

pytestmark = pytest.mark.gpu


def _inputs(w, layout, kvp, S, T, rng):
    """(q [B,T,Hq,Dqk], cache dict, capacity) for `layout`; paged caches get a
    scrambled block table of 16-token blocks."""
    wt = w.with_(q_tokens=T)
    if layout in ("striped", "staggered16"):
        _, cache = _sharded_inputs(w, kvp)
        return kvgen.gen_q(wt), cache, kvp * S
    inp = kvgen.make_inputs(w)
    q = kvgen.gen_q(wt)
    if layout == "contiguous":
        return q, {"k": inp.k_data, "k_scale": inp.k_scale, "v": inp.v_data, "v_scale": inp.v_scale}, S
    cache, num_blocks = _paged_from_contiguous(w, inp, 16, S // 16, rng)
    cache["num_blocks"] = num_blocks
    return q, cache, S


def _run(w, T, layout, kvp, S, q, cache, seq):
    """o_part, lse_part, o, lse from kvd_decode_partial and kvd_decode; checks
    kvd_decode equals partial + kvd_lse_merge over B*T*Hq rows bitwise."""
    import torch
    from long_context_decode_split_amd import kvd
    extra = {}
    table_dev = None
    if layout == "paged":
        table_dev = _dev(cache["block_table"])
        extra = dict(block_len=cache["block_len"], max_blocks=cache["block_table"].shape[1],
                     num_blocks=cache["num_blocks"], block_table=table_dev)
    p = kvd.problem(w.B, w.Hq, w.Hkv, w.Dqk, w.Dv, S, kvp, w.q_dtype, w.kv_dtype, 0.0, w.v_aliases_k,
                    layout=layout, q_tokens=T, **extra)
    k = (_dev(cache["k"]), _dev(cache["k_scale"]))
    v = None if w.v_aliases_k else (_dev(cache["v"]), _dev(cache["v_scale"]))
    f32 = dict(dtype=torch.float32, device="cuda")
    o_part = torch.full((kvp, w.B, T, w.Hq, w.Dv), float("nan"), **f32)
    lse_part = torch.full((kvp, w.B, T, w.Hq), float("nan"), **f32)
    seq_d = _dev(np.asarray(seq, dtype=np.int32))
    qd = _dev(q)
    kvd.kvd_decode_partial(p, qd, k, v, seq_d, o_part, lse_part)
    o_m = torch.full((w.B, T, w.Hq, w.Dv), float("nan"), **f32)
    lse_m = torch.full((w.B, T, w.Hq), float("nan"), **f32)
    kvd.kvd_lse_merge(kvp, w.B * T * w.Hq, w.Dv, o_part, lse_part, o_m, lse_m)
    ws = torch.empty(kvd.kvd_decode_workspace_bytes(p), dtype=torch.uint8, device="cuda")
    o = torch.full_like(o_m, float("nan"))
    lse = torch.full_like(lse_m, float("nan"))
    kvd.kvd_decode(p, qd, k, v, seq_d, ws, o, lse)
    torch.cuda.synchronize()
    res = [t.cpu().numpy() for t in (o_part, lse_part, o, lse, o_m, lse_m)]
    assert np.array_equal(res[2], res[4]) and np.array_equal(res[3], res[5]), "kvd_decode != partial + merge"
    return res[:4]


def _check(w, T, layout, kvp, S, seqs, seed):
    rng = np.random.default_rng(seed)
    q, cache, cap = _inputs(w, layout, kvp, S, T, rng)
    p = oracle.Problem(w.B, w.Hq, w.Hkv, w.Dqk, w.Dv, S, w.q_dtype, w.kv_dtype, w.v_aliases_k)
    for seq in seqs:
        seq = np.minimum(np.asarray(seq, dtype=np.int64), cap).astype(np.int32)
        what = "%s %s G=%d T=%d kvp=%d L=%s" % (layout, w.kv_dtype, w.G, T, kvp, tuple(int(x) for x in seq))
        gc.log("  case " + what)
        o_part, lse_part, o, lse = _run(w, T, layout, kvp, S, q, cache, seq)
        ref_po, ref_pl = op.decode_partials_tokens(p, T, layout, kvp, q, cache, seq)
        ref_o, ref_l = op.decode_tokens(p, T, layout, kvp, q, cache, seq)
        gc.compare(o_part, lse_part, ref_po, ref_pl, w.kv_dtype, what + " partials")
        gc.compare(o, lse, ref_o, ref_l, w.kv_dtype, what + " merged")


LAYOUTS = ("contiguous", "striped", "staggered16", "paged")
FORMATS = [(kv, sh) for sh in ("g16", "g4", "mla") for kv in ("f32", "bf16", "fp8", "mxfp4")
           if not (sh == "mla" and kv != "bf16") and not (sh == "g4" and kv == "mxfp4")
           and not (sh != "g4" and kv == "f32")]


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("kv,shape", FORMATS, ids=lambda x: str(x))
def test_multi_token_partials_and_merge(layout, kv, shape):
    """T = 5 query tokens: ragged lengths, a request shorter than T (its first
    queries see nothing), and lengths whose last shard holds only new tokens,
    so that early queries get empty shards."""
    kvp, T = 4, 5
    S = 80 if layout in ("striped", "staggered16") else 192
    sh = dict(SHAPES[shape])
    q_dtype = "f32" if kv == "f32" else "bf16"
    w = _wl(kv, S=S, q_dtype=q_dtype, **sh)
    seqs = [(S * kvp, 3), (163, 66), (T, 1)]
    _check(w, T, layout, kvp, S, seqs, seed=7)


@pytest.mark.parametrize("layout", ["contiguous", "paged"])
@pytest.mark.parametrize("T", [3, 4])
def test_token_cut_at_shard_start(layout, T):
    """fp8, 16 query heads per KV head, 1024 shard units (the one-wave kernel
    that puts the query tokens in the matrix-core columns): lengths that put a
    shard boundary at a later token's cut, so that within one tile some token
    columns see no row while the others see one to three (their running max
    moves while the others' stays at -inf), and a request of T - 1 rows,
    whose first token sees nothing at all."""
    kvp, S = 64, 1024
    w = _wl("fp8", B=2, S=S, Hq=128, Hkv=8, D=128)
    # 16-row shards (the rounded-up share of at most 1024 rows): shard 40
    # starts at row 640
    seqs = [(640 + T - 1, T - 1), (640 + T - 2, 656)]
    _check(w, T, layout, kvp, S, seqs, seed=12)


@pytest.mark.parametrize("T", [1, 2, 16, 40])
def test_token_counts_gqa_fp8(T):
    """The matrix-core GQA kernel over token counts that leave the last group
    of 8 shard units partial (kvp * B * Hkv = 3 * 2 * 2 = 12) and T up to 40."""
    kvp, S = 3, 192
    w = _wl("fp8", S=S, Hq=32, Hkv=2, D=128)
    _check(w, T, "contiguous", kvp, S, [(192, 100), (41, 17)], seed=8)


def test_token_counts_valu_f32():
    kvp, S = 3, 160
    w = _wl("f32", S=S, Hq=12, Hkv=3, D=64, q_dtype="f32")
    for T in (3, 33):
        _check(w, T, "contiguous", kvp, S, [(160, 40)], seed=9)


@pytest.mark.parametrize("kv", ["bf16", "mxfp4"])
def test_token_counts_ring_formats(kv):
    """Odd token counts: bf16 runs them four to a workgroup with the LDS ring,
    MXFP4 two to a workgroup, here with S_max % 4 != 0 (scale rows of a slab
    not 16-byte aligned)."""
    kvp = 3
    S = 190 if kv == "mxfp4" else 192
    w = _wl(kv, S=S, Hq=32, Hkv=2, D=128)
    for T in (3, 9):
        _check(w, T, "contiguous", kvp, S, [(S, 77), (19, S - 1)], seed=11)


@pytest.mark.parametrize("layout", ["contiguous", "paged"])
@pytest.mark.parametrize("kv,T", [("fp8", 2), ("mxfp4", 2), ("bf16", 2), ("bf16", 4)])
def test_one_chunk_token_counts(layout, kv, T):
    """Token counts that one workgroup chunk covers (two tokens; four on the
    bf16 ring): those instances read the cache with non-temporal loads."""
    kvp = 3
    S = 192
    w = _wl(kv, S=S, Hq=32, Hkv=2, D=128)
    _check(w, T, layout, kvp, S, [(S * kvp, 70), (T, 1)], seed=12 + T)


def test_mla_multi_token_paged():
    kvp, T, S = 5, 3, 192
    w = _wl("bf16", S=S, **SHAPES["mla"])
    _check(w, T, "paged", kvp, S, [(S, 100)], seed=10)


@pytest.mark.parametrize("layout", ["contiguous", "striped", "staggered16", "paged"])
@pytest.mark.parametrize("kv", ["f32", "bf16", "fp8", "mxfp4"])
def test_append_tokens_bitexact(layout, kv):
    """T = 4 new tokens per request per call, bit for bit against the oracle
    encoder; a negative start skips the request, tokens past the end are
    skipped one by one."""
    import torch
    from long_context_decode_split_amd import kvd
    kvp, S, T, steps = 3, 32, 4, 12
    w = _wl(kv, B=3, Hq=8, Hkv=2, D=64 if kv != "mxfp4" else 128, S=S)
    rng = np.random.default_rng(31)
    extra, table_dev = {}, None
    if layout == "paged":
        bl, max_blocks = 16, 4
        num_blocks = w.B * max_blocks + 2
        table = rng.permutation(num_blocks)[:w.B * max_blocks].reshape(w.B, max_blocks).astype(np.int32)
        zero = _zero_cache(w, "contiguous", 1, 1)
        def pool(a):
            return None if a is None else np.zeros((num_blocks, w.Hkv, bl) + a.shape[3:], a.dtype)
        host = {"k": pool(zero["k"]), "v": pool(zero["v"]), "block_len": bl, "block_table": table}
        if kv == "mxfp4":
            host["k_scale"], host["v_scale"] = pool(zero["k_scale"]), pool(zero["v_scale"])
        else:
            host["k_scale"], host["v_scale"] = zero["k_scale"], zero["v_scale"]
        table_dev = _dev(table)
        extra = dict(block_len=bl, max_blocks=max_blocks, num_blocks=num_blocks, block_table=table_dev)
        cap = bl * max_blocks
    else:
        host = _zero_cache(w, layout, kvp, S)
        cap = S if layout == "contiguous" else kvp * S
    dev = {n: _dev(host[n]) for n in ("k", "k_scale", "v", "v_scale")}
    p = kvd.problem(w.B, w.Hq, w.Hkv, w.Dqk, w.Dv, S, kvp, w.q_dtype, w.kv_dtype, 0.0, False, layout=layout,
                    q_tokens=T, **extra)
    po = oracle.Problem(w.B, w.Hq, w.Hkv, w.Dqk, w.Dv, S, w.q_dtype, w.kv_dtype)
    for step in range(steps):
        kn = rng.standard_normal((w.B, T, w.Hkv, w.Dqk)).astype(np.float32)
        vn = rng.standard_normal((w.B, T, w.Hkv, w.Dv)).astype(np.float32)
        kn[0, 1, 0, :4] *= 1e3
        pos = np.array([T * step, -1 if step % 3 == 0 else cap - 2 - step, (7 * step) % cap], dtype=np.int32)
        op.append_tokens(po, T, layout, kvp, host, pos, kn, vn)
        kvd.kvd_append_kv(p, _dev(kn), _dev(vn), _dev(pos), (dev["k"], dev["k_scale"]), (dev["v"], dev["v_scale"]))
    torch.cuda.synchronize()
    for n in ("k", "v"):
        assert np.array_equal(_host(dev[n], host[n]).view(np.uint8), host[n].view(np.uint8)), (layout, kv, n)
        if kv == "mxfp4":
            assert np.array_equal(_host(dev[n + "_scale"], host[n + "_scale"]), host[n + "_scale"]), n
    gc.log("  append T=%d %s %s: %d calls bit-exact" % (T, layout, kv, steps))


def test_prefill_loop_matches_oracle():
    """A turn loop on an fp8 cache: each step appends T new tokens per request
    with kvd_append_kv and attends with the same T queries; every step
    matches the oracle run on its own copy of the cache."""
    import torch
    from long_context_decode_split_amd import kvd
    kvp, S, T = 4, 160, 6
    w = _wl("fp8", B=2, Hq=32, Hkv=2, D=128, S=S)
    inp = kvgen.make_inputs(w)
    host = {"k": inp.k_data.copy(), "k_scale": inp.k_scale, "v": inp.v_data.copy(), "v_scale": inp.v_scale}
    dev = {n: _dev(a) for n, a in host.items()}
    p = kvd.problem(w.B, w.Hq, w.Hkv, 128, 128, S, kvp, "bf16", "fp8", 0.0, False, q_tokens=T)
    po = oracle.Problem(w.B, w.Hq, w.Hkv, 128, 128, S, "bf16", "fp8")
    L = np.array([40, 3], dtype=np.int32)
    rng = np.random.default_rng(22)
    ws = torch.empty(kvd.kvd_decode_workspace_bytes(p), dtype=torch.uint8, device="cuda")
    o = torch.empty((w.B, T, w.Hq, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((w.B, T, w.Hq), dtype=torch.float32, device="cuda")
    for step in range(5):
        q = kvgen.gen_q(w.with_(q_tokens=T, seed=100 + step))
        kn = rng.standard_normal((w.B, T, w.Hkv, 128)).astype(np.float32)
        vn = rng.standard_normal((w.B, T, w.Hkv, 128)).astype(np.float32)
        op.append_tokens(po, T, "contiguous", kvp, host, L, kn, vn)
        kvd.kvd_append_kv(p, _dev(kn), _dev(vn), _dev(L), (dev["k"], dev["k_scale"]), (dev["v"], dev["v_scale"]))
        L = L + T
        kvd.kvd_decode(p, _dev(q), (dev["k"], dev["k_scale"]), (dev["v"], dev["v_scale"]), _dev(L), ws, o, lse)
        torch.cuda.synchronize()
        ref_o, ref_l = op.decode_tokens(po, T, "contiguous", kvp, q, host, L)
        gc.compare(o.cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, "fp8", "turn %d L=%s" % (step, tuple(L)))


def _full_size_tokens(name, kvp, T, n_pairs=2):
    """The full-size cache (generated on the device once) with T query tokens
    per request; the oracle runs on sampled (request, KV head) slabs, each as a
    one-request, one-KV-head problem regenerated on the host."""
    import torch
    from long_context_decode_split_amd import kvd
    from tests.test_gpu_parity import _device_inputs
    dev = _device_inputs(name)
    w = dev.workload
    wt = w.with_(q_tokens=T)
    q = kvgen.gen_q(wt)
    gc.log("%s T=%d kvp=%d: running the library" % (name, T, kvp))
    p = kvd.problem(w.B, w.Hq, w.Hkv, w.Dqk, w.Dv, w.S_max, kvp, w.q_dtype, w.kv_dtype, 0.0, w.v_aliases_k,
                    q_tokens=T)
    f32 = dict(dtype=torch.float32, device="cuda")
    o_part = torch.full((kvp, w.B, T, w.Hq, w.Dv), float("nan"), **f32)
    lse_part = torch.full((kvp, w.B, T, w.Hq), float("nan"), **f32)
    o = torch.full((w.B, T, w.Hq, w.Dv), float("nan"), **f32)
    lse = torch.full((w.B, T, w.Hq), float("nan"), **f32)
    qd = _dev(q)
    kvd.kvd_decode_partial(p, qd, dev.k, dev.v, dev.seq_lens, o_part, lse_part)
    kvd.kvd_lse_merge(kvp, w.B * T * w.Hq, w.Dv, o_part, lse_part, o, lse)
    torch.cuda.synchronize()
    o_part, lse_part, o, lse = (t.cpu().numpy() for t in (o_part, lse_part, o, lse))
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    seq = dev.seq_lens.cpu().numpy()
    G = w.G
    for (b, kvh) in gc.sampled_pairs(w, n_pairs):
        L = int(seq[b])
        gc.log("  oracle on request %d, KV head %d (L=%d, T=%d)" % (b, kvh, L, T))
        kd, ks = kvgen.gen_kv_slab(w, "k", b, kvh)
        vd, vs = kvgen.gen_kv_slab(w, "v", b, kvh)
        if w.kv_dtype == "fp8":
            ks, vs = np.asarray(ks).reshape(1, 1), np.asarray(vs).reshape(1, 1)
        else:
            ks, vs = ks[None, None], vs[None, None]
        cache = {"k": kd[None, None], "k_scale": ks, "v": vd[None, None], "v_scale": vs}
        hs = slice(kvh * G, (kvh + 1) * G)
        sub = oracle.Problem(1, G, 1, w.Dqk, w.Dv, w.S_max, w.q_dtype, w.kv_dtype)
        qs = np.ascontiguousarray(q[b:b + 1, :, hs])
        ro, rl = op.decode_tokens(sub, T, "contiguous", kvp, qs, cache, [L])
        rpo, rpl = op.decode_partials_tokens(sub, T, "contiguous", kvp, qs, cache, [L])
        what = "%s T=%d kvp=%d b=%d kvh=%d" % (name, T, kvp, b, kvh)
        gc.compare(o[b:b + 1, :, hs], lse[b:b + 1, :, hs], ro, rl, w.kv_dtype, what)
        gc.compare(o_part[:, b:b + 1, :, hs], lse_part[:, b:b + 1, :, hs], rpo, rpl, w.kv_dtype, what + " partials")


@pytest.mark.slow
@pytest.mark.parametrize("name,T", [("helix_fp8", 4), ("helix_mxfp4", 3)])
def test_full_size_multi_token(name, T):
    """The Helix shape at S = 2^20 with T query tokens, in the configuration
    bench.py --q-tokens times (kvp = 32)."""
    _full_size_tokens(name, 32, T)


def test_append_tokens_latent_alias():
    """T = 3 new latent rows per request (V aliases K): only K is written, bit
    for bit, on a staggered cache."""
    import torch
    from long_context_decode_split_amd import kvd
    T, kvp, S = 3, 2, 40
    w = _wl("bf16", B=2, Hq=128, Hkv=1, D=576, Dv=512, S=S, alias=True)
    host = _zero_cache(w, "staggered16", kvp, S)
    dk = _dev(host["k"])
    p = kvd.problem(w.B, w.Hq, 1, 576, 512, S, kvp, "bf16", "bf16", 0.0, True, layout="staggered16", q_tokens=T)
    po = oracle.Problem(w.B, w.Hq, 1, 576, 512, S, "bf16", "bf16", True)
    rng = np.random.default_rng(4)
    for step in range(8):
        kn = rng.standard_normal((w.B, T, 1, 576)).astype(np.float32)
        pos = np.array([T * step, 70 - T * step], dtype=np.int32)
        op.append_tokens(po, T, "staggered16", kvp, host, pos, kn, None)
        kvd.kvd_append_kv(p, _dev(kn), None, _dev(pos), (dk, None), None)
    torch.cuda.synchronize()
    assert np.array_equal(_host(dk, host["k"]), host["k"])
