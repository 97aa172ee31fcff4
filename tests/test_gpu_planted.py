"""GPU parity on planted inputs that N(0,1) caches never produce.

* Logits that rise along the sequence, so every kernel instance moves its
  running max past the first tile: the one-token matrix-core GQA kernel on
  bf16, fp8 and MXFP4 caches; its two-token register ring (fp8, MXFP4, bf16
  T = 2) with one and with several token chunks; the one-wave two-token
  chunks of fp8 and MXFP4 caches (T = 2 to 4); the four-token LDS ring of
  the bf16 cache; the latent kernel and the vector-ALU kernel; contiguous
  and paged caches.
* MXFP4 block exponents far from 127 in K and in V, and all-zero blocks at
  the extreme exponents.
* fp8 scales that are negative or zero.
* Latent-cache values beyond fp16's range.

Every case compares every shard partial and the merged output with the
float64 oracle at the format's tolerances (the exactness of the split is the
"Sharding the sequence instead" section of the Helix article: each shard's
partial plus its log-sum-exp reproduce the full softmax with no
approximation).
"""
import numpy as np
import pytest

import kvgen
import oracle
from oracle import passq as op
from tests import gpu_cases as gc
from tests.test_gpu_cache import _paged_from_contiguous
from tests.test_gpu_passq import _run

pytestmark = pytest.mark.gpu


def _bf16_bits(x):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _wl(kv, T, B=2, Hq=32, Hkv=2, D=128, Dv=None, S=704, alias=False, seq=None, seed=5, q_dtype="bf16"):
    Dv = D if Dv is None else Dv
    seq = (S,) * B if seq is None else seq
    return kvgen.Workload("planted_%s" % kv, B=B, Hq=Hq, Hkv=Hkv, Dqk=D, Dv=Dv, S_max=S, kvp=(4,),
                          q_dtype=q_dtype, kv_dtype=kv, seed=seed, seq_lens=tuple(seq), v_aliases_k=alias,
                          q_tokens=T)


def _encode_rows(w, x):
    """(data, scale) of one (request, KV head) slab of K rows x [S, D] in w's format."""
    if w.kv_dtype == "bf16":
        return _bf16_bits(x), None
    if w.kv_dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32), None
    if w.kv_dtype == "fp8":
        return kvgen.encode_fp8_slab(x)
    return kvgen.encode_mxfp4(x)


def _ramp(w, growth, seed=5):
    """Inputs whose logits grow by about `growth` nats per token: key t of
    every slab is (t + 1) c u for one unit direction u (encoded to the cache
    format), every query is u growth / (sm_scale c), V is the generated cache.
    Returns (Inputs, q [B,T,Hq,Dqk])."""
    inp = kvgen.make_inputs(w)
    rng = np.random.default_rng(seed)
    u = rng.standard_normal(w.Dqk)
    u /= np.linalg.norm(u)
    c = 0.05
    sm = 1.0 / np.sqrt(w.Dqk)
    t = np.arange(w.S_max, dtype=np.float64)
    k = ((t[:, None] + 1.0) * c * u[None, :]).astype(np.float32)
    data, scale = _encode_rows(w, k)
    for b in range(w.B):
        for h in range(w.Hkv):
            inp.k_data[b, h] = data
            if w.kv_dtype == "fp8":
                inp.k_scale[b, h] = scale
            elif w.kv_dtype == "mxfp4":
                inp.k_scale[b, h] = scale
    qv = u * growth / (sm * c)
    T = w.q_tokens
    q = np.broadcast_to(qv, (w.B, T, w.Hq, w.Dqk))
    q = q.astype(np.float32) if w.q_dtype == "f32" else _bf16_bits(q)
    return inp, np.ascontiguousarray(q)


def _check_inputs(w, inp, q, layout, kvp, seqs, seed=3, scale_o=1.0):
    """Library vs oracle for explicit inputs (contiguous, or scattered into a
    scrambled paged pool of 16-token blocks).  scale_o divides every output
    before the comparison (a power of two, so the check is exact scaling)."""
    T = w.q_tokens
    S = w.S_max
    if layout == "paged":
        cache, nb = _paged_from_contiguous(w, inp, 16, S // 16, np.random.default_rng(seed))
        cache["num_blocks"] = nb
    else:
        cache = {"k": inp.k_data, "k_scale": inp.k_scale, "v": inp.v_data, "v_scale": inp.v_scale}
    p = oracle.Problem(w.B, w.Hq, w.Hkv, w.Dqk, w.Dv, S, w.q_dtype, w.kv_dtype, w.v_aliases_k)
    for seq in seqs:
        seq = np.asarray(seq, dtype=np.int32)
        what = "%s %s G=%d T=%d kvp=%d L=%s" % (layout, w.kv_dtype, w.G, T, kvp, tuple(int(x) for x in seq))
        gc.log("  case " + what)
        o_part, lse_part, o, lse = _run(w, T, layout, kvp, S, q, cache, seq)
        ref_po, ref_pl = op.decode_partials_tokens(p, T, layout, kvp, q, cache, seq)
        ref_o, ref_l = op.decode_tokens(p, T, layout, kvp, q, cache, seq)
        gc.compare(o_part / scale_o, lse_part, ref_po / scale_o, ref_pl, w.kv_dtype, what + " partials")
        gc.compare(o / scale_o, lse, ref_o / scale_o, ref_l, w.kv_dtype, what + " merged")


# Token counts per format and the instance each one selects: T = 1 the
# one-token kernel; fp8 / MXFP4 T = 2 one two-token chunk (non-temporal
# loads), T = 3 two chunks (the second with one token, plain loads); bf16
# T = 2 the two-token register ring, T = 3 one four-token LDS-ring chunk,
# T = 5 two of them.
RAMP_CASES = [(kv, T, lay) for kv in ("bf16", "fp8", "mxfp4") for T in (1, 2, 3, 5)
              for lay in ("contiguous", "paged") if not (kv != "bf16" and T == 5 and lay == "paged")]


@pytest.mark.parametrize("kv,T,layout", RAMP_CASES, ids=lambda x: str(x))
def test_rising_logits_gqa(kv, T, layout):
    """Logits rising ~0.3 nats per token (~10 per 32-token tile, more than the
    2^8 lazy-max margin in the exp2 domain), so the running max of every wave
    moves at every tile; lengths off the tile grid give masked last tiles."""
    w = _wl(kv, T)
    inp, q = _ramp(w, 0.3)
    _check_inputs(w, inp, q, layout, 4, [(700, 333), (545, 700)])
    _check_inputs(w, inp, q, layout, 1, [(700, 61)])


@pytest.mark.parametrize("kv,G", [("fp8", 8), ("mxfp4", 4), ("bf16", 1)])
@pytest.mark.parametrize("T", [1, 2])
def test_rising_logits_small_groups(kv, G, T):
    """Groups of fewer than 16 query heads on the matrix-core kernel (padded
    head columns): rising logits, contiguous cache."""
    w = _wl(kv, T, Hq=2 * G, Hkv=2)
    inp, q = _ramp(w, 0.3)
    _check_inputs(w, inp, q, "contiguous", 4, [(700, 333)])


@pytest.mark.parametrize("T", [1, 2])
def test_rising_logits_latent(T):
    """The latent kernel's restart pass (a later tile beyond its first tile's
    max by more than 2^64 in the exp2 domain) with one and two query tokens,
    on a paged cache."""
    w = _wl("bf16", T, B=1, Hq=128, Hkv=1, D=576, Dv=512, S=704, alias=True)
    inp, q = _ramp(w, 0.3)
    _check_inputs(w, inp, q, "paged", 3, [(700,)])


@pytest.mark.parametrize("layout", ["contiguous", "paged"])
def test_latent_values_beyond_fp16(layout):
    """The latent kernel takes V into its PV product as fp16; V elements of
    magnitude 2^18 .. 2^19 (beyond fp16's range) in the column slices of
    three of its four waves make it rerun the shard with those waves' V
    scaled by a power of two.  The queries are zero on the planted dims, so
    the logits are those of the generated cache; the planted columns are
    compared after division by 2^19, the others as they are."""
    import numpy as np
    w = _wl("bf16", 1, B=2, Hq=128, Hkv=1, D=576, Dv=512, S=704, alias=True, seed=81)
    inp = kvgen.make_inputs(w)
    q = np.ascontiguousarray(inp.q.reshape(w.B, 1, w.Hq, w.Dqk)).copy()
    big = np.array([5, 300, 511])
    q[..., big] = 0
    rng = np.random.default_rng(4)
    for b in range(w.B):
        rows = rng.choice(w.S_max, size=40, replace=False)
        vals = rng.choice([-1.0, 1.0], size=(40, 3)) * rng.uniform(2.0 ** 18, 2.0 ** 19, size=(40, 3))
        inp.k_data[b, 0][np.ix_(rows, big)] = _bf16_bits(vals)
    normal = np.setdiff1d(np.arange(w.Dv), big)
    T, S = 1, w.S_max
    if layout == "paged":
        cache, nb = _paged_from_contiguous(w, inp, 16, S // 16, np.random.default_rng(3))
        cache["num_blocks"] = nb
    else:
        cache = {"k": inp.k_data, "k_scale": inp.k_scale, "v": inp.v_data, "v_scale": inp.v_scale}
    p = oracle.Problem(w.B, w.Hq, w.Hkv, w.Dqk, w.Dv, S, w.q_dtype, w.kv_dtype, w.v_aliases_k)
    for kvp, seq in ((1, (704, 333)), (3, (700, 64))):
        seq = np.asarray(seq, dtype=np.int32)
        what = "%s latent big-V kvp=%d L=%s" % (layout, kvp, tuple(int(x) for x in seq))
        gc.log("  case " + what)
        o_part, lse_part, o, lse = _run(w, T, layout, kvp, S, q, cache, seq)
        ref_po, ref_pl = op.decode_partials_tokens(p, T, layout, kvp, q, cache, seq)
        ref_o, ref_l = op.decode_tokens(p, T, layout, kvp, q, cache, seq)
        for got, gl, ref, rl, tag in ((o_part, lse_part, ref_po, ref_pl, "partials"), (o, lse, ref_o, ref_l, "merged")):
            gc.compare(got[..., normal], gl, ref[..., normal], rl, "bf16", what + " " + tag + " other columns")
            gc.compare(got[..., big] / 2.0 ** 19, gl, ref[..., big] / 2.0 ** 19, rl, "bf16",
                       what + " " + tag + " planted columns / 2^19")


@pytest.mark.parametrize("kv", ["f32", "fp8"])
def test_rising_logits_valu(kv):
    """The vector-ALU kernel (4 query heads per KV head)."""
    w = _wl(kv, 2, Hq=8, Hkv=2, D=64, q_dtype="f32" if kv == "f32" else "bf16")
    inp, q = _ramp(w, 0.3)
    _check_inputs(w, inp, q, "contiguous", 4, [(700, 333)])


# ------------------------------------------------------------ E8M0 range
def _mx_inputs(T, seed):
    w = _wl("mxfp4", T, S=300, seq=(300, 77), seed=seed)
    return w, kvgen.make_inputs(w)


@pytest.mark.parametrize("T", [1, 2])
def test_mxfp4_key_exponents_far_from_127(T):
    """K block exponents shifted by +100 (E ~ 224..229) on KV head 0 and by
    -100 (E ~ 24..29) on KV head 1, with the queries of each group scaled by
    the inverse power of two: the logits are those of the unshifted cache, so
    the outputs are O(1) and the usual tolerances apply.  The matrix core
    applies the stored exponents; the two-part query's exponents stay inside
    their range."""
    w, inp = _mx_inputs(T, 51)
    ks = inp.k_scale.astype(np.int64)
    ks[:, 0] += 100
    ks[:, 1] -= 100
    assert ks.min() >= 1 and ks.max() <= 254
    inp.k_scale[...] = ks.astype(np.uint8)
    q = oracle.bf16_to_f64(inp.q).reshape(w.B, T, w.Hq, w.Dqk)
    q[:, :, :16] *= 2.0 ** -100
    q[:, :, 16:] *= 2.0 ** 100
    q = _bf16_bits(q)
    for kvp in (1, 5):
        _check_inputs(w, inp, q, "contiguous", kvp, [(300, 77)])


@pytest.mark.parametrize("T", [1, 2])
@pytest.mark.parametrize("shift", [40, -40, 20, -30])
def test_mxfp4_value_exponents_far_from_127(T, shift):
    """V block exponents shifted by `shift` on every token of KV head 0 and on
    every other 16-token run of KV head 1 (tiles mixing shifted and plain
    rows): outputs scale by 2^shift exactly, so they are compared after
    dividing by it (the KV head 1 rows mix scales and are compared at the
    same scale: their outputs are dominated by neither)."""
    w, inp = _mx_inputs(T, 52 + shift)
    vs = inp.v_scale.astype(np.int64)
    vs[:, 0] += shift
    runs = (np.arange(w.S_max) // 16) % 2 == 1
    vs[:, 1, runs] += shift
    assert vs.min() >= 1 and vs.max() <= 254
    inp.v_scale[...] = vs.astype(np.uint8)
    q = np.ascontiguousarray(inp.q.reshape(w.B, T, w.Hq, w.Dqk))
    # the KV head 0 outputs are 2^shift times O(1) values; compare that group
    # alone after scaling, and the mixed group alone at a scale that bounds it
    w0 = w.with_(Hq=16, Hkv=1)
    sub0 = kvgen.Inputs(w0, q[:, :, :16].copy(), inp.k_data[:, :1].copy(), inp.k_scale[:, :1].copy(),
                        inp.v_data[:, :1].copy(), inp.v_scale[:, :1].copy(), inp.seq_lens)
    sub1 = kvgen.Inputs(w0, q[:, :, 16:].copy(), inp.k_data[:, 1:].copy(), inp.k_scale[:, 1:].copy(),
                        inp.v_data[:, 1:].copy(), inp.v_scale[:, 1:].copy(), inp.seq_lens)
    for kvp in (1, 4):
        _check_inputs(w0, sub0, sub0.q, "contiguous", kvp, [(300, 77)], scale_o=2.0 ** shift)
        _check_inputs(w0, sub1, sub1.q, "contiguous", kvp, [(300, 77)], scale_o=2.0 ** max(shift, 0))


@pytest.mark.parametrize("T", [1, 2])
def test_mxfp4_zero_blocks_at_extreme_exponents(T):
    """All-zero E2M1 blocks (+0 and -0 codes) carrying E8M0 exponents 0, 1,
    200 and 254 in K and V contribute exactly nothing; blocks with E = 0 and
    nonzero codes (values of order 2^-127) contribute almost nothing.  The
    rest of the cache is the generated one."""
    w, inp = _mx_inputs(T, 53)
    rng = np.random.default_rng(9)
    for name_d, name_s, D in (("k_data", "k_scale", w.Dqk), ("v_data", "v_scale", w.Dv)):
        data = getattr(inp, name_d)
        sc = getattr(inp, name_s)
        nblk = D // 32
        for b in range(w.B):
            for h in range(w.Hkv):
                rows = rng.choice(w.S_max, size=w.S_max // 3, replace=False)
                for r in rows:
                    blk = int(rng.integers(nblk))
                    zero = rng.integers(2) == 0
                    fill = 0x00 if zero else 0x88            # +0 / -0 nibbles
                    data[b, h, r, blk * 16:(blk + 1) * 16] = fill
                    sc[b, h, r, blk] = rng.choice([0, 1, 200, 254])
                tiny = rng.choice(w.S_max, size=20, replace=False)
                sc[b, h, tiny, 0] = 0                        # nonzero codes, E = 0
    q = np.ascontiguousarray(inp.q.reshape(w.B, T, w.Hq, w.Dqk))
    for kvp in (1, 4):
        _check_inputs(w, inp, q, "contiguous", kvp, [(300, 77)])


# ------------------------------------------------------------- fp8 scales
@pytest.mark.parametrize("shape", ["g16", "g4"])
@pytest.mark.parametrize("T", [1, 2])
def test_fp8_negative_and_zero_scales(shape, T):
    """Element value = code x scale for any fp32 scale: negative K scales flip
    the sign of every logit of their slab (so the running max comes from the
    other end of the raw products), a zero K scale gives equal logits (the
    mean of V), negative and zero V scales flip or zero the output."""
    Hq, Hkv, D = (32, 2, 128) if shape == "g16" else (8, 2, 64)
    w = _wl("fp8", T, B=3, Hq=Hq, Hkv=Hkv, D=D, S=300, seq=(300, 77, 5), seed=61)
    inp = kvgen.make_inputs(w)
    inp.k_scale[0, 0] *= -1.0
    inp.k_scale[1, 1] = 0.0
    inp.k_scale[2, 0] *= -1.0
    inp.v_scale[0, 1] *= -1.0
    inp.v_scale[1, 0] = 0.0
    inp.v_scale[2, 1] *= -1.0
    q = np.ascontiguousarray(inp.q.reshape(w.B, T, w.Hq, w.Dqk))
    for kvp in (1, 4, 32):
        _check_inputs(w, inp, q, "contiguous", kvp, [(300, 77, 5)])


# ------------------------------------------------------- many shard units
@pytest.mark.parametrize("kv", ["bf16", "fp8", "mxfp4"])
@pytest.mark.parametrize("layout", ["contiguous", "paged"])
@pytest.mark.parametrize("S", [2048, 8192])
def test_one_wave_shard_groups(kv, layout, S):
    """From 1024 (fp8) or 2048 (MXFP4) shard units on, the one-token GQA kernel
    gives each wave a group of consecutive shards of one (request, KV head):
    when every shard length of the request is a multiple of the 32-token tile
    the group is streamed as one run of tokens with each shard's partial
    written at its boundary, otherwise shard by shard.  S = 2048 gives
    16-token shards (shard by shard), S = 8192 runs of 32- and 64-token
    shards next to 16-token ones; with empty shards, an empty request and
    groups cut short by kvp."""
    w = _wl(kv, 1, B=4, Hq=8 * 16, Hkv=8, S=S, seq=(S, S - 49, 37, 0), seed=71)
    inp = kvgen.make_inputs(w)
    q = np.ascontiguousarray(inp.q.reshape(w.B, 1, w.Hq, w.Dqk))
    for kvp in (128, 200, 256):
        _check_inputs(w, inp, q, layout, kvp, [(S, S - 49, 37, 0), (S // 2, S, 0, 33)])


# fp8 from 1024 shard units on (4 requests x 8 KV heads x kvp 64 / 100 at
# S = 4096: 64- and 48-token shards), MXFP4 from 8192 (kvp 256 / 300 at
# S = 16384: 64-token shards)
TOKEN_CHUNK_CASES = [("fp8", lay, T) for lay in ("contiguous", "paged") for T in (2, 3, 4)] + [
    ("mxfp4", "contiguous", 2), ("mxfp4", "paged", 3), ("mxfp4", "contiguous", 4)]


@pytest.mark.parametrize("kv,layout,T", TOKEN_CHUNK_CASES, ids=lambda x: str(x))
def test_one_wave_token_chunks(kv, layout, T):
    """With enough shard units, two to four query tokens of an fp8 or MXFP4
    cache run one wave per (shard, chunk of two tokens), the chunks of a shard
    in one workgroup.  Rising logits (the running max of every token moves at
    every tile), ragged and empty shards, an empty request."""
    S, kvps = (4096, (64, 100)) if kv == "fp8" else (16384, (256, 300))
    w = _wl(kv, T, B=4, Hq=8 * 16, Hkv=8, S=S, seq=(S, S - 49, 37, 0), seed=73)
    inp, q = _ramp(w, 0.3, seed=9)
    for kvp in kvps:
        _check_inputs(w, inp, q, layout, kvp, [(S, S - 49, 37, 0)])
