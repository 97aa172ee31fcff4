"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Small cases compare every output and every shard partial element by element;
they span several tiles, ragged tails, empty requests and empty shards.  The
full-size workloads compare sampled (request, KV head) slabs, regenerated on
the host and run through the oracle, plus properties that hold at any size.
"""
import numpy as np
import pytest

import kvgen
from tests import gpu_cases as gc

pytestmark = pytest.mark.gpu


def W(name, **kw):
    base = dict(B=3, Hq=16, Hkv=2, Dqk=128, Dv=128, S_max=300, kvp=(4,), q_dtype="bf16",
                kv_dtype="bf16", seed=7, seq_lens=(300, 17, 129))
    base.update(kw)
    return kvgen.Workload(name, **base)


# ------------------------------------------------------------- small cases
def test_mqa_f32_workload():
    """The MQA fp32 workload (B=1, 8 heads on 1 KV head, Hsz=64, S=4096) at its KVP=4 and others."""
    w = kvgen.WORKLOADS["mqa_f32"]
    for kvp in (4, 1, 3, 16):
        gc.check_full(w, kvp)


SWEEP = []
for kv in ("f32", "bf16", "fp8", "mxfp4"):
    for D in (64, 128):
        if kv == "mxfp4" and D == 64:
            continue
        for G in (1, 4, 8, 16):
            SWEEP.append((kv, D, G))


@pytest.mark.parametrize("kv,D,G", SWEEP, ids=lambda x: str(x))
def test_sweep(kv, D, G):
    Hkv = 2
    for q_dtype in ("bf16", "f32"):
        w = W("sweep_%s_d%d_g%d_%s" % (kv, D, G, q_dtype), Hq=G * Hkv, Hkv=Hkv, Dqk=D, Dv=D,
              kv_dtype=kv, q_dtype=q_dtype, seq_lens=(300, 1, 17), seed=100 + G + D)
        for kvp in (1, 3, 16):
            gc.check_full(w, kvp)


@pytest.mark.parametrize("kv", ["f32", "bf16", "fp8", "mxfp4"])
def test_valu_full_grid(kv):
    """Grids of at least one workgroup per compute unit take the vector-ALU
    kernel's many-heads-per-workgroup variant (the small cases above take the
    one-head variant): 8 requests x 4 KV heads x 16 shards."""
    for D, G, q_dtype in ((64, 4, "bf16"), (128, 8, "f32"), (128, 16, "f32"), (128, 1, "bf16")):
        if kv == "mxfp4" and D == 64:
            continue
        w = W("valu_grid_%s_d%d_g%d" % (kv, D, G), B=8, Hq=G * 4, Hkv=4, Dqk=D, Dv=D, S_max=400, kv_dtype=kv,
              q_dtype=q_dtype, seq_lens=(400, 1, 17, 399, 0, 250, 33, 128), seed=300 + G + D)
        gc.check_full(w, 16)


@pytest.mark.parametrize("kv", ["bf16", "fp8", "mxfp4"])
def test_group16_long_ragged(kv):
    """G=16 at a few thousand tokens with lengths off every tile boundary."""
    w = W("g16_%s" % kv, B=2, Hq=32, Hkv=2, S_max=5000, seq_lens=(4999, 2049), kv_dtype=kv, seed=9)
    for kvp in (1, 7, 32):
        gc.check_full(w, kvp)


def test_mxfp4_scale_rows_not_16b_aligned():
    """S_max % 4 != 0 leaves each slab's E8M0 scale array off 16-byte (and
    4-byte) alignment; the kernels load scale bytes one per lane."""
    w = W("mxfp4_smax1001", B=2, Hq=32, Hkv=2, S_max=1001, seq_lens=(1001, 37), kv_dtype="mxfp4", seed=13)
    for kvp in (1, 3, 16):
        gc.check_full(w, kvp)


def test_lengths_at_tile_edges():
    for L in (1, 15, 16, 17, 31, 32, 33, 63, 64, 65):
        w = W("edge_%d" % L, B=1, Hq=16, Hkv=1, S_max=80, seq_lens=(L,), kv_dtype="bf16", seed=L)
        for kvp in (1, 2, 5):
            gc.check_full(w, kvp)


def test_empty_request_and_empty_shards():
    """seq_len 0 gives o = 0, lse = -inf; lengths below kvp*16 leave empty shards."""
    for kv in ("f32", "bf16", "fp8", "mxfp4"):
        w = W("empty_%s" % kv, B=3, Hq=16, Hkv=1, S_max=64, seq_lens=(0, 5, 40), kv_dtype=kv)
        gc.check_full(w, 16)
        gc.check_full(w, 128)


def test_poisoned_tail_is_never_read():
    """Tokens past each request's length hold NaN codes; outputs stay finite and exact."""
    for kv in ("f32", "bf16", "fp8", "mxfp4"):
        w = W("poison_%s" % kv, B=3, Hq=16, Hkv=1, S_max=200, seq_lens=(1, 77, 150), kv_dtype=kv)
        gc.check_full(w, 3, poison=True)


def test_v_aliases_k_square():
    w = W("alias", B=2, Hq=8, Hkv=1, Dqk=128, Dv=128, S_max=100, seq_lens=(100, 33),
          kv_dtype="bf16", v_aliases_k=True)
    gc.check_full(w, 3)


def test_mla_small():
    """Latent heads (128 per KV head, Dqk=576, V = first 512 columns of K), ragged and empty."""
    for kvh, seq in ((1, (300, 17, 0)), (2, (77, 300, 33))):
        w = W("mla_small_%d" % kvh, B=3, Hq=128 * kvh, Hkv=kvh, Dqk=576, Dv=512, S_max=300,
              seq_lens=seq, kv_dtype="bf16", v_aliases_k=True, seed=31 + kvh)
        for kvp in (1, 3, 16):
            gc.check_full(w, kvp)


def _ramp_inputs(w, growth):
    """Planted inputs whose logits grow along the sequence: every cached key
    is (t + 1) times one direction u and every query is a multiple of u, so the
    running max keeps rising by `growth` (in natural-log units) per token."""
    import numpy as np
    inp = kvgen.make_inputs(w)
    rng = np.random.default_rng(5)
    u = rng.standard_normal(w.Dqk)
    u /= np.linalg.norm(u)
    sm = 1.0 / np.sqrt(w.Dqk)
    t = np.arange(w.S_max, dtype=np.float64)
    k = (t[:, None] + 1.0) * u[None, :] * 0.05
    qv = u * growth / (sm * 0.05)
    def bf16(x):
        import torch
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    inp.k_data[...] = bf16(k)[None, None]
    inp.q[...] = bf16(np.broadcast_to(qv, inp.q.shape))
    return inp


@pytest.mark.parametrize("kind", ["gqa", "mla"])
def test_rising_logits(kind):
    """Logits that rise by ~0.3 nats per token (hundreds of nats per shard)
    exercise the running-max updates of the GQA kernel and the restart pass of
    the latent kernel; the result is dominated by the last tokens."""
    from kvgen.device import upload
    import oracle
    if kind == "gqa":
        w = W("ramp_gqa", B=1, Hq=16, Hkv=1, S_max=700, seq_lens=(700,), kv_dtype="bf16")
    else:
        w = W("ramp_mla", B=1, Hq=128, Hkv=1, Dqk=576, Dv=512, S_max=700, seq_lens=(700,),
              kv_dtype="bf16", v_aliases_k=True)
    inp = _ramp_inputs(w, 0.3)
    dev = upload(inp)
    for kvp in (1, 4):
        o_part, lse_part, o, lse = gc.run_library(dev, kvp)
        p = oracle.Problem.from_workload(w)
        args = (inp.q, inp.k_data, inp.k_scale, inp.v_data, inp.v_scale, inp.seq_lens)
        ref_po, ref_pl = oracle.decode_partials(p, kvp, *args)
        ref_o, ref_l = oracle.decode(p, *args)
        gc.compare(o_part, lse_part, ref_po, ref_pl, w.kv_dtype, "%s ramp kvp=%d partials" % (kind, kvp))
        gc.compare(o, lse, ref_o, ref_l, w.kv_dtype, "%s ramp kvp=%d merged" % (kind, kvp))


@pytest.mark.parametrize("B", [64, 65])
def test_many_requests_mixed_lengths(B):
    """Up to 64 requests the shard units are taken longest request first
    (ranked on the device, one lane per request); from 65 on in plain order.
    Both must give every request's exact partials, including repeated and
    zero lengths."""
    import numpy as np
    rng = np.random.default_rng(B)
    lens = [int(x) for x in rng.integers(0, 120, B)]
    lens[3] = lens[5] = 77          # ties
    lens[7] = 0                     # empty request
    w = W("many_%d" % B, B=B, Hq=16, Hkv=1, S_max=120, seq_lens=tuple(lens), kv_dtype="fp8", seed=B)
    for kvp in (1, 3):
        gc.check_full(w, kvp)


@pytest.mark.parametrize("kv", ["fp8", "mxfp4"])
def test_query_dynamic_range(kv):
    """Queries far from N(0, 1): per-head magnitudes from 2^-40 to 2^4, elements
    within a head spread over 2^-30 of the head's largest, a head of zeros and
    bf16 subnormals.  The fp8 and MXFP4 logits take the query as two E4M3
    parts with one exponent pair per head, exact above 2^-13 of the head's
    largest |q| and within 2^-21 of it below; every head must still match."""
    import numpy as np
    import torch
    from kvgen.device import upload
    import oracle
    w = W("qrange_%s" % kv, B=2, Hq=32, Hkv=2, S_max=300, seq_lens=(300, 77), kv_dtype=kv, seed=41)
    inp = kvgen.make_inputs(w)
    rng = np.random.default_rng(17)
    q = rng.standard_normal((w.B, w.Hq, w.Dqk))
    q *= np.exp2(-rng.uniform(0.0, 30.0, q.shape))            # spread inside each head
    q *= np.exp2(rng.uniform(-40.0, 4.0, (w.B, w.Hq, 1)))     # per-head magnitude
    q[0, 3] = 0.0                                              # all-zero head
    q[1, 5] = rng.standard_normal(w.Dqk) * 2.0 ** -130         # bf16 subnormals
    q[1, 6, :64] = 0.0                                         # half a head zero
    bits = torch.from_numpy(q.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    inp.q[...] = bits
    dev = upload(inp)
    p = oracle.Problem.from_workload(w)
    args = (inp.q, inp.k_data, inp.k_scale, inp.v_data, inp.v_scale, inp.seq_lens)
    for kvp in (1, 5):
        o_part, lse_part, o, lse = gc.run_library(dev, kvp)
        ref_po, ref_pl = oracle.decode_partials(p, kvp, *args)
        ref_o, ref_l = oracle.decode(p, *args)
        gc.compare(o_part, lse_part, ref_po, ref_pl, kv, "%s qrange kvp=%d partials" % (kv, kvp))
        gc.compare(o, lse, ref_o, ref_l, kv, "%s qrange kvp=%d merged" % (kv, kvp))


def test_repeat_runs_bitwise_identical():
    from kvgen.device import upload
    w = W("det", kv_dtype="fp8", S_max=2000, seq_lens=(2000, 1999, 1000))
    dev = upload(kvgen.make_inputs(w))
    a = gc.run_library(dev, 8)
    b = gc.run_library(dev, 8)
    for x, y in zip(a, b):
        assert np.array_equal(x, y, equal_nan=True)


# -------------------------------------------------- full-size workloads
_DEV_CACHE = {}


def _device_inputs(name):
    from kvgen.device import generate_on_device
    import torch
    if name not in _DEV_CACHE:
        _DEV_CACHE.clear()
        torch.cuda.empty_cache()
        gc.log("generating %s on the host, slab by slab" % name)
        _DEV_CACHE[name] = generate_on_device(kvgen.WORKLOADS[name], progress=gc.log)
    return _DEV_CACHE[name]


def _check_sampled(name, kvp, n_pairs=3):
    dev = _device_inputs(name)
    w = dev.workload
    gc.log("%s kvp=%d: running the library" % (name, kvp))
    o_part, lse_part, o, lse = gc.run_library(dev, kvp)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    # any-size property: merged lse >= every shard lse, and equals their log-sum-exp
    lp = lse_part.astype(np.float64)
    assert (lse[None] >= np.where(np.isfinite(lp), lp, -np.inf) - 1e-4).all()
    q_np = dev.q.cpu().numpy()
    if w.q_dtype == "bf16":
        q_np = q_np.view(np.uint16)
    seq = dev.seq_lens.cpu().numpy()
    G = w.G
    for (b, kvh) in gc.sampled_pairs(w, n_pairs):
        gc.log("  oracle on request %d, KV head %d (L=%d)" % (b, kvh, seq[b]))
        ro, rl, parts = gc.oracle_slab(w, b, kvh, seq[b], q_np, kvp)
        hs = slice(kvh * G, (kvh + 1) * G)
        gc.compare(o[b, hs], lse[b, hs], ro, rl, w.kv_dtype, "%s kvp=%d b=%d kvh=%d" % (name, kvp, b, kvh))
        po = np.stack([p_[0] for p_ in parts])
        pl = np.stack([p_[1] for p_ in parts])
        gc.compare(o_part[:, b, hs], lse_part[:, b, hs], po, pl, w.kv_dtype,
                   "%s kvp=%d b=%d kvh=%d partials" % (name, kvp, b, kvh))


# Planted peak logits (nats) per query head of the peaked check, in turn; 0
# keeps the generated query.  With N(0,1) keys at these widths the other
# logits are N(0, (peak / |k[s*]|)^2), so over 2^19..2^20 tokens the planted
# token carries from about half (15) to all but ~e^-13 (30) of the weight.
PEAKS = (0.0, 15.0, 20.0, 30.0)


def _check_peaked(name, kvp, n_pairs=2):
    """The full-size cache with the softmax concentrated on one cached token
    per query head: for the heads of the sampled (request, KV head) slabs the
    query becomes beta k[s*] for a seeded position s*, with beta chosen so that
    the planted logit sm_scale q.k[s*] is 15, 20 or 30 nats (one head in four
    keeps its N(0,1) query).  Outputs are then O(1) (a few cached values
    dominate), so the absolute output bound is a tight check; the shards
    without s* still see N(0,1) logits."""
    import dataclasses
    import torch
    import oracle
    dev = _device_inputs(name)
    w = dev.workload
    assert w.q_dtype == "bf16" and w.q_tokens == 1
    seq = dev.seq_lens.cpu().numpy()
    q_np = dev.q.cpu().numpy().view(np.uint16).copy()
    sm = oracle.default_scale(w.Dqk)
    rng = np.random.default_rng(2024 + kvp)
    pairs = gc.sampled_pairs(w, n_pairs, seed=kvp)
    G = w.G
    for (b, kvh) in pairs:
        kd, ks = kvgen.gen_kv_slab(w, "k", b, kvh)
        L = int(seq[b])
        for i in range(G):
            peak = PEAKS[i % len(PEAKS)]
            if peak == 0.0:
                continue
            s = int(rng.integers(L))
            sc = ks if w.kv_dtype in ("fp8", "bf16", "f32") else ks[s:s + 1]
            krow = oracle.dequant(w.kv_dtype, kd[s:s + 1], sc, w.Dqk)[0]
            beta = peak / (sm * float(krow @ krow))
            q_np[b, kvh * G + i] = torch.from_numpy((krow * beta).astype(np.float32)).to(
                torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    dev_p = dataclasses.replace(dev, q=torch.from_numpy(q_np.view(np.int16)).cuda())
    gc.log("%s kvp=%d peaked: running the library" % (name, kvp))
    o_part, lse_part, o, lse = gc.run_library(dev_p, kvp)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    for (b, kvh) in pairs:
        gc.log("  oracle on request %d, KV head %d (L=%d), peaked queries" % (b, kvh, seq[b]))
        ro, rl, parts = gc.oracle_slab(w, b, kvh, seq[b], q_np, kvp)
        hs = slice(kvh * G, (kvh + 1) * G)
        assert np.abs(ro).max() > 0.5, "planted peaks should give O(1) outputs"
        gc.compare(o[b, hs], lse[b, hs], ro, rl, w.kv_dtype, "%s kvp=%d b=%d kvh=%d peaked" % (name, kvp, b, kvh))
        po = np.stack([p_[0] for p_ in parts])
        pl = np.stack([p_[1] for p_ in parts])
        gc.compare(o_part[:, b, hs], lse_part[:, b, hs], po, pl, w.kv_dtype,
                   "%s kvp=%d b=%d kvh=%d peaked partials" % (name, kvp, b, kvh))


@pytest.mark.slow
def test_full_gqa_bf16_varlen():
    _check_sampled("gqa_bf16_varlen", 16)
    _check_peaked("gqa_bf16_varlen", 16)


@pytest.mark.slow
@pytest.mark.parametrize("kvp", [8, 32, 128])
def test_full_helix_fp8(kvp):
    _check_sampled("helix_fp8", kvp, n_pairs=2)
    _check_peaked("helix_fp8", kvp)


@pytest.mark.slow
@pytest.mark.parametrize("kvp", [8, 32, 128])
def test_full_helix_mxfp4(kvp):
    _check_sampled("helix_mxfp4", kvp, n_pairs=2)
    _check_peaked("helix_mxfp4", kvp)


@pytest.mark.slow
@pytest.mark.parametrize("kvp", [32, 128])
def test_full_gqa8_fp8(kvp):
    """Eight query heads per KV head at S = 2^20 (fp8): the matrix-core kernel
    with half of its 16 head columns padded."""
    _check_sampled("gqa8_fp8", kvp, n_pairs=2)
    _check_peaked("gqa8_fp8", kvp)


@pytest.mark.slow
@pytest.mark.parametrize("name", ["mxfp4_b1_s256k", "mxfp4_b32_s256k"])
def test_full_mxfp4_batch_sweep(name):
    _check_sampled(name, 32, n_pairs=2)


@pytest.mark.slow
@pytest.mark.parametrize("name", ["helix_shard_fp8", "helix_shard_mxfp4"])
def test_full_helix_shard(name):
    """One GPU's share of the Helix shape (Hkv=1, 16 heads, S/8 tokens), split 64 ways."""
    _check_sampled(name, 64, n_pairs=2)


@pytest.mark.slow
def test_full_mla_bf16():
    from long_context_decode_split_amd import kvd
    w = kvgen.WORKLOADS["mla_bf16"]
    p = gc.problem_of(w, 32)
    import ctypes
    if kvd.lib().kvd_decode_workspace_bytes(ctypes.byref(p)) == 0:
        pytest.fail("invalid MLA problem")
    _check_sampled("mla_bf16", 32, n_pairs=2)
    _check_peaked("mla_bf16", 32, n_pairs=1)
