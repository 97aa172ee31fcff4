"""Helpers shared by the GPU parity tests: run the library, run the oracle, compare."""
from __future__ import annotations

import math
import sys

import numpy as np

import kvgen
import oracle

# Tolerances: max abs error on o and on lse, and relative RMS of o.
TOL = {
    "f32": dict(o=1e-4, lse=1e-5, rrms=1e-5),
    "bf16": dict(o=2e-3, lse=1e-3, rrms=1e-2),
    "fp8": dict(o=2e-3, lse=1e-3, rrms=1e-2),
    "mxfp4": dict(o=2e-3, lse=1e-3, rrms=1e-2),
}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def problem_of(w, kvp):
    from long_context_decode_split_amd import kvd
    return kvd.problem(w.B, w.Hq, w.Hkv, w.Dqk, w.Dv, w.S_max, kvp, w.q_dtype, w.kv_dtype, 0.0, w.v_aliases_k)


def run_library(dev, kvp, partials=True):
    """o_part, lse_part, o, lse (numpy float32) from kvd_decode_partial + kvd_lse_merge,
    and o2, lse2 from kvd_decode; checks the two agree bitwise."""
    import torch
    from long_context_decode_split_amd import kvd
    w = dev.workload
    p = problem_of(w, kvp)
    f32 = dict(dtype=torch.float32, device="cuda")
    o_part = torch.full((kvp, w.B, w.Hq, w.Dv), float("nan"), **f32)
    lse_part = torch.full((kvp, w.B, w.Hq), float("nan"), **f32)
    o = torch.full((w.B, w.Hq, w.Dv), float("nan"), **f32)
    lse = torch.full((w.B, w.Hq), float("nan"), **f32)
    kvd.kvd_decode_partial(p, dev.q, dev.k, dev.v, dev.seq_lens, o_part, lse_part)
    kvd.kvd_lse_merge(kvp, w.B * w.Hq, w.Dv, o_part, lse_part, o, lse)
    ws = torch.empty(kvd.kvd_decode_workspace_bytes(p), dtype=torch.uint8, device="cuda")
    o2 = torch.full_like(o, float("nan"))
    lse2 = torch.full_like(lse, float("nan"))
    kvd.kvd_decode(p, dev.q, dev.k, dev.v, dev.seq_lens, ws, o2, lse2)
    torch.cuda.synchronize()
    res = [t.cpu().numpy() for t in (o_part, lse_part, o, lse, o2, lse2)]
    assert np.array_equal(res[2], res[4], equal_nan=True), "kvd_decode differs from partial+merge"
    assert np.array_equal(res[3], res[5], equal_nan=True), "kvd_decode lse differs from partial+merge"
    return res[:4]


def compare(got_o, got_lse, ref_o, ref_lse, kv_dtype, what):
    """Element-wise comparison with the dtype's tolerances; -inf lse must match exactly."""
    tol = TOL[kv_dtype]
    got_o = np.asarray(got_o, dtype=np.float64)
    got_lse = np.asarray(got_lse, dtype=np.float64)
    assert got_o.shape == ref_o.shape and got_lse.shape == ref_lse.shape, what
    assert np.isfinite(got_o).all(), "%s: non-finite o" % what
    empty = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(got_lse), empty), "%s: empty-shard pattern differs" % what
    assert (got_o[empty] == 0).all(), "%s: empty shard output not zero" % what
    fin = ~empty
    err_o = np.max(np.abs(got_o - ref_o)) if got_o.size else 0.0
    err_l = np.max(np.abs(got_lse[fin] - ref_lse[fin])) if fin.any() else 0.0
    nrm = np.linalg.norm(ref_o)
    rrms = np.linalg.norm(got_o - ref_o) / nrm if nrm > 0 else np.linalg.norm(got_o)
    log("  %-40s max|do|=%.3g max|dlse|=%.3g rel_rms=%.3g" % (what, err_o, err_l, rrms))
    assert err_o <= tol["o"], "%s: max |o err| %.3g > %.3g" % (what, err_o, tol["o"])
    assert err_l <= tol["lse"], "%s: max |lse err| %.3g > %.3g" % (what, err_l, tol["lse"])
    assert rrms <= tol["rrms"], "%s: relative rms %.3g > %.3g" % (what, rrms, tol["rrms"])


def check_full(w, kvp, poison=False):
    """Whole problem: library vs oracle on every output and every shard partial."""
    from kvgen.device import upload
    inp = kvgen.make_inputs(w)
    if poison:
        kvgen.poison_tail(inp)
    dev = upload(inp)
    o_part, lse_part, o, lse = run_library(dev, kvp)
    p = oracle.Problem.from_workload(w)
    args = (inp.q, inp.k_data, inp.k_scale, inp.v_data, inp.v_scale, inp.seq_lens)
    ref_po, ref_pl = oracle.decode_partials(p, kvp, *args)
    ref_o, ref_l = oracle.decode(p, *args)
    compare(o_part, lse_part, ref_po, ref_pl, w.kv_dtype, "%s kvp=%d partials" % (w.name, kvp))
    compare(o, lse, ref_o, ref_l, w.kv_dtype, "%s kvp=%d merged" % (w.name, kvp))


def sampled_pairs(w, n, seed=0):
    rng = np.random.default_rng(seed)
    pairs = {(0, 0), (w.B - 1, w.Hkv - 1)}
    while len(pairs) < min(n, w.B * w.Hkv):
        pairs.add((int(rng.integers(w.B)), int(rng.integers(w.Hkv))))
    return sorted(pairs)


def oracle_slab(w, b, kvh, seq_len, q_np, kvp=None):
    """Oracle results for every head of one (request, KV head), regenerating
    only that slab: (o [G,Dv], lse [G]) and optionally shard partials."""
    kd, ks = kvgen.gen_kv_slab(w, "k", b, kvh)
    if w.v_aliases_k:
        vd, vs = None, None
    else:
        vd, vs = kvgen.gen_kv_slab(w, "v", b, kvh)
    L = int(seq_len)
    G = w.G
    qf = oracle.q_to_f64(q_np[b, kvh * G:(kvh + 1) * G], w.q_dtype)
    sm = oracle.default_scale(w.Dqk)

    def rows(lo, hi):
        if w.kv_dtype == "mxfp4":
            k = oracle.dequant("mxfp4", kd[lo:hi], ks[lo:hi], w.Dqk)
            v = k[:, :w.Dv] if w.v_aliases_k else oracle.dequant("mxfp4", vd[lo:hi], vs[lo:hi], w.Dv)
        else:
            k = oracle.dequant(w.kv_dtype, kd[lo:hi], ks, w.Dqk)
            v = k[:, :w.Dv] if w.v_aliases_k else oracle.dequant(w.kv_dtype, vd[lo:hi], vs, w.Dv)
        return k, v

    k, v = rows(0, L)
    o, lse = oracle.attend(qf, k, v, sm)
    parts = None
    if kvp is not None:
        parts = []
        for (s, e) in oracle.split_ranges(L, kvp):
            parts.append(oracle.attend(qf, k[s:e], v[s:e], sm))
    return o, lse, parts
