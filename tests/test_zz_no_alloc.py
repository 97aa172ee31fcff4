"""kvd_decode_noalloc (partials in the library's static device array) against
kvd_decode (partials in a caller workspace): identical results bit for bit on
consecutive calls, the second smaller than the first (what it reads must be
what that call wrote, not what the larger call left behind), and problems too
large for the static array refused before anything is enqueued."""
import numpy as np
import pytest

import kvgen
from tests import gpu_cases as gc

pytestmark = pytest.mark.gpu


def _decode_pair(w, kvp, T=1):
    """(o, lse) of kvd_decode and of kvd_decode_noalloc on the same inputs."""
    import torch
    from kvgen.device import upload
    from long_context_decode_split_amd import kvd
    w = w.with_(q_tokens=T)
    dev = upload(kvgen.make_inputs(w))
    p = kvd.problem(w.B, w.Hq, w.Hkv, w.Dqk, w.Dv, w.S_max, kvp, w.q_dtype, w.kv_dtype, 0.0, w.v_aliases_k,
                    q_tokens=T)
    assert kvd.kvd_decode_workspace_bytes(p) <= kvd.NOALLOC_SCRATCH_BYTES
    f32 = dict(dtype=torch.float32, device="cuda")
    ws = torch.empty(kvd.kvd_decode_workspace_bytes(p), dtype=torch.uint8, device="cuda")
    o1 = torch.full((w.B, T, w.Hq, w.Dv), float("nan"), **f32)
    l1 = torch.full((w.B, T, w.Hq), float("nan"), **f32)
    o2 = torch.full_like(o1, float("nan"))
    l2 = torch.full_like(l1, float("nan"))
    kvd.kvd_decode(p, dev.q, dev.k, dev.v, dev.seq_lens, ws, o1, l1)
    kvd.kvd_decode_noalloc(p, dev.q, dev.k, dev.v, dev.seq_lens, o2, l2)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in (o1, l1, o2, l2)]


def _same(w, kvp, T=1):
    o1, l1, o2, l2 = _decode_pair(w, kvp, T)
    gc.log("  noalloc %s kvp=%d T=%d: %d outputs" % (w.name, kvp, T, o1.size))
    assert np.array_equal(o1, o2, equal_nan=True), "o differs from kvd_decode"
    assert np.array_equal(l1, l2, equal_nan=True), "lse differs from kvd_decode"
    assert np.isfinite(o2).all()


def test_noalloc_equals_workspace_decode_large_then_small():
    big = kvgen.Workload("noalloc_big", B=4, Hq=64, Hkv=4, Dqk=128, Dv=128, S_max=3000, kvp=(64,),
                         q_dtype="bf16", kv_dtype="fp8", seed=91, seq_lens=(3000, 2500, 17, 0))
    small = kvgen.Workload("noalloc_small", B=2, Hq=32, Hkv=2, Dqk=128, Dv=128, S_max=400, kvp=(3,),
                           q_dtype="bf16", kv_dtype="mxfp4", seed=92, seq_lens=(400, 33))
    _same(big, 64)
    _same(small, 3)
    # other kernel families, each after a larger call
    _same(kvgen.WORKLOADS["mqa_f32"], 4)
    latent = kvgen.Workload("noalloc_latent", B=2, Hq=128, Hkv=1, Dqk=576, Dv=512, S_max=500, kvp=(5,),
                            q_dtype="bf16", kv_dtype="bf16", seed=93, seq_lens=(500, 61), v_aliases_k=True)
    _same(latent, 5, T=2)
    _same(small.with_(name="noalloc_small_t3"), 2, T=3)


def test_noalloc_refuses_oversized_problem():
    """kvp * B * Hq * (Dv + 1) floats beyond the static array: KVD_ERR_UNSUPPORTED,
    nothing enqueued (the outputs keep their contents)."""
    import torch
    from long_context_decode_split_amd import kvd
    w = kvgen.Workload("noalloc_huge", B=8, Hq=128, Hkv=8, Dqk=128, Dv=128, S_max=64, kvp=(256,),
                       q_dtype="bf16", kv_dtype="fp8", seed=94)
    p = kvd.problem(w.B, w.Hq, w.Hkv, 128, 128, 64, 256, "bf16", "fp8")
    assert kvd.kvd_decode_workspace_bytes(p) > kvd.NOALLOC_SCRATCH_BYTES
    from kvgen.device import upload
    dev = upload(kvgen.make_inputs(w))
    o = torch.full((w.B, w.Hq, 128), 7.0, dtype=torch.float32, device="cuda")
    lse = torch.full((w.B, w.Hq), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(kvd.KvdError) as ei:
        kvd.kvd_decode_noalloc(p, dev.q, dev.k, dev.v, dev.seq_lens, o, lse)
    assert ei.value.status == kvd.KVD_ERR_UNSUPPORTED
    assert "static array" in ei.value.message
    torch.cuda.synchronize()
    assert (o == 7.0).all().item() and (lse == 7.0).all().item()
