"""The library's launches under HIP graph capture: a decode step (append the
new token, then partial pass and merge) captured once into a graph and
replayed, with eager work and synchronizations between the replays; every
replay must equal the eager result bit for bit.  The entry points allocate
nothing and clear nothing with memsets, so they can be captured as they are."""
import numpy as np
import pytest

import kvgen
from tests import gpu_cases as gc
from tests.test_gpu_cache import _dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kv,T", [("fp8", 1), ("mxfp4", 1), ("bf16", 4), ("f32", 2)])
def test_captured_decode_step_replays_like_eager(kv, T):
    import torch
    from long_context_decode_split_amd import kvd
    Hq, Hkv, D = (32, 2, 128) if kv != "f32" else (8, 1, 64)
    q_dtype = "f32" if kv == "f32" else "bf16"
    w = kvgen.Workload("graph_" + kv, B=2, Hq=Hq, Hkv=Hkv, Dqk=D, Dv=D, S_max=400, kvp=(5,), q_dtype=q_dtype,
                       kv_dtype=kv, seed=61, seq_lens=(380, 45), q_tokens=T)
    inp = kvgen.make_inputs(w)
    kvp = 5
    p = kvd.problem(w.B, w.Hq, w.Hkv, D, D, w.S_max, kvp, q_dtype, kv, q_tokens=T)
    q = _dev(inp.q)
    k = (_dev(inp.k_data), _dev(inp.k_scale))
    v = (_dev(inp.v_data), _dev(inp.v_scale))
    seq = _dev(inp.seq_lens.astype(np.int32))
    pos = _dev((inp.seq_lens - T).astype(np.int32))
    rng = np.random.default_rng(3)
    kn = _dev(rng.standard_normal((w.B, T, Hkv, D)).astype(np.float32))
    vn = _dev(rng.standard_normal((w.B, T, Hkv, D)).astype(np.float32))
    ws = torch.empty(kvd.kvd_decode_workspace_bytes(p), dtype=torch.uint8, device="cuda")
    o = torch.empty((w.B, T, w.Hq, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((w.B, T, w.Hq), dtype=torch.float32, device="cuda")

    def step():
        kvd.kvd_append_kv(p, kn, vn, pos, k, v)
        kvd.kvd_decode(p, q, k, v, seq, ws, o, lse)

    step()                                   # eager (also sets kernel attributes once)
    torch.cuda.synchronize()
    ref_o, ref_l = o.clone(), lse.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    torch.cuda.synchronize()
    for r in range(4):
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o) and torch.equal(lse, ref_l), "replay %d differs from eager" % r
        # eager work between the replays
        step()
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o) and torch.equal(lse, ref_l)
    gc.log("  graph %s T=%d: 4 replays equal to eager" % (kv, T))
