"""The C ABI from plain C: long_context_decode_split_amd/examples/decode_from_c
(built by __graft_entry__.build()) allocates its own device buffers, runs
kvd_decode and writes o and lse; they must match the oracle.  The program
runs as a child process of the test, on the same GPU."""
import os
import subprocess

import numpy as np
import pytest

import kvgen
import oracle
from oracle import passq as op
from tests import gpu_cases as gc

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "long_context_decode_split_amd", "examples", "decode_from_c")
CODES = {"f32": 0, "bf16": 1, "fp8": 2, "mxfp4": 3}


def _run_c(tmp_path, w, kvp, T, inp, q):
    d = str(tmp_path)
    with open(os.path.join(d, "problem.txt"), "w") as f:
        f.write("%d %d %d %d %d %d %d %d %d %d\n" % (w.B, w.Hq, w.Hkv, w.Dqk, w.Dv, w.S_max, kvp,
                                                   CODES[w.q_dtype], CODES[w.kv_dtype], T))
    def put(name, a):
        if a is not None:
            np.ascontiguousarray(a).tofile(os.path.join(d, name))
    put("q.bin", q)
    put("k.bin", inp.k_data)
    put("k_scale.bin", inp.k_scale)
    put("v.bin", inp.v_data)
    put("v_scale.bin", inp.v_scale)
    put("seq_lens.bin", inp.seq_lens.astype(np.int32))
    gc.log("  running %s on %s" % (os.path.basename(EXE), w.name))
    r = subprocess.run([EXE, d], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    o = np.fromfile(os.path.join(d, "o.bin"), dtype=np.float32).reshape(w.B, T, w.Hq, w.Dv)
    lse = np.fromfile(os.path.join(d, "lse.bin"), dtype=np.float32).reshape(w.B, T, w.Hq)
    return o, lse


CASES = {
    "gqa_fp8": dict(B=2, Hq=32, Hkv=2, Dqk=128, Dv=128, S_max=300, kv_dtype="fp8", q_dtype="bf16",
                    seq_lens=(300, 77)),
    "mqa_f32": dict(B=1, Hq=8, Hkv=1, Dqk=64, Dv=64, S_max=512, kv_dtype="f32", q_dtype="f32", seq_lens=(500,)),
    "mxfp4": dict(B=2, Hq=16, Hkv=1, Dqk=128, Dv=128, S_max=256, kv_dtype="mxfp4", q_dtype="bf16",
                  seq_lens=(256, 3)),
    "latent": dict(B=2, Hq=128, Hkv=1, Dqk=576, Dv=512, S_max=160, kv_dtype="bf16", q_dtype="bf16",
                   seq_lens=(160, 45), v_aliases_k=True),
}


@pytest.mark.skipif(not os.path.exists(EXE), reason="the C example is built by __graft_entry__.build()")
@pytest.mark.parametrize("name", sorted(CASES))
@pytest.mark.parametrize("T", [1, 3])
def test_decode_from_c(tmp_path, name, T):
    w = kvgen.Workload("c_" + name, kvp=(4,), seed=51, **CASES[name])
    inp = kvgen.make_inputs(w)
    q = kvgen.gen_q(w.with_(q_tokens=T))
    o, lse = _run_c(tmp_path, w, 4, T, inp, q)
    p = oracle.Problem.from_workload(w)
    cache = {"k": inp.k_data, "k_scale": inp.k_scale, "v": inp.v_data, "v_scale": inp.v_scale}
    ro, rl = op.decode_tokens(p, T, "contiguous", 4, q, cache, inp.seq_lens)
    gc.compare(o, lse, ro, rl, w.kv_dtype, "decode_from_c %s T=%d" % (name, T))
