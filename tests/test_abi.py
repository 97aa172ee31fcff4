"""The C ABI: the library loads, exports what include/kvd.h declares, and
rejects malformed calls on the host before enqueueing anything (CPU only:
none of these calls reaches a kernel launch)."""
import ctypes
import os
import re
import subprocess

import pytest

from long_context_decode_split_amd import kvd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvd.h")

FAKE = 1 << 40          # 16-byte aligned, never dereferenced by these tests
INV, UNS = kvd.KVD_ERR_INVALID, kvd.KVD_ERR_UNSUPPORTED

# These calls pass fake device addresses that host validation must reject.
# Keep them off machines with a GPU, where a validation bug would launch a
# kernel on them.
import torch  # noqa: E402

pytestmark = pytest.mark.skipif(torch.cuda.device_count() > 0,
                                reason="fake device pointers: run on a host without a GPU")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvd_[a-z_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert header_functions() == sorted(kvd.EXPORTED)


def test_library_exports_every_declared_symbol():
    out = subprocess.check_output(["nm", "-D", "--defined-only", kvd.LIB_PATH], text=True)
    syms = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in header_functions():
        assert name in syms, name
        assert hasattr(kvd.lib(), name)


def test_abi_version_and_strings():
    assert kvd.kvd_abi_version() == kvd.ABI_VERSION == 5
    for s in range(4):
        assert kvd.kvd_status_string(s).startswith(("KVD_OK", "KVD_ERR"))
    assert "unknown" in kvd.kvd_status_string(99)


def good_problem(**kw):
    base = dict(B=2, Hq=32, Hkv=2, Dqk=128, Dv=128, S_max=1024, kvp=4, q_dtype="bf16", kv_dtype="fp8")
    base.update(kw)
    return kvd.problem(**base)


def call_partial(p, q=FAKE, k=(FAKE, FAKE), v=(FAKE, FAKE), seq=FAKE, o=FAKE, lse=FAKE):
    L = kvd.lib()
    return L.kvd_decode_partial(ctypes.byref(p) if p is not None else None, q, kvd._kv(k), kvd._kv(v),
                                seq, o, lse, None)


def call_decode(p, ws=FAKE, o=FAKE, lse=FAKE, k=(FAKE, FAKE), v=(FAKE, FAKE)):
    L = kvd.lib()
    return L.kvd_decode(ctypes.byref(p), FAKE, kvd._kv(k), kvd._kv(v), FAKE, ws, o, lse, None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), INV), (dict(Hq=0), INV), (dict(Hkv=0), INV), (dict(Dqk=0), INV), (dict(Dv=-1), INV),
    (dict(Hq=31), INV),                     # not a multiple of Hkv
    (dict(S_max=0), INV), (dict(kvp=0), INV), (dict(kvp=5000), INV),
    (dict(q_dtype=7), INV), (dict(kv_dtype=9), INV), (dict(q_dtype="fp8"), INV),
    (dict(sm_scale=-1.0), INV), (dict(sm_scale=float("inf")), INV), (dict(sm_scale=float("nan")), INV),
    (dict(kv_dtype="mxfp4", Dqk=48, Dv=48), INV),
    (dict(layout=3), INV), (dict(layout=-1), INV),
    (dict(q_tokens=-1), INV), (dict(q_tokens=65537), INV),
    (dict(q_tokens=65536, kvp=4096, B=64), UNS),         # too many workgroups
    (dict(Dqk=96, Dv=96), UNS),             # well formed, no kernel for this width
    (dict(Dqk=128, Dv=64), UNS),
])
def test_partial_rejects_bad_problem(kw, status):
    assert call_partial(good_problem(**kw)) == status
    assert kvd.kvd_last_error() != ""


def test_null_problem():
    assert kvd.lib().kvd_decode_partial(None, FAKE, kvd._kv((FAKE, FAKE)), kvd._kv((FAKE, FAKE)),
                                        FAKE, FAKE, FAKE, None) == INV


@pytest.mark.parametrize("args", [
    dict(q=None), dict(q=FAKE + 8), dict(k=(None, FAKE)), dict(k=(FAKE + 4, FAKE)),
    dict(k=(FAKE, None)),                   # fp8 needs scales
    dict(v=(None, FAKE)), dict(v=(FAKE, None)), dict(v=(FAKE + 2, FAKE)),
    dict(seq=None), dict(seq=FAKE + 2), dict(o=None), dict(o=FAKE + 4), dict(lse=None),
    dict(lse=FAKE + 1), dict(k=(FAKE, FAKE + 1)),
])
def test_partial_rejects_bad_pointers(args):
    assert call_partial(good_problem(), **args) == INV


def test_scale_must_be_null_for_plain_formats():
    assert call_partial(good_problem(kv_dtype="bf16")) == INV            # scales given
    assert call_partial(good_problem(kv_dtype="bf16"), k=(FAKE, None), v=(FAKE, FAKE)) == INV


def test_alias_rules():
    p = good_problem(kv_dtype="bf16", v_aliases_k=True, Dqk=576, Dv=512, Hkv=1, Hq=128)
    assert call_partial(p, k=(FAKE, None), v=(FAKE, None)) == INV        # v must be NULL
    p = good_problem(kv_dtype="bf16", v_aliases_k=True, Dqk=64, Dv=128)
    assert call_partial(p, k=(FAKE, None), v=(None, None)) == INV        # Dv > Dqk


def test_merge_validation():
    L = kvd.lib()
    assert L.kvd_lse_merge(0, 8, 128, FAKE, FAKE, FAKE, FAKE, None) == INV
    assert L.kvd_lse_merge(4, -1, 128, FAKE, FAKE, FAKE, FAKE, None) == INV
    assert L.kvd_lse_merge(4, 8, 126, FAKE, FAKE, FAKE, FAKE, None) == INV
    assert L.kvd_lse_merge(4, 8, 128, None, FAKE, FAKE, FAKE, None) == INV
    assert L.kvd_lse_merge(4, 8, 128, FAKE + 4, FAKE, FAKE, FAKE, None) == INV
    assert L.kvd_lse_merge(4, 8, 128, FAKE, FAKE + 1, FAKE, FAKE, None) == INV
    # zero rows is a valid no-op that launches nothing
    assert L.kvd_lse_merge(4, 0, 128, None, None, None, None, None) == kvd.KVD_OK


def test_workspace_bytes():
    p = good_problem(kvp=8)
    n = kvd.kvd_decode_workspace_bytes(p)
    o_bytes = 8 * 2 * 32 * 128 * 4
    lse_bytes = 8 * 2 * 32 * 4
    assert n == -(-o_bytes // 256) * 256 + -(-lse_bytes // 256) * 256
    assert kvd.kvd_decode_workspace_bytes(good_problem(B=0)) == 0
    # T query tokens: T times the rows; q_tokens = 0 means one token
    assert kvd.kvd_decode_workspace_bytes(good_problem(kvp=8, q_tokens=0)) == n
    t5 = kvd.kvd_decode_workspace_bytes(good_problem(kvp=8, q_tokens=5))
    assert t5 == -(-5 * o_bytes // 256) * 256 + -(-5 * lse_bytes // 256) * 256


def test_decode_validation_happens_before_launch():
    assert call_decode(good_problem(), ws=None) == INV
    assert call_decode(good_problem(), ws=FAKE + 8) == INV
    assert call_decode(good_problem(), o=None) == INV
    assert call_decode(good_problem(Dqk=96, Dv=96)) == UNS


def test_binding_raises_with_message():
    with pytest.raises(kvd.KvdError) as ei:
        kvd.kvd_decode_partial(good_problem(B=0), FAKE, (FAKE, FAKE), (FAKE, FAKE), FAKE, FAKE, FAKE, stream=0)
    assert ei.value.status == INV and "B, Hq" in ei.value.message


def test_binding_refuses_host_tensors():
    import torch
    with pytest.raises(ValueError):
        kvd._ptr(torch.zeros(4))


def call_append(p, k_new=FAKE, v_new=FAKE, pos=FAKE, k=(FAKE, FAKE), v=(FAKE, FAKE)):
    return kvd.lib().kvd_append_kv(ctypes.byref(p), k_new, v_new, pos, kvd._kv(k), kvd._kv(v), None)


@pytest.mark.parametrize("args", [
    dict(k_new=None), dict(k_new=FAKE + 2), dict(v_new=None), dict(v_new=FAKE + 1),
    dict(pos=None), dict(pos=FAKE + 2), dict(k=(None, FAKE)), dict(k=(FAKE, None)),
    dict(v=(FAKE + 4, FAKE)), dict(v=(FAKE, None)),
])
def test_append_rejects_bad_pointers(args):
    for layout in ("contiguous", "striped", "staggered16"):
        assert call_append(good_problem(layout=layout), **args) == INV


def test_append_alias_and_problem_rules():
    p = good_problem(kv_dtype="bf16", v_aliases_k=True, Dqk=576, Dv=512, Hkv=1, Hq=128)
    assert call_append(p, k=(FAKE, None), v=(None, None)) == INV          # v_new must be NULL
    assert call_append(good_problem(layout=7)) == INV
    assert call_append(good_problem(B=0)) == INV


@pytest.mark.parametrize("kw", [
    dict(block_len=8), dict(block_len=24), dict(block_len=0), dict(block_len=1 << 21),
    dict(max_blocks=0), dict(num_blocks=0), dict(block_table=None), dict(block_table=FAKE + 2),
])
def test_paged_problem_validation(kw):
    base = dict(layout="paged", block_len=16, max_blocks=8, num_blocks=32, block_table=FAKE)
    base.update(kw)
    assert call_partial(good_problem(**base)) == INV
    assert call_append(good_problem(**base)) == INV
    assert kvd.kvd_decode_workspace_bytes(good_problem(**base)) == 0


def test_problem_struct_matches_header(tmp_path):
    """The binding's kvd_problem has the C struct's size and field offsets
    (compiled against include/kvd.h with the host compiler)."""
    fields = [f[0] for f in kvd.KvdProblem._fields_]
    src = tmp_path / "layout.c"
    src.write_text('#include <stddef.h>\n#include <stdio.h>\n#include "kvd.h"\nint main(void) {\n'
                   '  printf("size %zu\\n", sizeof(kvd_problem));\n' +
                   "".join('  printf("%s %%zu\\n", offsetof(kvd_problem, %s));\n' % (f, f) for f in fields) +
                   "  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.check_call(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)])
    got = dict(line.split() for line in subprocess.check_output([str(exe)], text=True).splitlines())
    assert int(got["size"]) == ctypes.sizeof(kvd.KvdProblem)
    for f in fields:
        assert int(got[f]) == getattr(kvd.KvdProblem, f).offset, f
