"""Host-side checks of bench.py's bookkeeping (no GPU): the recorded counter
tables are keyed on sources that exist, every kernel family has its
arithmetic and dtype strings, and a changed kernel source changes the key."""
import os

import bench


def test_kernel_sources_exist():
    csrc = os.path.join(bench.HERE, "long_context_decode_split_amd", "csrc")
    for fam, names in bench.KERNEL_SOURCES.items():
        for n in names + ("kvd_device.hpp",):
            assert os.path.exists(os.path.join(csrc, n)), (fam, n)


def test_every_family_is_described():
    for fam in ("f32", "bf16", "fp8", "fp8_tokens", "mxfp4", "latent"):
        assert bench.ARITH[fam] and bench.DTYPE[fam]


def test_recorded_counters_match_a_hash_form():
    for table in (bench.TRAFFIC, bench.MFMA_BUSY):
        for key in table:
            assert len(key) == 5 and len(key[4]) == 16 and int(key[4], 16) >= 0


def test_hash_ignores_comments_only(tmp_path, monkeypatch):
    # a copy of the sources with one comment changed hashes the same; one
    # code token changed hashes differently
    import shutil
    src = os.path.join(bench.HERE, "long_context_decode_split_amd", "csrc")
    dst = tmp_path / "long_context_decode_split_amd" / "csrc"
    shutil.copytree(src, dst)
    monkeypatch.setattr(bench, "HERE", str(tmp_path))
    h0 = bench.kernel_hash("fp8")
    p = dst / "gqa_mfma_kernel.hpp"
    text = p.read_text()
    p.write_text(text.replace("// Split-KV partial attention", "// Split-KV  partial attention (edited)", 1))
    assert bench.kernel_hash("fp8") == h0
    p.write_text(text.replace("constexpr float kLazyMax = 8.0f;", "constexpr float kLazyMax = 9.0f;", 1))
    assert bench.kernel_hash("fp8") != h0
