"""Roofline arithmetic against the numbers the pages print (CPU only)."""
import json
import os

import pytest

from long_context_decode_split_amd import roofline

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "pages_roofline.json")


def _fx():
    with open(GOLDEN) as f:
        return json.load(f)


def test_helix_figure1_kv_read():
    fx = _fx()["helix_figure1"]
    p = fx["params"]
    for row in fx["rows"]:
        t = roofline.helix_t_kv(p["B"], p["K"], row["TPA"], p["Hsz"], p["S"], row["KVP"],
                                p["bytes_param"], p["membw_bytes_per_s"])
        assert t * 1e6 == pytest.approx(row["kv_read_us"], rel=1e-9)


def test_helix_via_kv_bytes():
    """kv_bytes on one GPU's Helix share (1 KV head, TPA=8) reproduces t_kv's numerator (FP4, no scales)."""
    fx = _fx()["helix_figure1"]
    p = fx["params"]
    # one KV head per GPU; 0.5 B/elem is row_bytes('mxfp4') without its 1/32 scale term
    nbytes = roofline.kv_bytes(1, [p["S"]] * p["B"], p["Hsz"], p["Hsz"], "mxfp4", False)
    scale_bytes = p["B"] * p["S"] * 2 * p["Hsz"] / 32
    assert (nbytes - scale_bytes) / p["membw_bytes_per_s"] * 1e6 == pytest.approx(128.0, rel=1e-9)


@pytest.mark.parametrize("cp", [1, 2])
def test_survey_dcp_estimate(cp):
    fx = _fx()["survey_dcp"]
    p = fx["params"]
    ref = fx["cp%d" % cp]
    hkv_rank = p["h_kv"] // p["TP"]
    hq_rank = p["h_q"] // p["TP"]
    seq = [p["S"] // cp] * p["B"]
    nbytes = roofline.kv_bytes(hkv_rank, seq, p["d_h"], p["d_h"], "bf16", False)
    assert nbytes == ref["kv_bytes"]
    assert nbytes / p["hbm_bytes_per_s"] * 1e6 == pytest.approx(ref["scan_us"], abs=0.005)
    fl = roofline.attention_flops(hq_rank, seq, p["d_h"], p["d_h"])
    assert fl / 1e9 == pytest.approx(ref["gflop"], abs=0.05)
    assert fl / p["peak_flops"] * 1e6 == pytest.approx(ref["compute_us"], abs=0.005)


def test_row_bytes():
    assert roofline.row_bytes("mxfp4", 128) == 68
    assert roofline.row_bytes("fp8", 128) == 128
    assert roofline.kv_bytes(8, [1 << 20] * 8, 128, 128, "fp8", False) == 17179869184 + 8 * 8 * 8
    assert roofline.kv_bytes(1, [1 << 19] * 8, 576, 512, "bf16", True) == 4831838208


def test_multi_token_flops_count_each_visible_pair():
    # T = 3 queries over L = 5 tokens see 3, 4, 5 tokens; L = 1 sees 0, 0, 1
    fl = roofline.attention_flops_tokens(2, [5, 1], 3, 8, 4)
    assert fl == 2 * 2 * (3 + 4 + 5 + 0 + 0 + 1) * (8 + 4)
    assert roofline.attention_flops_tokens(7, [9, 4], 1, 16, 16) == roofline.attention_flops(7, [9, 4], 16, 16)
