"""The seeded input generator: determinism, slicing, encoders (CPU only)."""
import numpy as np
import pytest

import kvgen


def test_slices_equal_whole_and_thread_independent():
    whole = kvgen.normals_f64(11, 1, 0, 100_003, threads=1)
    for start, n in ((0, 17), (1, 1), (999, 5000), (50_001, 50_002)):
        part = kvgen.normals_f64(11, 1, start, n, threads=3)
        assert np.array_equal(part, whole[start:start + n])
    assert np.array_equal(kvgen.normals_f64(11, 1, 0, 100_003, threads=7), whole)


def test_streams_and_seeds_differ():
    a = kvgen.normals_f64(1, 0, 0, 1000)
    assert not np.array_equal(a, kvgen.normals_f64(1, 1, 0, 1000))
    assert not np.array_equal(a, kvgen.normals_f64(2, 0, 0, 1000))


def test_moments():
    z = kvgen.normals_f64(3, 2, 0, 2_000_000)
    assert abs(z.mean()) < 3e-3
    assert abs(z.var() - 1) < 5e-3
    assert abs((z ** 4).mean() - 3) < 3e-2


def test_f32_bf16_are_roundings_of_the_stream():
    import torch
    z = kvgen.normals_f64(5, 1, 0, 10_000)
    f = kvgen.normals_f32(5, 1, 0, 10_000)
    assert np.array_equal(f, z.astype(np.float32))
    b = kvgen.normals_bf16(5, 1, 0, 10_000)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b, ref)


def test_e4m3_encoder_matches_torch_rne():
    import torch
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(20000) * 50, rng.standard_normal(5000) * 0.01,
                        np.array([0.0, -0.0, 447.9, 448.0, -448.0, 2.0 ** -10, 3 * 2.0 ** -10])]).astype(np.float32)
    v = v[np.abs(v) <= 448]
    ours = kvgen.encode_e4m3(v)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)
    # saturation beyond the largest normal
    assert kvgen.encode_e4m3(np.array([1e6, -500.0], dtype=np.float32)).tolist() == [0x7E, 0xFE]


def test_e2m1_encoder_rne_ties_and_roundtrip():
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert kvgen.encode_e2m1(np.array(grid)).tolist() == list(range(8))
    assert kvgen.encode_e2m1(-np.array(grid[1:])).tolist() == list(range(9, 16))
    ties = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    # ties go to the even code: 0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0
    assert kvgen.encode_e2m1(np.array(ties)).tolist() == [0, 2, 2, 4, 4, 6, 6]
    assert kvgen.encode_e2m1(np.array([7.0, 100.0])).tolist() == [7, 7]


def test_fp8_slab_scale_and_codes():
    codes, scales = kvgen.fp8_slabs(9, 1, 0, 3, 4096)
    f = kvgen.normals_f32(9, 1, 0, 3 * 4096).reshape(3, 4096)
    amax = np.abs(f).max(axis=1)
    assert np.array_equal(scales, (amax / np.float32(448)).astype(np.float32))
    # the largest magnitude maps to (or next to) the top code
    top = np.max(codes.reshape(3, 4096) & 0x7F, axis=1)
    assert (top >= 0x7D).all()
    # slab s regenerated alone is identical
    c1, s1 = kvgen.fp8_slabs(9, 1, 1, 1, 4096)
    assert np.array_equal(c1, codes[4096:8192]) and s1[0] == scales[1]


def test_mxfp4_block_exponent_rule():
    D = 64
    data, sc = kvgen.mxfp4_rows(4, 2, 0, 100, D)
    f = kvgen.normals_f32(4, 2, 0, 100 * D).reshape(100, D // 32, 32)
    amax = np.abs(f).max(axis=2).astype(np.float64)
    expect = np.clip(np.floor(np.log2(amax)).astype(int) - 2 + 127, 0, 254)
    assert np.array_equal(sc.reshape(100, D // 32), expect)
    d2, s2 = kvgen.mxfp4_rows(4, 2, 37, 5, D)
    assert np.array_equal(d2, data[37 * 32:42 * 32]) and np.array_equal(s2, sc[37 * 2:42 * 2])


def test_seq_lens_uniform_range():
    s = kvgen.uniform_int(1002, 3, 10000, 65536, 131072)
    assert s.min() >= 65536 and s.max() <= 131072
    assert abs(s.mean() - (65536 + 131072) / 2) < 1000
    w = kvgen.WORKLOADS["gqa_bf16_varlen"]
    sl = kvgen.gen_seq_lens(w)
    assert sl.shape == (8,) and (sl >= 65536).all() and (sl <= 131072).all()


@pytest.mark.parametrize("kv", ["f32", "bf16", "fp8", "mxfp4"])
def test_slab_generation_matches_whole(kv):
    w = kvgen.Workload("t", B=2, Hq=4, Hkv=2, Dqk=64, Dv=64, S_max=48, kvp=(2,), q_dtype="bf16",
                       kv_dtype=kv, seed=77)
    inp = kvgen.make_inputs(w)
    for b in range(2):
        for h in range(2):
            for which, data, scale in (("k", inp.k_data, inp.k_scale), ("v", inp.v_data, inp.v_scale)):
                d, s = kvgen.gen_kv_slab(w, which, b, h)
                assert np.array_equal(d, data[b, h])
                if kv == "fp8":
                    assert s == scale[b, h]
                elif kv == "mxfp4":
                    assert np.array_equal(s, scale[b, h])


def test_poison_tail():
    w = kvgen.Workload("t", B=2, Hq=2, Hkv=1, Dqk=32, Dv=32, S_max=40, kvp=(2,), q_dtype="f32",
                       kv_dtype="fp8", seed=5, seq_lens=(40, 17))
    inp = kvgen.poison_tail(kvgen.make_inputs(w))
    assert (inp.k_data[1, :, 17:] == 0x7F).all() and (inp.k_data[1, :, :17] != 0x7F).all()
    assert (inp.v_data[0] != 0x7F).all()


def test_encoders_of_given_values_match_generated_encodings():
    """encode_fp8_slab / encode_mxfp4 of the stream's fp32 values reproduce the
    generator's own fp8 slab and MXFP4 rows byte for byte (planted inputs are
    encoded by the same rules as generated ones)."""
    seed, stream, S, D = 77, 1, 96, 128
    vals = kvgen.normals_f32(seed, stream, 0, S * D).reshape(S, D)
    codes, scale = kvgen.fp8_slabs(seed, stream, 0, 1, S * D)
    c2, s2 = kvgen.encode_fp8_slab(vals)
    assert np.float32(s2) == scale[0]
    assert np.array_equal(c2.ravel(), codes)
    data, sc = kvgen.mxfp4_rows(seed, stream, 0, S, D)
    d2, sc2 = kvgen.encode_mxfp4(vals)
    assert np.array_equal(d2.ravel(), data) and np.array_equal(sc2.ravel(), sc)


def test_pack_mxfp4_nibble_order_and_zero_block():
    codes = np.arange(64, dtype=np.uint8).reshape(2, 32) % 16
    data, sc = kvgen.pack_mxfp4(codes, [[254], [0]])
    assert data.shape == (2, 16) and sc.tolist() == [[254], [0]]
    assert data[0, 0] == (0 | (1 << 4)) and data[1, 7] == (14 | (15 << 4))
    d0, s0 = kvgen.encode_mxfp4(np.zeros((1, 64), np.float32))
    assert (d0 == 0).all() and (s0 == 127).all()
