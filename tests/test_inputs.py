"""Seeded input generator: E4M3 encoding, block scales, routing (CPU only)."""
import numpy as np
import pytest
import torch

from moe_grouped_gemm_block_amd import inputs as I


def torch_decode(codes):
    """Library decode of E4M3FN bytes (independent of the generator)."""
    t = torch.from_numpy(np.asarray(codes, np.uint8).copy())
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


FINITE = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)


def test_roundtrip_all_finite_codes():
    vals = torch_decode(FINITE)
    back = I.encode_e4m3(vals)
    np.testing.assert_array_equal(back, FINITE)


def test_matches_library_cast_in_range():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(200_000).astype(np.float32) * 30,
        rng.uniform(-448, 448, 100_000).astype(np.float32),
        (rng.standard_normal(100_000) * 1e-3).astype(np.float32),   # subnormal range
    ])
    ours = I.encode_e4m3(x.astype(np.float64))
    lib = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(ours, lib)


def test_ties_to_even_at_every_midpoint():
    pos = np.array([c for c in range(0x7F)], np.uint8)          # 0 .. 448
    v = torch_decode(pos)
    mids = (v[:-1] + v[1:]) / 2                                   # exact in float64
    got = I.encode_e4m3(mids)
    lo, hi = pos[:-1], pos[1:]
    want = np.where(lo % 2 == 0, lo, hi)                         # even mantissa wins
    np.testing.assert_array_equal(got, want)
    np.testing.assert_array_equal(I.encode_e4m3(-mids), want | 0x80)


def test_saturation_and_signed_zero():
    assert I.encode_e4m3(np.array([448.0]))[0] == 0x7E
    assert I.encode_e4m3(np.array([463.9, 464.0, 1e9]))[:].tolist() == [0x7E] * 3
    assert I.encode_e4m3(np.array([-1e30]))[0] == 0xFE
    assert I.encode_e4m3(np.array([0.0, -0.0]))[:].tolist() == [0x00, 0x80]
    assert I.encode_e4m3(np.array([2.0 ** -10]))[0] == 0x00     # tie to even -> 0
    assert I.encode_e4m3(np.array([3 * 2.0 ** -10]))[0] == 0x02


def test_block_scales_and_quantisation_invariants():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((300, 384)).astype(np.float32)
    x[256:, 128:256] = 0.0                                       # an all-zero (partial) block
    q, s = I.quantize(x)
    assert s.shape == (3, 3) and s.dtype == np.float32
    assert s[2, 1] == 1.0
    # fp32(amax / 448) per block
    for rb in range(3):
        for kb in range(3):
            blk = x[rb * 128:(rb + 1) * 128, kb * 128:(kb + 1) * 128]
            amax = np.float32(np.abs(blk).max())
            if amax == 0:
                continue
            assert s[rb, kb] == amax / np.float32(448.0)
            dq = torch_decode(q[rb * 128:(rb + 1) * 128, kb * 128:(kb + 1) * 128])
            assert np.abs(dq).max() == 448.0                     # the block max hits 448
            # error of one RNE step: half a quantum of the code's binade
            err = np.abs(dq * np.float64(s[rb, kb]) - blk.astype(np.float64))
            assert np.all(err <= np.maximum(np.abs(blk) * 2.0 ** -4, 2.0 ** -10 * s[rb, kb]) * (1 + 1e-6))
    assert not np.any((q == 0x7F) | (q == 0xFF))


def test_seeded_determinism():
    a = I.make_config(1)
    b = I.make_config(1)
    np.testing.assert_array_equal(a.A, b.A)
    np.testing.assert_array_equal(a.sB, b.sB)
    c = I.make_config(1, seed=7)
    assert not np.array_equal(a.A, c.A)


def test_config_shapes_small():
    p = I.make_config(1)
    assert (p.M, p.N, p.K, p.out_dtype) == (256, 256, 256, "f32")
    assert p.A.shape == (256, 256) and p.B.shape == (256, 256)
    assert p.sA.shape == (2, 2) and p.sB.shape == (2, 2)


@pytest.mark.parametrize("seed", [0, 1, 2, 4])
def test_uniform_top2_routing(seed):
    off, toks, counts = I.route(8, 4096, I.streams(seed)[3], "uniform")
    assert counts.sum() == 8192
    assert np.all(off % 128 == 0) and off[0] == 0
    assert 8192 < off[-1] <= 8192 + 8 * 127
    # two distinct experts per token: every token appears exactly twice
    allt = np.concatenate(toks)
    assert np.all(np.bincount(allt, minlength=4096) == 2)
    for t in toks:
        assert np.all(np.diff(t) > 0)                              # token-id order


@pytest.mark.parametrize("seed", [0, 1, 2, 5])
def test_zipf_top2_routing(seed):
    off, toks, counts = I.route(64, 8192, I.streams(seed)[3], "zipf")
    assert counts.sum() == 16384
    assert (counts == 0).sum() == 4                                # the zeroed experts
    seg = np.diff(off)
    assert np.all(seg[counts == 0] == 0)
    assert np.all(seg == -(-counts // 128) * 128)
    # Zipf: the most popular expert receives far more than the least popular live one
    live = counts[counts > 0]
    assert live.max() > 8 * live.min()


def test_grouped_layout_small():
    p = I.grouped_problem(G=5, N=256, K=256, T=300, seed=3, popularity="zipf", zero_lowest=1)
    off = p.group_offsets
    assert p.A.shape == (off[-1], 256) and p.B.shape == (5, 256, 256)
    assert p.sA.shape == (off[-1] // 128, 2) and p.sB.shape == (5, 2, 2)
    # padding rows are zero codes
    off_, toks, counts = I.route(5, 300, I.streams(3)[3], "zipf", zero_lowest=1)
    for e in range(5):
        pad = p.A[off[e] + counts[e]:off[e + 1]]
        assert not pad.any()


def test_e5m2_encoder_matches_library_cast():
    """The generator's E5M2 encoder (binade snapping) against torch's RNE cast,
    inside the finite range."""
    import torch
    rng = np.random.default_rng(7)
    v = np.concatenate([rng.standard_normal(20000) * 3000, rng.uniform(-57344, 57344, 20000),
                        rng.standard_normal(5000) * 1e-4]).astype(np.float32).astype(np.float64)
    lib = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e5m2).view(torch.uint8).numpy()
    np.testing.assert_array_equal(I.encode_e5m2(v), lib)
    assert I.encode_e5m2(np.array([1e9]))[0] == 0x7B and I.encode_e5m2(np.array([-1e9]))[0] == 0xFB


def test_e5m2_problem_blocks_reach_the_format_max():
    p = I.dense_problem(130, 136, 256, seed=1, a_fmt="e5m2", b_fmt="e5m2")
    tab = (np.arange(256, dtype=np.uint16) << 8).view(np.float16).astype(np.float64)
    for X, R in ((p.A, 130), (p.B, 136)):
        for rb in range(-(-R // 128)):
            for kb in range(2):
                blk = X[rb * 128:(rb + 1) * 128, kb * 128:(kb + 1) * 128]
                assert np.abs(tab[blk]).max() == 57344.0
    assert p.a_fmt == "e5m2" and p.b_fmt == "e5m2"


def test_decode_workload_is_packed_top2():
    """Workload 6: 128 tokens, two distinct experts each, segments packed with
    no padding rows, one A scale per row, some experts empty."""
    p = I.make_config(6)
    offs = p.group_offsets.astype(np.int64)
    counts = np.diff(offs)
    assert p.packed and p.sa_rows == 1
    assert offs[0] == 0 and offs[-1] == p.M == 2 * 128 == p.real_rows
    assert np.all(counts >= 0) and np.any(counts == 0) and counts.max() <= 64
    assert p.sA.shape == (p.M, p.K // 128) and p.A.shape == (p.M, p.K)
    assert p.active_groups() == np.count_nonzero(counts)
    # a quantised row is the same token wherever it appears: each token's row
    # occurs in exactly two segments
    rows = {}
    for e in range(p.G):
        for r in range(offs[e], offs[e + 1]):
            rows.setdefault(p.A[r].tobytes(), []).append(e)
    assert all(len(v) == 2 and v[0] != v[1] for v in rows.values())
    assert len(rows) == 128
