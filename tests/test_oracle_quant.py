"""Pins of the quantisation oracle (oracle/quantize.py) to things other than
itself: the E4M3 value table of the FP8 kernel write-up (section 3.1, via the
golden fixture), ties-to-even at exact midpoints, saturation, a library cast
(torch.float8_e4m3fn), the block invariants that follow from amax / 448, and
the operand generator's encoder, which is written differently (binade
arithmetic instead of a table search).  CPU only."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from moe_grouped_gemm_block_amd import inputs as I

LUT = oracle.decode_table()
FINITE = [c for c in range(256) if c not in (0x7F, 0xFF)]


def test_round_trip_every_finite_code():
    for c in FINITE:
        v = LUT[c]
        got = int(oracle.encode_nearest(np.array([v]))[0])
        if v == 0.0:
            assert got == c                      # +0 -> 0x00, -0 -> 0x80
        else:
            assert got == c, (hex(c), v, hex(got))


def test_golden_table_values(golden_dir):
    fmt = json.load(open(os.path.join(golden_dir, "e4m3_format.json")))["formats"]["E4M3"]
    top = float(fmt["max_approx"])
    assert oracle.encode_nearest(np.array([top]))[0] == 0x7E
    assert oracle.encode_nearest(np.array([-top]))[0] == 0xFE
    # every finite magnitude has 1 + mantissa_bits significant bits at most
    for c in FINITE:
        v = abs(LUT[c])
        if v:
            m, e = np.frexp(v)
            assert (m * 2 ** (1 + fmt["mantissa_bits"])) % 1 == 0


def test_midpoints_go_to_even_code():
    # between every pair of neighbouring non-negative values
    vals = LUT[:0x7F]
    for c in range(0x7E):
        mid = (vals[c] + vals[c + 1]) / 2
        want = c if c % 2 == 0 else c + 1
        assert oracle.encode_nearest(np.array([mid]))[0] == want, (c, mid)
        assert oracle.encode_nearest(np.array([-mid]))[0] == want | 0x80
        below, above = np.nextafter(mid, 0.0), np.nextafter(mid, np.inf)
        assert oracle.encode_nearest(np.array([below]))[0] == c
        assert oracle.encode_nearest(np.array([above]))[0] == c + 1


def test_known_cases():
    cases = {1.0625: 0x38, 1.1875: 0x3A, 2.0 ** -10: 0x00, 3 * 2.0 ** -10: 0x02, 2.0 ** -6: 0x08,
             448.0: 0x7E, 460.0: 0x7E, 1e30: 0x7E, 432.0: 0x7E, 431.9: 0x7D, 0.0: 0x00}
    for v, c in cases.items():
        assert oracle.encode_nearest(np.array([v]))[0] == c, (v, hex(c))
    assert oracle.encode_nearest(np.array([-0.0]))[0] == 0x80
    assert oracle.encode_nearest(np.array([-1e-30]))[0] == 0x80


def test_matches_library_cast_in_range():
    rng = np.random.default_rng(5)
    v = np.concatenate([rng.standard_normal(20000) * 50, rng.uniform(-448, 448, 20000),
                        rng.standard_normal(5000) * 1e-3])
    v = v.astype(np.float32).astype(np.float64)
    lib = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(oracle.encode_nearest(v), lib)


@pytest.mark.parametrize("R", [1, 128])
def test_block_invariants(R):
    rng = np.random.default_rng(R)
    x = (rng.standard_normal((300, 384)) * np.exp2(rng.uniform(-8, 8, (300, 1)))).astype(np.float32)
    x[0:R, 128:256] = 0.0                        # an all-zero block
    q, s = oracle.quantize_blockscaled(x, R)
    assert s.shape == (-(-300 // R), 3) and s.dtype == np.float32
    assert s[0, 1] == 1.0 and np.all(q[0:R, 128:256] == 0)
    for rb in range(s.shape[0]):
        for kb in range(3):
            blk = x[rb * R:(rb + 1) * R, kb * 128:(kb + 1) * 128]
            amax = np.abs(blk).max()
            if amax == 0:
                continue
            assert s[rb, kb] == np.float32(np.float64(amax) / 448.0)
            qb = q[rb * R:(rb + 1) * R, kb * 128:(kb + 1) * 128]
            # the element of largest magnitude lands exactly on +-448
            i = np.unravel_index(np.argmax(np.abs(blk)), blk.shape)
            assert qb[i] & 0x7F == 0x7E
            # dequantised block within half an E4M3 step of x
            deq = LUT[qb] * np.float64(s[rb, kb])
            err = np.abs(deq - blk.astype(np.float64))
            step = np.maximum(np.abs(blk), 2.0 ** -6 * s[rb, kb]) * 2.0 ** -3
            assert np.all(err <= step * 0.5 * (1 + 1e-12) + 2.0 ** -10 * s[rb, kb])


def test_matches_generator_encoder_at_128():
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((256, 512)) * np.exp2(rng.uniform(-4, 4, (256, 512)))).astype(np.float32)
    q, s = oracle.quantize_blockscaled(x, 128)
    qg, sg = I.quantize(x)
    np.testing.assert_array_equal(s, sg)
    np.testing.assert_array_equal(q, qg)


def test_planted_mistake_is_caught():
    """An encoder that breaks ties away from zero (a plausible slip) differs
    on the midpoint pin's inputs."""
    vals = LUT[:0x7F]
    mids = (vals[1:0x7F] + vals[:0x7E]) / 2
    ties_away = np.searchsorted(vals, mids, side="right")   # always the upper neighbour
    assert np.any(ties_away != oracle.encode_nearest(mids))
