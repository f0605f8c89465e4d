"""Pins for the oracle's C quantizer and decoder (oracle/nvfp4_ref.c): the same brute-force
references with exact rationals as the NumPy oracle's pins, the hand-worked bytes of
tests/golden/nvfp4_layout_literal.txt, the E4M3 closed form of the amax block, and agreement with
the NumPy oracle (itself pinned) on random tensors, ragged valid rows and calibrated scales."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import nvfp4_oracle as O
from oracle import nvfp4_ref as R

from test_oracle_pins import E2M1_FR, E4M3_FR, bf16_values, brute_block_scale, brute_code, read_layout_literal


def test_literal_bytes():
    g = read_layout_literal()
    x = np.stack([g["x0"], g["x1"]])
    codes, scales, gs = R.quantize_bits(O.bf16_bits(x))
    assert float(gs) == g["gs"]
    assert codes.tolist() == [g["codes0"], g["codes1"]]
    assert scales.tolist() == [g["scales0"], g["scales1"]]
    assert np.array_equal(R.dequantize(codes, scales)[0] / float(gs), x[0])


def test_bruteforce_random_elements_and_scales():
    rng = np.random.default_rng(31)
    for trial in range(40):
        x = bf16_values(rng, 128, 0.09 * 2.0 ** rng.integers(-8, 8)).reshape(4, 32)
        if trial % 4 == 0:
            x[rng.integers(0, 4), rng.integers(0, 32)] = -0.0
        codes, scales, gs = R.quantize_bits(O.bf16_bits(x), threads=3)
        assert gs == O.global_scale(float(np.abs(x).max()))
        c = O.unpack_nibbles(codes)
        for r in range(4):
            for b in range(2):
                blk = x[r, 16 * b:16 * b + 16]
                assert scales[r, b] == brute_block_scale(np.abs(blk).max(), gs)
                for i in range(16):
                    assert c[r, 16 * b + i] == brute_code(blk[i], gs, scales[r, b])


def test_bruteforce_every_scale_code_and_element_tie():
    """gs = 1 (amax 2688): for every E4M3 code s, a block with amax 6s and elements on each E2M1
    midpoint times s (exact ties) and on each grid point."""
    rows = []
    for c in range(1, 127):
        s = O.E4M3_GRID[c]
        blk = [6 * s] + [m * s * (-1) ** j for j, m in enumerate(O.E2M1_MIDPOINTS)] + [0.0, -0.0] + \
            list(O.E2M1_MAGNITUDES[1:7] * s)
        rows.append(O.bf16_round(np.array(blk)))
    x = np.array(rows)
    x = np.concatenate([np.full((1, 16), 0.0), x])
    x[0, 0] = 2688.0
    codes, scales, gs = R.quantize_bits(O.bf16_bits(x))
    assert gs == np.float32(1.0)
    c = O.unpack_nibbles(codes)
    for r in range(1, x.shape[0]):
        assert scales[r, 0] == brute_block_scale(np.abs(x[r]).max(), gs)
        for i in range(16):
            assert c[r, i] == brute_code(x[r, i], gs, scales[r, 0])
    # the same bytes as the NumPy oracle
    c2, s2, g2 = O.quantize_nvfp4(x)
    assert np.array_equal(codes, c2) and np.array_equal(scales, s2) and g2 == gs


def test_block_scale_ties_go_to_even_code():
    mids = (O.E4M3_GRID[:-1] + O.E4M3_GRID[1:]) / 2
    a = O.bf16_round(6 * mids / 4.0)
    assert np.array_equal(a, 6 * mids / 4.0)
    x = np.zeros((len(a), 16))
    x[:, 0] = a
    # gs = 2688 / 672 = 4 exactly: the tensor amax sits in a row of its own
    x = np.concatenate([x, np.full((1, 16), 0.0)])
    x[-1, 0] = 672.0
    codes, scales, gs = R.quantize_bits(O.bf16_bits(x))
    assert gs == np.float32(4.0)
    for r in range(len(a)):
        assert scales[r, 0] == brute_block_scale(a[r], gs)
        assert scales[r, 0] % 2 == 0


def test_dequantize_every_code_and_scale():
    """Every (code, scale) pair decodes to e2m1 * e4m3 from the bit fields (exact Fractions)."""
    codes = np.array([[(2 * i) % 16 | (((2 * i + 1) % 16) << 4) for i in range(8)]], np.uint8)
    for s in range(0x7F):
        d = R.dequantize(codes, np.array([[s]], np.uint8))[0]
        for i in range(16):
            mag = E2M1_FR[i % 8] * E4M3_FR[s]
            assert Fraction(float(d[i])) == (-mag if i % 16 >= 8 else mag)
    assert np.isnan(R.dequantize(codes, np.array([[0x7F]], np.uint8))).all()


@pytest.mark.parametrize("threads", [1, 5])
def test_agrees_with_numpy_oracle(threads):
    rng = np.random.default_rng(32)
    x = bf16_values(rng, 37 * 256, 0.09).reshape(37, 256)
    x[3, 17] = 8.0  # an outlier sets the global scale
    valid = rng.random(37) > 0.3
    for vr in (None, valid):
        c1, s1, g1 = O.quantize_nvfp4(x, vr)
        c2, s2, g2 = R.quantize_bits(O.bf16_bits(x), vr, threads=threads)
        assert g1 == g2 and np.array_equal(c1, c2) and np.array_equal(s1, s2)
        assert np.array_equal(O.dequantize_blocks(c1, s1), R.dequantize(c2, s2, threads=threads))


def test_calibrated_scale_saturates_like_numpy_oracle():
    """A given global scale too large for the data (the pages' 3977.6 on amax 8): scale 448, codes +-6."""
    rng = np.random.default_rng(33)
    x = bf16_values(rng, 8 * 64, 0.5).reshape(8, 64)
    x[0, :4] = O.bf16_round(np.array([8.0, -8.0, 2.0, 1.27]))
    gs = np.float32(3977.6)
    c1, s1 = O.quantize_rows_with_global_scale(x, gs)
    c2, s2, g2 = R.quantize_bits(O.bf16_bits(x), gs=gs)
    assert g2 == gs and np.array_equal(c1, c2) and np.array_equal(s1, s2)
    assert s2[0, 0] == 0x7E and (O.unpack_nibbles(c2)[0, :2] & 7 == 7).all()


def test_amax_block_closed_form():
    rng = np.random.default_rng(34)
    x = bf16_values(rng, 64 * 128, 0.09).reshape(64, 128)
    codes, scales, gs = R.quantize_bits(O.bf16_bits(x))
    r, k = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    assert scales[r, k // 16] == 0x7E and O.unpack_nibbles(codes)[r, k] & 7 == 7
    assert scales.max() <= 0x7E
