"""Pins of oracle.quant (the MXFP8 conversion of activations) to facts fixed
outside it: the E4M3 code table of the OCP MX format, the conversion's scale
rule on blocks built to have a known shared exponent, round-to-nearest-even
ties, saturation, zero and clamped blocks, and torch's float8_e4m3fn cast."""

import numpy as np
import pytest
import torch

from oracle import formats
from oracle import quant

FINITE = [c for c in range(256) if (c & 0x7F) != 0x7F]


@pytest.mark.parametrize("shift", [-30, -3, 0, 7, 100])
def test_every_finite_code_round_trips_at_a_known_exponent(shift):
    # a block holding 256 * 2^shift has max |v| in [256, 448] * 2^shift, so
    # X = floor(log2(max)) - 8 = shift, and every E4M3 value times 2^shift
    # comes back as its own code (zero may come back as +0 or -0: sign by v < 0)
    vals = formats.e4m3_to_f64(np.array(FINITE, dtype=np.uint8))
    rows = []
    for v in vals:
        row = np.zeros(32)
        row[0] = v * 2.0 ** shift
        row[1] = 256.0 * 2.0 ** shift
        rows.append(row)
    codes, scales = quant.mx_quantize_e4m3(np.array(rows))
    assert (scales == shift + 127).all()
    want = np.array(FINITE, dtype=np.uint8)
    want = np.where(want == 0x80, 0x00, want)  # -0.0 is not < 0
    assert np.array_equal(codes[:, 0], want)
    assert (codes[:, 1] == 0x78).all()  # 256 = 2^8: exponent field 15, mantissa 0
    assert (codes[:, 2:] == 0).all()


def test_scale_rule_on_powers_of_two():
    # max |v| = 2^p gives X = p - 8 for every p in the clamp-free range
    for p in range(-100, 120, 7):
        row = np.zeros((1, 32))
        row[0, 5] = -(2.0 ** p)
        codes, scales = quant.mx_quantize_e4m3(row)
        assert scales[0, 0] == p - 8 + 127
        assert codes[0, 5] == 0xF8  # -256


def test_saturation():
    row = np.zeros((1, 32))
    row[0, :4] = [500.0, -511.0, 448.0, 449.0]  # floor(log2 511) = 8: X = 0
    codes, scales = quant.mx_quantize_e4m3(row)
    assert scales[0, 0] == 127
    assert list(codes[0, :4]) == [0x7E, 0xFE, 0x7E, 0x7E]
    assert formats.e4m3_to_f64(np.uint8(0x7E)) == 448.0


def test_ties_go_to_the_even_code():
    # with X = 0 fixed by a 256 in the block: midpoints between neighbours
    pairs = [(0x38, 0x39), (0x39, 0x3A), (0x00, 0x01), (0x07, 0x08), (0x6E, 0x6F)]
    row = np.zeros((len(pairs), 32))
    row[:, 31] = 256.0
    for i, (a, b) in enumerate(pairs):
        row[i, 0] = (formats.e4m3_to_f64(np.uint8(a)) + formats.e4m3_to_f64(np.uint8(b))) / 2
    codes, _ = quant.mx_quantize_e4m3(row)
    for i, (a, b) in enumerate(pairs):
        assert codes[i, 0] == (a if a % 2 == 0 else b)


def test_zero_and_clamped_blocks():
    x = np.zeros((3, 64))
    x[1, 32:] = 2.0 ** -140            # X = -148 -> clamped to -127
    x[2, :32] = 3.0 * 2.0 ** 120       # X = 121 - 8 = 113, in range
    codes, scales = quant.mx_quantize_e4m3(x)
    assert list(scales[0]) == [0, 0] and (codes[0] == 0).all()
    assert scales[1, 1] == 0
    # 2^-140 / 2^-127 = 2^-13: below half the smallest subnormal (2^-10) -> 0
    assert (codes[1, 32:] == 0).all()
    assert scales[2, 0] == 113 + 127
    assert (codes[2, :32] == 0x7C).all()  # 3 * 2^120 / 2^113 = 384 = 1.5 * 2^8


def test_agrees_with_torch_cast_in_range():
    # v / 2^X never exceeds 512; for blocks whose max stays below 448 after
    # scaling, every element's code is torch's RNE float8_e4m3fn cast
    rng = np.random.default_rng(5)
    x = rng.standard_normal((64, 256)) * np.exp(rng.uniform(-8, 8, size=(64, 1)))
    x = torch.tensor(x, dtype=torch.bfloat16).double().numpy()
    codes, scales = quant.mx_quantize_e4m3(x)
    X = scales.astype(np.int64) - 127
    q = x.reshape(64, 8, 32) / np.ldexp(1.0, X)[:, :, None]
    ok = np.abs(q).max(axis=2) <= 448.0
    ref = torch.tensor(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = codes.reshape(64, 8, 32)
    assert ok.sum() > 100
    neg_zero = (ref == 0x80) & (got == 0x00)
    assert np.array_equal(np.where(neg_zero, 0x80, got)[ok], ref[ok])


def test_dequantize_error_bound():
    # each element lands within half an E4M3 step (relative 2^-4) of its
    # value, or within half the smallest subnormal step 2^(X-9) absolutely
    rng = np.random.default_rng(6)
    x = torch.tensor(rng.standard_normal((32, 128)), dtype=torch.bfloat16).double().numpy()
    codes, scales = quant.mx_quantize_e4m3(x)
    back = quant.mx_dequantize_e4m3(codes, scales)
    X = np.repeat(scales.astype(np.int64) - 127, 32, axis=1)
    sat = np.abs(x) > 448.0 * np.ldexp(1.0, X)  # saturated: exactly +-448 * 2^X
    assert sat.any()
    assert np.array_equal(back[sat], np.sign(x[sat]) * 448.0 * np.ldexp(1.0, X[sat]))
    bound = np.maximum(np.abs(x) * 2.0 ** -4, np.ldexp(1.0, X - 10))
    assert (np.abs(back - x) <= bound)[~sat].all()


def test_non_finite_blocks_become_nan_blocks():
    # a block holding a NaN, +inf or -inf converts to scale 0xFF (E8M0 NaN)
    # and codes 0x7F (E4M3 NaN); the other blocks of the row are unaffected
    row = np.zeros((3, 96))
    row[:, 32:64] = np.linspace(-3.0, 5.0, 32)
    row[:, 64:] = 256.0
    row[0, 40] = np.nan
    row[1, 33] = np.inf
    row[2, 63] = -np.inf
    codes, scales = quant.mx_quantize_e4m3(row)
    assert (scales[:, 1] == 0xFF).all() and (codes[:, 32:64] == 0x7F).all()
    clean = np.zeros((1, 96))
    clean[0, 64:] = 256.0
    c0, s0 = quant.mx_quantize_e4m3(clean)
    assert (scales[:, [0, 2]] == s0[:, [0, 2]]).all()
    assert (codes[:, :32] == c0[:, :32]).all() and (codes[:, 64:] == c0[:, 64:]).all()
    deq = quant.mx_dequantize_e4m3(codes, scales)
    assert np.isnan(deq[:, 32:64]).all() and not np.isnan(deq[:, :32]).any() and not np.isnan(deq[:, 64:]).any()
