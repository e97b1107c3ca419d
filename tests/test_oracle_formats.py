"""Pins for the oracle's decoders: library decoders over every code, the OCP MX
value table for E2M1, and the E8M0 edge values printed by the aiter review."""

import math

import numpy as np
import torch

from oracle import formats


def test_e8m0_all_codes_match_library():
    codes = np.arange(256, dtype=np.uint8)
    ours = formats.e8m0_to_f64(codes)
    lib = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.isnan(ours[255]) and np.isnan(lib[255])
    np.testing.assert_array_equal(ours[:255], lib[:255])


def test_e8m0_printed_edge_values(page_facts):
    f = page_facts["e8m0"]
    v0 = formats.e8m0_to_f64(np.array([0], dtype=np.uint8))[0]
    assert v0 == math.ldexp(1.0, f["code_0x00_value_log2"])
    # 2^-127 as an fp32 is the subnormal with bit pattern 0x00400000.
    assert np.float32(v0).view(np.uint32) == int(f["code_0x00_fp32_bits"], 16)
    assert math.isnan(formats.e8m0_to_f64(np.array([255], dtype=np.uint8))[0])
    assert formats.e8m0_to_f64(np.array([127], dtype=np.uint8))[0] == 1.0
    assert formats.e8m0_to_f64(np.array([254], dtype=np.uint8))[0] == 2.0 ** 127


def test_e4m3_all_codes_match_library():
    codes = np.arange(256, dtype=np.uint8)
    ours = formats.e4m3_to_f64(codes)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan_o, nan_l = np.isnan(ours), np.isnan(lib)
    np.testing.assert_array_equal(nan_o, nan_l)
    assert sorted(np.nonzero(nan_o)[0].tolist()) == [0x7F, 0xFF]
    np.testing.assert_array_equal(ours[~nan_o], lib[~nan_l])
    # sign of zero
    assert math.copysign(1.0, ours[0x80]) == -1.0


def test_e4m3_spec_landmarks():
    # OCP MX spec, E4M3: max normal 448 (S.1111.110), min normal 2^-6,
    # min subnormal 2^-9, and 1.0 = S.0111.000.
    v = formats.e4m3_to_f64(np.array([0x7E, 0x08, 0x01, 0x38, 0xB8], dtype=np.uint8))
    assert v.tolist() == [448.0, 2.0 ** -6, 2.0 ** -9, 1.0, -1.0]


def test_e2m1_spec_table():
    # OCP MX spec, E2M1 element values for codes 0..7; codes 8..15 are negatives.
    table = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    codes = np.arange(16, dtype=np.uint8)
    v = formats.e2m1_to_f64(codes)
    assert v[:8].tolist() == table
    assert v[8:].tolist() == [-t for t in table]
    assert math.copysign(1.0, v[8]) == -1.0


def test_e2m1_unpack_order():
    # byte 0x71: low nibble (element 0) = code 1 = 0.5, high nibble (element 1) = code 7 = 6.0
    packed = np.array([[0x71, 0x2A]], dtype=np.uint8)
    nib = formats.e2m1x2_unpack(packed)
    assert nib.tolist() == [[1, 7, 0xA, 2]]
    assert formats.e2m1_to_f64(nib).tolist() == [[0.5, 6.0, -1.0, 1.0]]


def test_bf16_all_patterns_match_library():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = formats.bf16_to_f64(bits)
    lib = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan_o = np.isnan(ours)
    np.testing.assert_array_equal(nan_o, np.isnan(lib))
    np.testing.assert_array_equal(ours[~nan_o], lib[~nan_o])
