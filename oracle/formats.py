"""Element and scale decoders (oracle; test infrastructure only).

Pure bit arithmetic into float64. Every code of every format is representable
exactly in float64, so these decoders are exact.

Sources: ROCm/aiter PR #5310 "Add MoE GEMM variants and weight-gradient
kernel", Summary (moe_gemm_mxfp8: one E8M0 byte per 32 K-elements, turned into
an fp32 power of two) and the second review (an E8M0 byte of 0x00 means
2^-127, 0xFF means NaN; a bare shift into the exponent field is wrong at both).
The E4M3 and E2M1 element formats are those of the OCP Microscaling (MX)
specification; E4M3 is the "FN" flavour (no infinities, NaN at S.1111.111).
"""

import numpy as np

E8M0_NAN = 0xFF


def e8m0_to_f64(codes):
    """E8M0 scale byte b -> 2^(b - 127); b = 255 -> NaN.

    b = 0 gives 2^-127 (a subnormal in fp32, an ordinary number here).
    Pinned: tests/test_oracle_formats.py (all codes vs torch.float8_e8m0fnu,
    and the printed edge values of the aiter review).
    """
    b = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    out = np.ldexp(np.ones(b.shape, dtype=np.float64), b - 127)
    out = np.where(b == E8M0_NAN, np.nan, out)
    return out


def e4m3_to_f64(codes):
    """OCP E4M3 (FN) byte -> value.

    Layout s.eeee.mmm, exponent bias 7. e = 0: (-1)^s * 2^-6 * m/8 (subnormal).
    e > 0: (-1)^s * 2^(e-7) * (1 + m/8). e = 15 with m = 7 is NaN; there is no
    infinity, so the largest finite magnitude is 2^8 * 1.75 = 448.
    Pinned: tests/test_oracle_formats.py (all 256 codes vs torch.float8_e4m3fn).
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 0x7
    sign = np.where(s == 1, -1.0, 1.0)
    sub = np.ldexp(m.astype(np.float64) / 8.0, -6)
    nor = np.ldexp(1.0 + m.astype(np.float64) / 8.0, e - 7)
    out = sign * np.where(e == 0, sub, nor)
    out = np.where((e == 15) & (m == 7), np.nan, out)
    return out


def e2m1_to_f64(nibbles):
    """OCP E2M1 4-bit code -> value.

    Layout s.ee.m, exponent bias 1. e = 0: (-1)^s * m/2 (subnormal: 0 or 0.5).
    e > 0: (-1)^s * 2^(e-1) * (1 + m/2). Magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.
    Pinned: tests/test_oracle_formats.py (the format's 16-entry value table).
    """
    c = np.asarray(nibbles).astype(np.int64) & 0xF
    s = (c >> 3) & 1
    e = (c >> 1) & 0x3
    m = c & 0x1
    sign = np.where(s == 1, -1.0, 1.0)
    sub = m.astype(np.float64) / 2.0
    nor = np.ldexp(1.0 + m.astype(np.float64) / 2.0, e - 1)
    return sign * np.where(e == 0, sub, nor)


def e2m1x2_unpack(packed):
    """Packed E2M1 bytes [..., K/2] -> nibble codes [..., K].

    Element 2i sits in the low nibble of byte i, element 2i+1 in the high
    nibble (the packing the weights use throughout this project).
    """
    p = np.asarray(packed, dtype=np.uint8)
    lo = p & 0xF
    hi = (p >> 4) & 0xF
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def bf16_to_f64(bits):
    """bfloat16 bit pattern (uint16) -> value: the upper half of an fp32.

    Pinned: tests/test_oracle_formats.py (all 65536 patterns vs torch.bfloat16).
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):  # NaN patterns stay NaN
        return b.view(np.float32).astype(np.float64)
