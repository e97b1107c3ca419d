"""MXFP8 conversion of activations (oracle; test infrastructure only).

The MXFP8 grouped GEMM of ROCm/aiter PR #5310 "Add MoE GEMM variants and
weight-gradient kernel" (Summary; the second review's excerpt of the kernel,
which decodes an a_scale and a b_scale E8M0 byte per K block) takes both
operands as E4M3 codes with one E8M0 scale per 32 consecutive K elements.
The pages do not say how bf16 activations become such codes. Reading: the
conversion of the OCP Microscaling Formats (MX) v1.0 specification, for each
row and each block of 32 consecutive K elements v_0 .. v_31:

    X = floor(log2(max_i |v_i|)) - 8        (8 = largest exponent of E4M3)
    X clamped to [-127, 127] (the E8M0 range); an all-zero block takes -127
    scale byte = X + 127
    code_i = E4M3 value nearest to v_i / 2^X, ties to the even code,
             magnitudes above 448 (the largest finite E4M3) saturate to 448,
             sign bit set exactly when v_i < 0

so that dec(code_i) * 2^X approximates v_i.

A block holding a NaN or an infinity has no finite shared exponent: it
converts to a NaN block, scale byte 0xFF (the E8M0 NaN) and every code 0x7F
(an E4M3 NaN), so the non-finite input is never replaced by finite numbers
and neighbouring blocks are unaffected (a reading: the pages give no
conversion, and the MX format's NaN scale marks the whole block NaN).

Pinned by tests/test_oracle_quant.py: every finite code survives a round trip
at a fixed shared exponent, saturation, ties, zero and clamped blocks, and
agreement with torch's float8_e4m3fn cast on in-range values.
"""

import numpy as np

from .formats import e4m3_to_f64

E4M3_EMAX = 8
E4M3_MAX = 448.0
MX_BLOCK = 32


def _e4m3_table():
    """Non-negative finite E4M3 values in increasing order and their codes."""
    codes = np.arange(0x7F, dtype=np.uint8)  # 0x00 .. 0x7E (0x7F is NaN)
    vals = e4m3_to_f64(codes)
    return vals, codes


_VALS, _CODES = _e4m3_table()


def e4m3_round(q):
    """float64 array -> E4M3 codes: nearest finite value, ties to the even
    code, magnitudes beyond 448 saturate, sign bit for negative inputs."""
    q = np.asarray(q, dtype=np.float64)
    a = np.minimum(np.abs(q), E4M3_MAX)
    hi = np.searchsorted(_VALS, a, side="left")  # first table value >= a
    hi = np.minimum(hi, len(_VALS) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = a - _VALS[lo], _VALS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_CODES[hi] % 2 == 0))
    mag = np.where(pick_hi, _CODES[hi], _CODES[lo]).astype(np.uint8)
    return np.where(q < 0, mag | np.uint8(0x80), mag).astype(np.uint8)


def mx_quantize_e4m3(x):
    """x float64 [R, K] (K a multiple of 32) -> (codes uint8 [R, K],
    scales uint8 [R, K / 32]) as the module docstring defines."""
    x = np.asarray(x, dtype=np.float64)
    R, K = x.shape
    assert K % MX_BLOCK == 0
    blocks = x.reshape(R, K // MX_BLOCK, MX_BLOCK)
    bad = ~np.isfinite(blocks).all(axis=2)          # blocks holding a NaN or an infinity
    blocks = np.where(bad[:, :, None], 0.0, blocks)
    amax = np.abs(blocks).max(axis=2)
    # floor(log2(amax)) exactly: amax = m * 2^e with m in [0.5, 1)
    _, e = np.frexp(np.where(amax > 0, amax, 1.0))
    X = np.where(amax > 0, e - 1 - E4M3_EMAX, -127)
    X = np.clip(X, -127, 127)
    q = blocks / np.ldexp(1.0, X)[:, :, None]
    codes = np.where(bad[:, :, None], np.uint8(0x7F), e4m3_round(q)).astype(np.uint8).reshape(R, K)
    scales = np.where(bad, 0xFF, X + 127).astype(np.uint8)
    return codes, scales


def mx_dequantize_e4m3(codes, scales):
    """Inverse map: dec(code) * 2^(scale - 127), float64 [R, K]."""
    codes = np.asarray(codes, dtype=np.uint8)
    R, K = codes.shape
    s = np.repeat(np.asarray(scales, dtype=np.int64), MX_BLOCK, axis=1)[:, :K]
    return e4m3_to_f64(codes) * np.ldexp(1.0, s - 127)
