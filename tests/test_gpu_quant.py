"""GPU tests of moe_quantize_mxfp8 (the MXFP8 conversion of activations):
codes and scale bytes bit-identical to oracle.quant on seeded inputs with a
spread of block magnitudes, strided rows, zero, tiny, saturating and tied
blocks, and at the MXFP8 workload's activation shape."""

import numpy as np
import pytest
import torch

import synth
from helpers import bf16_to_f64, need_gpu
from oracle import formats
from oracle import quant as oquant

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _moe():
    import mixture_experts_grouped_moe_amd as moe
    return moe


def _check(x, **kw):
    moe = _moe()
    q, s = moe.moe_quantize_mxfp8(x, **kw)
    torch.cuda.synchronize()
    R, K = x.shape
    ref_q, ref_s = oquant.mx_quantize_e4m3(bf16_to_f64(x))
    assert np.array_equal(synth.bits(s[:R, :K // 32]), ref_s)
    assert np.array_equal(synth.bits(q[:R, :K]), ref_q)


@pytest.mark.parametrize("R,K", [(1, 32), (37, 96), (130, 2048), (5, 7168)])
def test_codes_and_scales_bit_exact(R, K):
    # rows of N(0,1) times a per-row magnitude from 2^-130 to 2^120
    g = synth.gen(R * 31 + K, "quant")
    mag = torch.pow(2.0, torch.randint(-130, 121, (R, 1), generator=g).double())
    x = (torch.randn((R, K), generator=g, dtype=torch.float64) * mag).to(torch.bfloat16).cuda()
    _check(x)


def test_strided_rows():
    g = synth.gen(7, "quant")
    base = torch.randn((40, 320), generator=g).to(torch.bfloat16).cuda()
    x = base[:, :256]                                   # x_ld = 320
    q = torch.full((40, 272), 0xAB, dtype=torch.uint8, device="cuda")
    s = torch.full((40, 12), 0xCD, dtype=torch.uint8, device="cuda")
    _moe().moe_quantize_mxfp8(x, out=q[:, :256], out_scales=s[:, :8])
    torch.cuda.synchronize()
    ref_q, ref_s = oquant.mx_quantize_e4m3(bf16_to_f64(x))
    assert np.array_equal(synth.bits(q[:, :256]), ref_q)
    assert np.array_equal(synth.bits(s[:, :8]), ref_s)
    assert (synth.bits(q[:, 256:]) == 0xAB).all() and (synth.bits(s[:, 8:]) == 0xCD).all()


def test_edge_blocks():
    # zero block, bf16 subnormals, saturating and exactly tied elements,
    # negative zeros and negative tiny values, the largest bf16 magnitudes
    rows = np.zeros((6, 64))
    rows[1, :32] = np.ldexp(1.0, -133) * np.arange(1, 33)      # bf16 subnormals
    rows[2, :4] = [500.0, -511.0, 448.0, 449.0]
    e = formats.e4m3_to_f64(np.arange(0x38, 0x58, dtype=np.uint8))
    rows[3, :31] = (e[:-1] + e[1:])[:31] / 2                   # midpoints: ties
    rows[3, 31] = 256.0
    rows[4, :32] = -np.ldexp(1.0, -20)
    rows[4, 0] = 1.0                                            # the rest round to -0 (0x80)
    rows[4, 32:] = -0.0
    rows[5, :32] = 3.0e38 * np.linspace(-1, 1, 32)
    x = torch.tensor(rows, dtype=torch.float64).to(torch.bfloat16).cuda()
    _check(x)


def test_mxfp8_workload_activation_shape():
    # the MXFP8 workload's activations (the same draw as its x): [4096, 7168] bf16 N(0,1)
    x = synth.bf16_normal((4096, 7168), 1.0, 1004, "x", "cuda")
    _check(x)


def test_every_bf16_value_under_a_power_of_two_block_max():
    # every finite bf16 value v with |v| <= M, in 32-element blocks led by M,
    # for block maxima M = 2^e across the range: each value's code at each
    # block scale, bit-exact with the oracle
    allbits = torch.arange(0, 1 << 16, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    vals = allbits.double()
    vals = vals[torch.isfinite(vals)]
    blocks = []
    for e in range(-126, 128, 9):
        M = 2.0 ** e
        v = vals[vals.abs() <= M]
        v = torch.cat([v, torch.zeros((-v.numel()) % 31, dtype=torch.float64)]).reshape(-1, 31)
        blocks.append(torch.cat([torch.full((v.shape[0], 1), M, dtype=torch.float64), v], dim=1))
    b = torch.cat(blocks)
    b = torch.cat([b, torch.zeros(((-b.shape[0]) % 32, 32), dtype=torch.float64)])
    x = b.reshape(-1, 1024).to(torch.bfloat16).cuda()
    _check(x)


def test_non_finite_blocks():
    # blocks holding a NaN, +inf or -inf become NaN blocks (scale 0xFF, codes
    # 0x7F) exactly as the oracle defines; their neighbours are unaffected
    g = synth.gen(11, "quant")
    x = torch.randn((6, 128), generator=g).to(torch.bfloat16)
    x[0, 5] = float("nan")
    x[1, 40] = float("inf")
    x[2, 127] = float("-inf")
    x[3, 64:96] = float("nan")
    x[4, 0] = float("inf")
    x[4, 33] = float("nan")
    _check(x.cuda())
    moe = _moe()
    q, s = moe.moe_quantize_mxfp8(x.cuda())
    torch.cuda.synchronize()
    s = synth.bits(s)
    assert s[0, 0] == 0xFF and s[1, 1] == 0xFF and s[2, 3] == 0xFF and s[3, 2] == 0xFF
    assert (s[5] != 0xFF).all()
