"""The large-M GEMM kernels store C in two ways: 16-byte row pieces staged
through LDS when C is 16-byte aligned with a row stride that is a multiple of
8 elements, else each lane's 2-byte values directly. Both round the same
fp32 values once, so C must be bit-identical either way, in every kernel
(bf16 activations over each weight encoding, MXFP8 activations, per-token
scales) and epilogue, with N tails that end inside a 16-byte piece and rows
of unrouted slots left as they were; the oracle checks the values."""

import pytest
import torch

import synth
from helpers import assert_parity, bf16_to_f64, host, need_gpu, to_dev
from oracle import gemm as ogemm

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _moe():
    import mixture_experts_grouped_moe_amd as moe
    return moe


def _outs(rows, cols):
    """(aligned C, C with row stride cols + 1, C at a 2-byte offset), NaN-filled."""
    a = torch.full((rows, cols), float("nan"), dtype=torch.bfloat16, device="cuda")
    b = torch.full((rows, cols + 1), float("nan"), dtype=torch.bfloat16, device="cuda")[:, :cols]
    ld = (cols + 7) // 8 * 8
    flat = torch.full((rows * ld + 8,), float("nan"), dtype=torch.bfloat16, device="cuda")
    c = flat[1:1 + rows * ld].view(rows, ld)[:, :cols]
    assert a.data_ptr() % 16 == 0 and b.stride(0) % 8 != 0 and c.data_ptr() % 16 != 0
    return a, b, c


def _same_bits(x, y, what):
    assert torch.equal(x.contiguous().view(torch.int16), y.contiguous().view(torch.int16)), what


@pytest.mark.parametrize("epilogue", ["none", "swiglu", "relu2"])
@pytest.mark.parametrize("wd", ["e2m1x2", "e4m3", "bf16"])
def test_bf16_activation_kernel_stores(wd, epilogue):
    moe = _moe()
    T, k, E, N, K = 150, 3, 5, 300, 288  # 450 slots (large-M kernel); N / 2 = 150: both end mid-piece
    d = synth.gemm_case(T, k, E, N, K, wd, seed=401, bias=True, w_std=0.5)
    dd = to_dev(d)
    bm = moe.moe_gemm_block_m(wd, T)
    routing = moe.moe_align(dd["ids"], E, bm)
    out_w = N // 2 if epilogue == "swiglu" else N
    outs = _outs(T * k, out_w)
    for out in outs:
        moe.moe_grouped_gemm(dd["x"], dd["w"], wd, routing, T, k, E, k, w_scale=dd["w_scale"], bias=dd["bias"],
                             epilogue=epilogue, out=out)
    torch.cuda.synchronize()
    _same_bits(outs[0], outs[1], f"{wd} {epilogue}: row stride")
    _same_bits(outs[0], outs[2], f"{wd} {epilogue}: offset")
    h = host(d)
    ref, routed = ogemm.grouped_gemm(h["x"], k, h["w"], wd, h["w_scale"], h["ids"], E, bias=h["bias"],
                                     epilogue=epilogue)
    assert routed.all()
    assert_parity(bf16_to_f64(outs[0]), ref, what=f"{wd} {epilogue}")


def test_unrouted_rows_untouched_by_both_stores():
    moe = _moe()
    T, k, E, N, K = 120, 2, 6, 264, 160
    d = synth.gemm_case(T, k, E, N, K, "e4m3", seed=402, w_std=0.5)
    ids = d["ids"].clone()
    ids[::7, 1] = -1
    ids[3::11, 0] = E + 3
    d["ids"] = ids
    dd = to_dev(d)
    routing = moe.moe_align(dd["ids"], E, moe.moe_gemm_block_m("e4m3", T))
    outs = _outs(T * k, N)
    for out in outs:
        moe.moe_grouped_gemm(dd["x"], dd["w"], "e4m3", routing, T, k, E, k, w_scale=dd["w_scale"], out=out)
    torch.cuda.synchronize()
    _same_bits(outs[0], outs[1], "row stride")
    _same_bits(outs[0], outs[2], "offset")
    h = host(d)
    ref, routed = ogemm.grouped_gemm(h["x"], k, h["w"], "e4m3", h["w_scale"], h["ids"], E)
    got = bf16_to_f64(outs[0])
    assert (~routed).sum() > 0 and torch.isnan(outs[0].float()[torch.from_numpy(~routed).cuda()]).all()
    assert_parity(got[routed], ref[routed], what="routed rows")


@pytest.mark.parametrize("epilogue", ["none", "swiglu"])
def test_mxfp8_activation_kernel_stores(epilogue):
    moe = _moe()
    T, k, E, N, K = 150, 3, 5, 300, 288
    d = synth.gemm_case(T, k, E, N, K, "e4m3", seed=403, bias=True, w_std=0.5)
    a_codes = synth.e4m3_normal((T, K), 1.0, 403, "xq")
    a_scales = synth.e8m0_uniform((T, K // 32), 120, 130, 403, "xs")
    dd = to_dev(d)
    routing = moe.moe_align(dd["ids"], E, moe.moe_gemm_block_m("e4m3", T, moe.MOE_E4M3))
    out_w = N // 2 if epilogue == "swiglu" else N
    outs = _outs(T * k, out_w)
    for out in outs:
        moe.moe_grouped_gemm(a_codes.cuda(), dd["w"], "e4m3", routing, T, k, E, k, w_scale=dd["w_scale"],
                             bias=dd["bias"], epilogue=epilogue, out=out, a_scale=a_scales.cuda())
    torch.cuda.synchronize()
    _same_bits(outs[0], outs[1], f"{epilogue}: row stride")
    _same_bits(outs[0], outs[2], f"{epilogue}: offset")
    h = host(d)
    ref, _ = ogemm.grouped_gemm(synth.bits(a_codes), k, h["w"], "e4m3", h["w_scale"], h["ids"], E, bias=h["bias"],
                                epilogue=epilogue, a_dtype="e4m3", a_scale=synth.bits(a_scales))
    assert_parity(bf16_to_f64(outs[0]), ref, what=f"mxfp8 activations {epilogue}")


def test_per_token_kernel_stores():
    moe = _moe()
    d = synth.per_token_case([70, 0, 5, 130, 1, 64], 300, 96, 404, bias=True, device="cuda")
    mapping = moe.moe_block_mapping(d["group_sizes"], d["R"])
    outs = _outs(d["R"], 300)
    for out in outs:
        moe.moe_grouped_gemm_per_token(d["a"], d["a_scale"], d["w"], d["w_scale"], mapping, bias=d["bias"], out=out)
    torch.cuda.synchronize()
    _same_bits(outs[0], outs[1], "row stride")
    _same_bits(outs[0], outs[2], "offset")
    h = {kk: synth.bits(v) if isinstance(v, torch.Tensor) else v for kk, v in d.items()}
    ref = ogemm.grouped_gemm_per_token(h["a"], h["a_scale"], h["w"], h["w_scale"], h["group_sizes"], bias=h["bias"])
    assert_parity(bf16_to_f64(outs[0]), ref, what="per-token")
