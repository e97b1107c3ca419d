"""GPU tests of the K-block weight layout: moe_pack_weights is a bit-exact
copy into the layout oracle.layout defines, and the grouped GEMM (large-M and
decode variants, every encoding, bias and SwiGLU) gives the same bits from
packed weights as from rows-layout weights, and so the same oracle parity."""

import numpy as np
import pytest
import torch

import synth
from helpers import assert_parity, bf16_to_f64, combine_scale, host, need_gpu, to_dev
from oracle import gemm as ogemm
from oracle import layer as olayer
from oracle import layout as olayout

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _moe():
    import mixture_experts_grouped_moe_amd as moe
    return moe


@pytest.mark.parametrize("wd", ["e2m1x2", "e4m3", "bf16"])
@pytest.mark.parametrize("K", [96, 320])
def test_pack_is_bit_exact(wd, K):
    moe = _moe()
    E, N = 3, 70
    d = synth.gemm_case(4, 1, E, N, K, wd, seed=K, device="cuda")
    # strided input: rows of a wider buffer (row stride past the row's end)
    U = d["w"].shape[2]
    wide = torch.zeros((E, N, U + 16), dtype=d["w"].dtype, device="cuda")
    wide[:, :, :U] = d["w"]
    w_in = wide[:, :, :U]
    pw = moe.moe_pack_weights(w_in, wd, w_scale=d["w_scale"])
    torch.cuda.synchronize()
    ref_w, ref_s = olayout.pack_kblock(synth.bits(d["w"]), wd,
                                       None if d["w_scale"] is None else synth.bits(d["w_scale"]))
    assert np.array_equal(synth.bits(pw.codes), ref_w)
    if wd == "bf16":
        assert pw.scales is None
    else:
        assert np.array_equal(synth.bits(pw.scales), ref_s)
    assert moe.moe_packed_sizes(wd, N, K) == (pw.codes[0].numel(), 0 if pw.scales is None else pw.scales[0].numel())


CASES = [
    # T, k, E, N, K, w_dtype: large-M and decode, ragged N and K tails (K % 64 == 32)
    (200, 2, 4, 640, 320, "e2m1x2"),
    (300, 4, 16, 1056, 352, "e2m1x2"),
    (150, 3, 5, 300, 288, "e4m3"),
    (97, 2, 3, 200, 96, "bf16"),
    (1, 2, 8, 640, 320, "e2m1x2"),
    (7, 6, 16, 200, 352, "e4m3"),
    (32, 4, 16, 1056, 2080, "bf16"),
]


def _run(moe, d, w, w_scale, epilogue):
    T, k, E = d["T"], d["k"], d["E"]
    bm = moe.moe_gemm_block_m(d["w_dtype"], T)
    routing = moe.moe_align(d["ids"], E, bm)
    n_out = d["N"] // 2 if epilogue == "swiglu" else d["N"]
    out = torch.full((T * k, n_out), float("nan"), dtype=torch.bfloat16, device="cuda")
    moe.moe_grouped_gemm(d["x"], w, d["w_dtype"], routing, T, k, E, k, w_scale=w_scale, bias=d["bias"],
                         epilogue=epilogue, out=out)
    return out


@pytest.mark.parametrize("epilogue", ["none", "swiglu"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "T{}k{}E{}N{}K{}{}".format(*c))
def test_packed_gemm_matches_rows_bitwise_and_oracle(case, epilogue):
    moe = _moe()
    T, k, E, N, K, wd = case
    d = to_dev(synth.gemm_case(T, k, E, N, K, wd, seed=T + N + K + 1, bias=True, w_std=0.5))
    pw = moe.moe_pack_weights(d["w"], wd, w_scale=d["w_scale"])
    c_rows = _run(moe, d, d["w"], d["w_scale"], epilogue)
    c_pack = _run(moe, d, pw, None, epilogue)
    torch.cuda.synchronize()
    assert torch.equal(c_rows.view(torch.int16), c_pack.view(torch.int16)), f"{case} {epilogue}"
    h = host(d)
    ref, routed = ogemm.grouped_gemm(h["x"], k, h["w"], wd, h["w_scale"], h["ids"], E, bias=h["bias"],
                                     epilogue=epilogue)
    assert routed.all()
    assert_parity(bf16_to_f64(c_pack), ref, what=f"packed {case} {epilogue}")


def test_packed_layer_matches_oracle_and_padding_is_exact():
    moe = _moe()
    T = 150
    d = synth.config3(160, seed=23, bias=True, device="cuda", E=8, H=256, I=192)
    d["x"][T:] = 0
    p1 = moe.moe_pack_weights(d["w1"], "e2m1x2", w_scale=d["s1"])
    p2 = moe.moe_pack_weights(d["w2"], "e2m1x2", w_scale=d["s2"])
    y = moe.moe_w4a16_layer(d["x"], d["ids"], d["topk_w"], p1, None, p2, None, b1=d["b1"], b2=d["b2"],
                            num_tokens=T)
    y_pad = moe.moe_w4a16_layer(d["x"], d["ids"], d["topk_w"], p1, None, p2, None, b1=d["b1"],
                                b2=d["b2"], num_tokens=T, pad_token_dim=True)
    y_rows = moe.moe_w4a16_layer(d["x"], d["ids"], d["topk_w"], d["w1"], d["s1"], d["w2"], d["s2"],
                                 b1=d["b1"], b2=d["b2"], num_tokens=T)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_pad.view(torch.int16))
    assert torch.equal(y.view(torch.int16), y_rows.view(torch.int16))
    hh = host(d)
    _, rc2, ry = olayer.w4a16_layer(hh["x"][:T], hh["ids"][:T], hh["topk_w"][:T], 4, 8, hh["w1"], hh["s1"],
                                    hh["b1"], hh["w2"], hh["s2"], hh["b2"])
    assert_parity(bf16_to_f64(y), ry, scale=combine_scale(rc2, hh["topk_w"][:T], 4), what="packed layer y")


def test_packed_gpt_oss_layer_matches_rows_bitwise():
    # the gpt-oss-shaped layer (E=128, H=I=2880, top-4) at 8192 tokens and at
    # 7000 tokens padded to its bucket: packed and rows-layout weights agree
    # bit for bit, so the rows layout's oracle parity carries over
    moe = _moe()
    d = synth.config3(8192, seed=1003, bias=True, device="cuda")
    p1 = moe.moe_pack_weights(d["w1"], "e2m1x2", w_scale=d["s1"])
    p2 = moe.moe_pack_weights(d["w2"], "e2m1x2", w_scale=d["s2"])
    for T, pad in ((8192, False), (7000, True)):
        x = d["x"].clone()
        x[T:] = 0
        y_p = moe.moe_w4a16_layer(x, d["ids"], d["topk_w"], p1, None, p2, None, b1=d["b1"], b2=d["b2"],
                                  num_tokens=T, pad_token_dim=pad)
        y_r = moe.moe_w4a16_layer(x, d["ids"], d["topk_w"], d["w1"], d["s1"], d["w2"], d["s2"], b1=d["b1"],
                                  b2=d["b2"], num_tokens=T)
        torch.cuda.synchronize()
        assert torch.equal(y_p.view(torch.int16), y_r.view(torch.int16)), T
        assert not torch.isnan(y_p.float()).any()
