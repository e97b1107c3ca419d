"""GPU parity of the squared-ReLU epilogue (max(pre, 0)^2) in every grouped
GEMM path (decode and large-M, each weight encoding, MXFP8 activations) and of
the non-gated relu2 expert layer at the Nemotron decode shape (E=128, top-6,
hidden 2688, N=1856) against the float64 oracle."""

import numpy as np
import pytest
import torch

import synth
from helpers import assert_parity, bf16_to_f64, combine_scale, host, need_gpu, to_dev
from oracle import gemm as ogemm
from oracle import layer as olayer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _moe():
    import mixture_experts_grouped_moe_amd as moe
    return moe


@pytest.mark.parametrize("case", [
    # T, k, E, N, K, w_dtype (T <= 32 runs the decode GEMM)
    (5, 6, 16, 200, 352, "bf16"),
    (28, 4, 16, 256, 2080, "e4m3"),
    (7, 2, 8, 640, 320, "e2m1x2"),
    (97, 2, 3, 200, 96, "bf16"),
    (150, 3, 5, 300, 288, "e4m3"),
    (200, 2, 4, 640, 320, "e2m1x2"),
], ids=lambda c: "T{}k{}E{}N{}K{}{}".format(*c))
def test_relu2_epilogue(case):
    moe = _moe()
    T, k, E, N, K, wd = case
    d = synth.gemm_case(T, k, E, N, K, wd, seed=T + N + K + 5, bias=True, w_std=0.5)
    dd = to_dev(d)
    routing = moe.moe_align(dd["ids"], E, moe.moe_gemm_block_m(wd, T))
    out = torch.full((T * k, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    moe.moe_grouped_gemm(dd["x"], dd["w"], wd, routing, T, k, E, k, w_scale=dd["w_scale"], bias=dd["bias"],
                         epilogue="relu2", out=out)
    torch.cuda.synchronize()
    h = host(d)
    ref, routed = ogemm.grouped_gemm(h["x"], k, h["w"], wd, h["w_scale"], h["ids"], E, bias=h["bias"],
                                     epilogue="relu2")
    assert routed.all()
    got = bf16_to_f64(out)
    assert (got >= 0).all()
    assert (got == 0).sum() > got.size // 4          # about half the pre-activations are negative
    assert_parity(got, ref, what=f"relu2 {case}")


def test_relu2_epilogue_mxfp8_activations():
    moe = _moe()
    T, k, E, N, K = 100, 4, 8, 512, 192
    d = synth.gemm_case(T, k, E, N, K, "e4m3", seed=9, bias=True, w_std=0.5)
    a_codes = synth.e4m3_normal((T, K), 1.0, 9, "xq")
    a_scales = synth.e8m0_uniform((T, K // 32), 120, 130, 9, "xs")
    dd = to_dev(d)
    routing = moe.moe_align(dd["ids"], E, moe.moe_gemm_block_m("e4m3", T, moe.MOE_E4M3))
    out = moe.moe_grouped_gemm(a_codes.cuda(), dd["w"], "e4m3", routing, T, k, E, k, w_scale=dd["w_scale"],
                               bias=dd["bias"], epilogue="relu2", a_scale=a_scales.cuda())
    torch.cuda.synchronize()
    h = host(d)
    ref, _ = ogemm.grouped_gemm(synth.bits(a_codes), k, h["w"], "e4m3", h["w_scale"], h["ids"], E, bias=h["bias"],
                                epilogue="relu2", a_dtype="e4m3", a_scale=synth.bits(a_scales))
    assert_parity(bf16_to_f64(out), ref, what="relu2 mxfp8 activations")


@pytest.mark.parametrize("M", [1, 7, 28, 120])
def test_nemotron_relu2_layer(M):
    # the full Nemotron-shaped layer: the decode GEMM for M <= 32, the large-M
    # one at 120 (the steady-state mid-M bucket). The layer's steps run one
    # by one so that h (after the relu2 epilogue) and the down GEMM's c2 are
    # checked as well as y; the binding's one-call layer gives y's bits.
    moe = _moe()
    d = synth.nemotron_layer(M, device="cuda", bias=(M == 7))
    k, E = 6, 128
    routing = moe.moe_align(d["ids"], E, moe.moe_gemm_block_m("bf16", M))
    h = moe.moe_grouped_gemm(d["x"], d["w1"], "bf16", routing, M, k, E, k, bias=d["b1"], epilogue="relu2")
    c2 = moe.moe_grouped_gemm(h, d["w2"], "bf16", routing, M, k, E, 1, bias=d["b2"])
    y_steps = moe.moe_combine(c2, d["topk_w"], k)
    y = moe.moe_relu2_layer(d["x"], d["ids"], d["topk_w"], d["w1"], d["w2"], b1=d["b1"], b2=d["b2"])
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_steps.view(torch.int16))
    hh = host(d)
    rh, rc2, ry = olayer.relu2_layer(hh["x"], hh["ids"], hh["topk_w"], k, E, hh["w1"], hh["b1"], hh["w2"],
                                     hh["b2"])
    assert_parity(bf16_to_f64(h), rh, what=f"nemotron h M={M}")
    assert_parity(bf16_to_f64(c2), rc2, what=f"nemotron c2 M={M}")
    assert_parity(bf16_to_f64(y), ry, scale=combine_scale(rc2, hh["topk_w"], k), what=f"nemotron layer M={M}")
