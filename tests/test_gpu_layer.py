"""The W4A16 MXFP4 expert layer on the GPU (align -> gate+up GEMM with SwiGLU
-> down GEMM -> combine): parity with the float64 oracle on a small layer in
full and on the gpt-oss-shaped layer on sampled tokens, and padded ==
unpadded, bit for bit, on the real tokens."""

import numpy as np
import pytest
import torch

import synth
from helpers import assert_parity, bf16_to_f64, combine_scale, host, need_gpu
from oracle import gemm as ogemm
from oracle import layer as olayer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _moe():
    import mixture_experts_grouped_moe_amd as moe
    return moe


def run_layer(d, T, pad):
    """Run the layer over the first T tokens (or their bucket, with pad).
    Returns (h, c2, y, Tr): h and c2 cover the Tr*k slots that ran."""
    moe = _moe()
    k, E = d["k"], d["E"]
    Tr = moe.moe_bucket_round_up(T) if pad else T
    bm = moe.moe_gemm_block_m("e2m1x2", Tr)
    routing = moe.moe_align(d["ids"], E, bm, num_tokens=Tr)
    h = moe.moe_grouped_gemm(d["x"], d["w1"], "e2m1x2", routing, Tr, k, E, k, w_scale=d["s1"],
                             bias=d["b1"], epilogue="swiglu")
    c2 = moe.moe_grouped_gemm(h, d["w2"], "e2m1x2", routing, Tr, k, E, 1, w_scale=d["s2"], bias=d["b2"])
    y = moe.moe_combine(c2, d["topk_w"], k, num_tokens=T)
    torch.cuda.synchronize()
    return h, c2, y, Tr


@pytest.mark.parametrize("bias", [False, True])
def test_small_layer_full_parity(bias):
    d = synth.config3(150, seed=21, bias=bias, device="cuda", E=8, H=256, I=192)
    h, c2, y, _ = run_layer(d, 150, pad=False)
    hh = host(d)
    rh, rc2, ry = olayer.w4a16_layer(hh["x"], hh["ids"], hh["topk_w"], 4, 8, hh["w1"], hh["s1"], hh["b1"],
                                     hh["w2"], hh["s2"], hh["b2"])
    assert_parity(bf16_to_f64(h), rh, what="h")
    assert_parity(bf16_to_f64(c2), rc2, what="c2")
    assert_parity(bf16_to_f64(y), ry, scale=combine_scale(rc2, hh["topk_w"], 4), what="y")


def test_layer_binding_matches_steps():
    moe = _moe()
    d = synth.config3(160, seed=22, bias=True, device="cuda", E=8, H=256, I=192)
    d["x"][150:] = 0
    _, _, y_steps, _ = run_layer(d, 150, pad=True)
    y = moe.moe_w4a16_layer(d["x"], d["ids"], d["topk_w"], d["w1"], d["s1"], d["w2"], d["s2"],
                            b1=d["b1"], b2=d["b2"], num_tokens=150, pad_token_dim=True)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_steps.view(torch.int16))


@pytest.fixture(scope="module")
def big_layer():
    d = {False: synth.config3(8192, bias=False, device="cuda"),
         True: synth.config3(8192, bias=True, device="cuda")}
    return d


@pytest.mark.parametrize("bias", [False, True])
def test_gpt_oss_layer_sampled_parity(big_layer, bias):
    d = big_layer[bias]
    T = 8192
    h, c2, y, _ = run_layer(d, T, pad=False)
    hh = host(d)
    # h of 64 tokens spread over [0, 8192) (all 256 of their slots) on 96
    # SwiGLU columns, both edges of every 256-column tile among them: the
    # oracle's up GEMM over the matching gate and up weight rows
    rng = np.random.default_rng(8)
    tokens64 = sorted(set([0, 8191] + rng.choice(np.arange(1, 8191), 62, replace=False).tolist()))
    slots64 = [t * 4 + j for t in tokens64 for j in range(4)]
    half = 2880
    cols = sorted(set([0, half - 1] + [c for t in range(half // 256 + 1) for c in (256 * t, 256 * t + 255)
                                        if c < half] + rng.choice(half, 60, replace=False).tolist()))
    rows = torch.as_tensor(np.array(cols + [half + c for c in cols], dtype=np.int64), device=d["w1"].device)

    class _Rows:
        def __init__(self, t):
            self.t, self.shape = t, (t.shape[0], rows.numel()) + tuple(t.shape[2:])

        def __getitem__(self, e):
            return synth.bits(self.t[int(e)].index_select(0, rows))

    b1 = None if hh["b1"] is None else synth.bits(d["b1"].index_select(1, rows))
    rh64, _ = ogemm.grouped_gemm(hh["x"], 4, _Rows(d["w1"]), "e2m1x2", _Rows(d["s1"]), hh["ids"], 128,
                                 bias=b1, epilogue="swiglu", slots=slots64)
    assert_parity(bf16_to_f64(h[slots64][:, cols]), rh64[slots64], what="h of 64 tokens")
    # the whole layer (h, c2, y in full width) for 8 tokens
    tokens = [0, 1, 1234, 4097, 5000, 6553, 7680, 8191]
    slots = [t * 4 + j for t in tokens for j in range(4)]
    rh, rc2, _ = olayer.w4a16_layer(hh["x"], hh["ids"], hh["topk_w"], 4, 128, hh["w1"], hh["s1"], hh["b1"],
                                    hh["w2"], hh["s2"], hh["b2"], slots=slots)
    assert_parity(bf16_to_f64(h[slots]), rh[slots], what="h sampled")
    assert_parity(bf16_to_f64(c2[slots]), rc2[slots], what="c2 sampled")
    ry = ogemm.combine(rc2[slots], hh["topk_w"][tokens], 4)
    assert_parity(bf16_to_f64(y[tokens]), ry, scale=combine_scale(rc2[slots], hh["topk_w"][tokens], 4),
                  what="y sampled")


PAD_T = [6554, 6656, 6657, 7680, 8191, 8192] + synth.draw_token_counts(2, 6554, 8192, seed=1003)


@pytest.mark.parametrize("bias", [False, True])
@pytest.mark.parametrize("T", PAD_T)
def test_padded_equals_unpadded_bitwise(big_layer, T, bias):
    moe = _moe()
    d = dict(big_layer[bias])
    Tb = moe.moe_bucket_round_up(T)
    assert Tb <= 8192 and 8 * Tb <= 9 * T
    x = d["x"].clone()
    x[T:] = 0  # the padded rows are zero activations; their routing is drawn like any row
    d["x"] = x
    hp, cp, yp, Tr = run_layer(d, T, pad=True)
    assert Tr == Tb
    hu, cu, yu, _ = run_layer(d, T, pad=False)
    S = T * 4
    assert torch.equal(hp[:S].view(torch.int16), hu[:S].view(torch.int16))
    assert torch.equal(cp[:S].view(torch.int16), cu[:S].view(torch.int16))
    assert torch.equal(yp.view(torch.int16), yu.view(torch.int16))
    assert yp.shape[0] == T
    assert not torch.isnan(yu.float()).any()
