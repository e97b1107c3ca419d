"""Pins for the oracle's W4A16 layer: it is the composition of its pinned
parts, and padding the token dimension with zero rows leaves the real rows'
results unchanged (the row-independence the TensorRT-LLM page relies on)."""

import numpy as np

import synth
from oracle import bucket, gemm, layer


def _small_case(T_pad, seed=11, bias=True):
    return synth.config3(T_pad, seed=seed, bias=bias, E=8, H=64, I=96)


def test_layer_is_composition():
    d = _small_case(24)
    b = {k: synth.bits(v) for k, v in d.items() if hasattr(v, "shape")}
    h, c2, y = layer.w4a16_layer(b["x"], b["ids"], b["topk_w"], 4, 8,
                                 b["w1"], b["s1"], b["b1"], b["w2"], b["s2"], b["b2"])
    h_ref, _ = gemm.grouped_gemm(b["x"], 4, b["w1"], "e2m1x2", b["s1"], b["ids"], 8,
                                 bias=b["b1"], epilogue="swiglu")
    np.testing.assert_array_equal(h, h_ref)
    c2_ref, _ = gemm.grouped_gemm(h_ref, 1, b["w2"], "e2m1x2", b["s2"], b["ids"], 8,
                                  bias=b["b2"], a_dtype="f64")
    np.testing.assert_array_equal(c2, c2_ref)
    np.testing.assert_array_equal(y, gemm.combine(c2_ref, b["topk_w"], 4))


def test_padded_rows_do_not_change_real_rows():
    T = 19
    Tb = bucket.bucket_round_up(T)
    assert Tb == 20
    d = _small_case(Tb)
    b = {k: synth.bits(v) for k, v in d.items() if hasattr(v, "shape")}
    xp = b["x"].copy()
    xp[T:] = 0  # padded rows are zero activations; their routing is drawn like any row
    hp, cp, yp = layer.w4a16_layer(xp, b["ids"], b["topk_w"], 4, 8,
                                   b["w1"], b["s1"], b["b1"], b["w2"], b["s2"], b["b2"])
    hu, cu, yu = layer.w4a16_layer(xp[:T], b["ids"][:T], b["topk_w"][:T], 4, 8,
                                   b["w1"], b["s1"], b["b1"], b["w2"], b["s2"], b["b2"])
    # float64 products of different row counts may differ in the last bits
    np.testing.assert_allclose(hp[:T * 4], hu, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(cp[:T * 4], cu, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(yp[:T], yu, rtol=1e-13, atol=1e-13)
