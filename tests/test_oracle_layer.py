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


def _bf16(vals):
    import torch
    return torch.tensor(np.asarray(vals, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_relu2_layer_closed_form():
    # x = a, w1 = 1, w2 = c, no bias: h = relu(H a)^2 on every column,
    # c2 = N h c, y = (sum of the token's routing weights) * c2
    T, k, E, H, N = 3, 2, 4, 32, 16
    ids = np.array([[0, 1], [2, 3], [1, 0]], dtype=np.int32)
    tw = np.array([[0.5, 0.25], [1.0, 2.0], [0.125, 0.125]])
    for a, expect_h in ((0.5, 256.0), (-0.5, 0.0)):
        x = np.full((T, H), _bf16([a])[0], dtype=np.uint16)
        w1 = np.full((E, N, H), _bf16([1.0])[0], dtype=np.uint16)
        w2 = np.full((E, H, N), _bf16([0.25])[0], dtype=np.uint16)
        h, c2, y = layer.relu2_layer(x, ids, tw, k, E, w1, None, w2, None)
        np.testing.assert_array_equal(h, np.full((T * k, N), expect_h))
        np.testing.assert_array_equal(c2, np.full((T * k, H), N * expect_h * 0.25))
        np.testing.assert_array_equal(y, tw.sum(axis=1)[:, None] * N * expect_h * 0.25 * np.ones((T, H)))


def test_relu2_layer_is_composition():
    rng = np.random.default_rng(3)
    T, k, E, H, N = 9, 3, 6, 64, 96
    x = _bf16(rng.standard_normal((T, H)))
    w1 = _bf16(rng.standard_normal((E, N, H)) * 0.1)
    w2 = _bf16(rng.standard_normal((E, H, N)) * 0.1)
    b1 = _bf16(rng.standard_normal((E, N)))
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    tw = rng.random((T, k))
    h, c2, y = layer.relu2_layer(x, ids, tw, k, E, w1, b1, w2, None)
    h_ref, _ = gemm.grouped_gemm(x, k, w1, "bf16", None, ids, E, bias=b1, epilogue="relu2")
    np.testing.assert_array_equal(h, h_ref)
    c2_ref, _ = gemm.grouped_gemm(h_ref, 1, w2, "bf16", None, ids, E, a_dtype="f64")
    np.testing.assert_array_equal(c2, c2_ref)
    np.testing.assert_array_equal(y, gemm.combine(c2_ref, tw, k))
