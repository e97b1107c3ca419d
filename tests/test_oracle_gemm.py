"""Pins for the oracle's grouped GEMM, SwiGLU and combine.

Against: the constant-input closed form and bias variant (the aiter page's
GEMM tests), linearity, an exact Fraction triple loop on tiny shapes whose
element values come from torch's decoders and the OCP E2M1 table (not from
the oracle's decoders), and closed forms of silu."""

import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import gemm

E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _bf16_bits(vals):
    t = torch.tensor(np.asarray(vals, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _routing(T, k, E, seed):
    rng = np.random.default_rng(seed)
    return np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)


@pytest.mark.parametrize("w_dtype,code,val", [("e4m3", 0x38, 1.0), ("e4m3", 0x44, 3.0),
                                               ("e2m1x2", 0x22, 1.0), ("e2m1x2", 0x77, 6.0),
                                               ("bf16", None, 1.5)])
@pytest.mark.parametrize("q", [-4, 0, 2])
def test_constant_input_roundtrip(w_dtype, code, val, q):
    # A == a, W == code, scale == 2^q -> C = K * a * val * 2^q (+ bias[e])
    T, k, E, N, K, a = 6, 2, 3, 8, 64, 0.5
    ids = _routing(T, k, E, 0)
    x = np.full((T, K), _bf16_bits([a])[0], dtype=np.uint16)
    if w_dtype == "bf16":
        w = np.full((E, N, K), _bf16_bits([val])[0], dtype=np.uint16)
        ws = None
        q = 0
    else:
        kk = K // 2 if w_dtype == "e2m1x2" else K
        w = np.full((E, N, kk), code, dtype=np.uint8)
        ws = np.full((E, N, K // 32), 127 + q, dtype=np.uint8)
    bias = _bf16_bits(np.repeat(np.array([1.0, -2.0, 0.25]), N).reshape(E, N))
    C, routed = gemm.grouped_gemm(x, k, w, w_dtype, ws, ids, E, bias=bias)
    assert routed.all()
    expect = K * a * val * 2.0 ** q + np.array([1.0, -2.0, 0.25])[ids.reshape(-1)][:, None]
    np.testing.assert_array_equal(C, np.broadcast_to(expect, C.shape))


def test_bias_variant_is_exact_difference():
    rng = np.random.default_rng(3)
    T, k, E, N, K = 9, 3, 4, 16, 96
    ids = _routing(T, k, E, 1)
    x = _bf16_bits(rng.standard_normal((T, K)))
    w = rng.integers(0, 256, (E, N, K), dtype=np.uint8)
    w[(w & 0x7F) == 0x7F] = 0  # no NaN codes
    ws = rng.integers(123, 130, (E, N, K // 32), dtype=np.uint8)
    bias = _bf16_bits(rng.standard_normal((E, N)))
    c0, _ = gemm.grouped_gemm(x, k, w, "e4m3", ws, ids, E)
    c1, _ = gemm.grouped_gemm(x, k, w, "e4m3", ws, ids, E, bias=bias)
    bvals = torch.from_numpy(bias.view(np.int16)).view(torch.bfloat16).double().numpy()
    np.testing.assert_allclose(c1 - c0, bvals[ids.reshape(-1)], rtol=0, atol=1e-12)


def test_linearity_in_activations():
    rng = np.random.default_rng(4)
    T, k, E, N, K = 7, 2, 5, 12, 64
    ids = _routing(T, k, E, 2)
    a1 = rng.integers(-8, 9, (T, K)).astype(np.float64)
    a2 = rng.integers(-8, 9, (T, K)).astype(np.float64)
    w = rng.integers(0, 256, (E, N, K // 2), dtype=np.uint8)
    ws = rng.integers(120, 130, (E, N, K // 32), dtype=np.uint8)
    c1, _ = gemm.grouped_gemm(_bf16_bits(a1), k, w, "e2m1x2", ws, ids, E)
    c2, _ = gemm.grouped_gemm(_bf16_bits(a2), k, w, "e2m1x2", ws, ids, E)
    c3, _ = gemm.grouped_gemm(_bf16_bits(3 * a1 - 2 * a2), k, w, "e2m1x2", ws, ids, E)
    np.testing.assert_allclose(c3, 3 * c1 - 2 * c2, rtol=1e-12, atol=1e-9)


def _fraction_gemm(a_vals, a_row_div, w_vals, ids, E, bias_vals):
    """Exact triple loop over Fractions: C[s][n] = sum_k A[s//d][k] W[e][n][k] + b."""
    S = len(ids)
    N, K = len(w_vals[0]), len(w_vals[0][0])
    out = {}
    for s in range(S):
        e = ids[s]
        if not (0 <= e < E):
            continue
        row = a_vals[s // a_row_div]
        out[s] = [sum((row[kk] * w_vals[e][n][kk] for kk in range(K)), Fraction(0))
                  + (bias_vals[e][n] if bias_vals is not None else 0) for n in range(N)]
    return out


def _frac(x):
    return Fraction(float(x))


@pytest.mark.parametrize("w_dtype", ["e4m3", "e2m1x2", "bf16"])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_fraction_brute_force(w_dtype, seed):
    rng = np.random.default_rng(100 + seed)
    T, k, E, N, K = 5, 2, 3, 3, 64   # N != K and N != T: a transposed operand fails
    ids = _routing(T, k, E, seed).reshape(-1).copy()
    ids[rng.integers(0, ids.size)] = E  # one unrouted slot
    x = _bf16_bits(rng.standard_normal((T, K)))
    a_vals = [[_frac(v) for v in row] for row in torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).double().numpy()]
    if w_dtype == "bf16":
        w = _bf16_bits(rng.standard_normal((E, N, K)) * 0.1)
        ws = None
        wv = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).double().numpy()
    else:
        ws = rng.integers(120, 135, (E, N, K // 32), dtype=np.uint8)
        scale = np.array([[[Fraction(2) ** (int(b) - 127) for b in row] for row in ex] for ex in ws], dtype=object)
        if w_dtype == "e4m3":
            w = rng.integers(0, 256, (E, N, K), dtype=np.uint8)
            w[(w & 0x7F) == 0x7F] = 0x01
            elem = torch.from_numpy(w).view(torch.float8_e4m3fn).double().numpy()
        else:
            w = rng.integers(0, 256, (E, N, K // 2), dtype=np.uint8)
            lo = np.vectorize(lambda c: (-1 if c & 8 else 1) * E2M1_TABLE[c & 7])(w & 0xF)
            hi = np.vectorize(lambda c: (-1 if c & 8 else 1) * E2M1_TABLE[c & 7])(w >> 4)
            elem = np.empty((E, N, K))
            elem[..., 0::2] = lo
            elem[..., 1::2] = hi
        wv = np.empty((E, N, K), dtype=object)
        for e in range(E):
            for n in range(N):
                for kk in range(K):
                    wv[e, n, kk] = _frac(elem[e, n, kk]) * scale[e, n, kk // 32]
    if w_dtype == "bf16":
        wv = [[[_frac(v) for v in row] for row in ex] for ex in wv]
    bias = _bf16_bits(rng.standard_normal((E, N)))
    bv = [[_frac(v) for v in row] for row in torch.from_numpy(bias.view(np.int16)).view(torch.bfloat16).double().numpy()]
    expect = _fraction_gemm(a_vals, k, wv, ids.tolist(), E, bv)
    C, routed = gemm.grouped_gemm(x, k, w, w_dtype, ws, ids, E, bias=bias)
    assert sorted(np.nonzero(routed)[0].tolist()) == sorted(expect)
    for s, row in expect.items():
        for n in range(N):
            exact = row[n]
            got = Fraction(float(C[s, n]))
            # float64 accumulation of K dyadic products: within a few ulps
            assert abs(got - exact) <= Fraction(1, 2 ** 45) * (1 + abs(exact)), (s, n)


def test_slot_subset_matches_full():
    rng = np.random.default_rng(5)
    T, k, E, N, K = 20, 4, 8, 10, 64
    ids = _routing(T, k, E, 5)
    x = _bf16_bits(rng.standard_normal((T, K)))
    w = _bf16_bits(rng.standard_normal((E, N, K)))
    full, _ = gemm.grouped_gemm(x, k, w, "bf16", None, ids, E)
    sub = [0, 7, 33, 79]
    part, routed = gemm.grouped_gemm(x, k, w, "bf16", None, ids, E, slots=sub)
    assert np.nonzero(routed)[0].tolist() == sub
    np.testing.assert_array_equal(part[sub], full[sub])


def test_silu_closed_forms():
    assert gemm.silu(0.0) == 0.0
    assert math.isclose(gemm.silu(math.log(3.0)), 0.75 * math.log(3.0), rel_tol=1e-15)
    z = np.random.default_rng(6).standard_normal(1000) * 10
    np.testing.assert_allclose(gemm.silu(z) - gemm.silu(-z), z, rtol=1e-13, atol=1e-13)
    assert gemm.silu(-800.0) == 0.0 and gemm.silu(800.0) == 800.0


def test_swiglu_halves():
    pre = np.array([[0.0, math.log(3.0), 2.0, 5.0]])  # gate = [0, ln3], up = [2, 5]
    h = gemm.swiglu(pre)
    np.testing.assert_allclose(h, [[0.0, 0.75 * math.log(3.0) * 5.0]], rtol=1e-15)


def test_swiglu_epilogue_in_gemm():
    # constant input: pre = K*a*1 + bias, gate bias 0, up bias 1 -> h = silu(K a) * (K a + 1)
    T, k, E, N, K, a = 4, 1, 2, 6, 32, 0.25
    ids = np.zeros((T, k), dtype=np.int32)
    x = np.full((T, K), _bf16_bits([a])[0], dtype=np.uint16)
    w = np.full((E, N, K), 0x38, dtype=np.uint8)
    ws = np.full((E, N, 1), 127, dtype=np.uint8)
    bias = _bf16_bits(np.array([[0, 0, 0, 1, 1, 1]] * E, dtype=np.float64))
    h, _ = gemm.grouped_gemm(x, k, w, "e4m3", ws, ids, E, bias=bias, epilogue="swiglu")
    z = K * a
    expect = z / (1 + math.exp(-z)) * (z + 1)
    np.testing.assert_allclose(h, np.full((T, 3), expect), rtol=1e-15)


def test_relu2_closed_forms():
    np.testing.assert_array_equal(gemm.relu2(np.array([-3.0, -0.0, 0.0, 0.5, 3.0])), [0.0, 0.0, 0.0, 0.25, 9.0])


def test_relu2_epilogue_in_gemm():
    # constant input: pre = K*a + bias per column; bias -1 on the first three
    # columns (K a = 8 -> 7 -> 49) and -9 on the rest (-> -1 -> 0)
    T, k, E, N, K, a = 4, 1, 2, 6, 32, 0.25
    ids = np.zeros((T, k), dtype=np.int32)
    x = np.full((T, K), _bf16_bits([a])[0], dtype=np.uint16)
    w = np.full((E, N, K), 0x38, dtype=np.uint8)
    ws = np.full((E, N, 1), 127, dtype=np.uint8)
    bias = _bf16_bits(np.array([[-1, -1, -1, -9, -9, -9]] * E, dtype=np.float64))
    h, _ = gemm.grouped_gemm(x, k, w, "e4m3", ws, ids, E, bias=bias, epilogue="relu2")
    np.testing.assert_array_equal(h, np.tile([49.0, 49.0, 49.0, 0.0, 0.0, 0.0], (T, 1)))


def test_combine_identity_and_example():
    c = np.arange(12, dtype=np.float64).reshape(4, 3)
    np.testing.assert_array_equal(gemm.combine(c, np.ones((4, 1)), 1), c)
    c = np.array([[1, 2], [3, 4], [5, 6], [7, 8]], dtype=np.float64)
    w = np.array([[0.5, 0.25], [1.0, -1.0]])
    np.testing.assert_array_equal(gemm.combine(c, w, 2), [[1.25, 2.0], [-2.0, -2.0]])


def test_combine_linear_in_weights():
    rng = np.random.default_rng(7)
    c = rng.standard_normal((30, 5))
    w1, w2 = rng.standard_normal((10, 3)), rng.standard_normal((10, 3))
    np.testing.assert_allclose(gemm.combine(c, 2 * w1 + w2, 3),
                               2 * gemm.combine(c, w1, 3) + gemm.combine(c, w2, 3), rtol=1e-12, atol=1e-12)


def test_nan_scale_propagates_to_its_rows_only():
    T, k, E, N, K = 3, 1, 1, 4, 64
    ids = np.zeros((T, k), dtype=np.int32)
    x = np.full((T, K), _bf16_bits([1.0])[0], dtype=np.uint16)
    w = np.full((E, N, K), 0x38, dtype=np.uint8)
    ws = np.full((E, N, 2), 127, dtype=np.uint8)
    ws[0, 2, 1] = 0xFF
    C, _ = gemm.grouped_gemm(x, k, w, "e4m3", ws, ids, E)
    assert np.all(np.isnan(C[:, 2])) and not np.any(np.isnan(C[:, [0, 1, 3]]))


def test_block_mapping_example_and_cover():
    eid, beg, end = gemm.build_block_mapping([3, 0, 5, 1], 2, 8)
    assert eid.tolist() == [0, 0, 2, 2, 2, 3, -1, -1]
    assert beg.tolist() == [0, 2, 3, 5, 7, 8, 9, 9]
    assert end.tolist() == [3, 3, 8, 8, 8, 9, 9, 9]
    rng = np.random.default_rng(9)
    for _ in range(20):
        g = rng.integers(0, 9, size=int(rng.integers(1, 12)))
        bm = int(rng.integers(1, 6))
        mb = int(g.sum()) // bm + len(g) + 1
        eid, beg, end = gemm.build_block_mapping(g, bm, mb)
        covered = np.zeros(int(g.sum()), dtype=int)
        offs = np.concatenate([[0], np.cumsum(g)])
        for b in range(mb):
            if eid[b] >= 0:
                e = eid[b]
                assert offs[e] <= beg[b] < end[b] == offs[e + 1]
                covered[beg[b]:min(beg[b] + bm, end[b])] += 1
        assert (covered == 1).all()


def test_per_token_gemm_constant_input_and_bias():
    # A = W = 1.0 (E4M3 0x38): the dot product is K, times both scales, plus bias
    E, N, K = 3, 4, 64
    g = [2, 0, 3]
    a = np.full((5, K), 0x38, dtype=np.uint8)
    a_s = np.array([1.0, 0.5, 2.0, 0.25, 4.0])
    w = np.full((E, N, K), 0x38, dtype=np.uint8)
    w_s = np.array([0.5, 7.0, 3.0])
    bias = _bf16_bits(np.array([[1.0] * N, [0.0] * N, [-2.0] * N]))
    C = gemm.grouped_gemm_per_token(a, a_s, w, w_s, g, bias=bias)
    expect = np.array([K * 1.0 * 0.5 + 1, K * 0.5 * 0.5 + 1, K * 2.0 * 3 - 2, K * 0.25 * 3 - 2, K * 4.0 * 3 - 2])
    np.testing.assert_array_equal(C, np.repeat(expect[:, None], N, axis=1))
    assert gemm.grouped_gemm_per_token(a[:0], a_s[:0], w, w_s, [0, 0, 0]).shape == (0, N)


def test_per_token_gemm_scalar_loop():
    rng = np.random.default_rng(10)
    E, N, K = 3, 5, 32
    g = [1, 3, 0]
    codes = [c for c in range(256) if (c & 0x7F) != 0x7F]
    a = rng.choice(codes, size=(4, K)).astype(np.uint8)
    w = rng.choice(codes, size=(E, N, K)).astype(np.uint8)
    a_s, w_s = rng.random(4), rng.random(E)
    C = gemm.grouped_gemm_per_token(a, a_s, w, w_s, g)

    def dec(c):  # E4M3 from its definition: sign, 4-bit exponent (bias 7), 3-bit mantissa
        c = int(c)
        e, m = (c >> 3) & 15, c & 7
        v = m / 8 * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
        return -v if c & 0x80 else v
    owner = [0, 1, 1, 1]
    for r in range(4):
        e = owner[r]
        for n in range(N):
            acc = sum(dec(a[r, k]) * dec(w[e, n, k]) for k in range(K))
            assert C[r, n] == pytest.approx(acc * a_s[r] * w_s[e], rel=1e-12)


# ---- the both-operands-MXFP8 branch (a_dtype="e4m3" with an E8M0 a_scale):
# the aiter kernel decodes an a_scale and a b_scale byte per 32-element K
# block (second review). Pins: a constant-input closed form whose activation
# and weight scales differ per K block and per token row, an exact Fraction
# triple loop decoded with torch's float8_e4m3fn and Fraction powers of two,
# and slots of one token reading one scale row.

@pytest.mark.parametrize("a_row_div", ["top_k", 1])
def test_mxfp8_activations_constant_input_closed_form(a_row_div):
    # A codes == ca, W codes == cw; a_scale[r, b] and w_scale[e, n, b] vary
    # with the row, the K block and the weight row, so
    # C[s, n] = sum_b 32 dec(ca) dec(cw) 2^(sa[r, b] + sw[e, n, b] - 254), r = s // d
    T, k, E, N, K = 5, 3, 4, 6, 128
    d = k if a_row_div == "top_k" else 1
    R = T * k // d
    ids = _routing(T, k, E, 11)
    ca, cw = 0x40, 0xBC  # 2.0 and -1.5
    a = np.full((R, K), ca, dtype=np.uint8)
    w = np.full((E, N, K), cw, dtype=np.uint8)
    nb = K // 32
    sa = np.array([[120 + (r % 5) + 2 * b for b in range(nb)] for r in range(R)], dtype=np.uint8)
    sw = np.array([[[125 + e + (n % 3) - b for b in range(nb)] for n in range(N)] for e in range(E)],
                  dtype=np.uint8)
    C, routed = gemm.grouped_gemm(a, d, w, "e4m3", sw, ids, E, a_dtype="e4m3", a_scale=sa)
    assert routed.all()
    flat = ids.reshape(-1)
    for s in range(T * k):
        r, e = s // d, flat[s]
        for n in range(N):
            expect = sum(32 * 2.0 * -1.5 * 2.0 ** (int(sa[r, b]) + int(sw[e, n, b]) - 254) for b in range(nb))
            assert C[s, n] == expect, (s, n)


def test_mxfp8_activations_one_scale_row_per_token():
    # a_row_div = top_k: the top_k slots of a token read one activation row
    # and one scale row. With every expert's weights equal, those slots'
    # outputs are equal, and each token's differ from its neighbours' (its
    # own scale row), so reading the scale by slot (or by the wrong token)
    # changes the result.
    T, k, E, N, K = 4, 3, 5, 4, 64
    ids = _routing(T, k, E, 12)
    rng = np.random.default_rng(13)
    codes = [c for c in range(256) if (c & 0x7F) != 0x7F]
    a = rng.choice(codes, size=(T, K)).astype(np.uint8)
    sa = (124 + np.arange(T)[:, None] + np.array([[0, 3]])).astype(np.uint8)  # per token and block
    w1 = rng.choice(codes, size=(1, N, K)).astype(np.uint8)
    w = np.repeat(w1, E, axis=0)
    sw = np.full((E, N, K // 32), 127, dtype=np.uint8)
    C, _ = gemm.grouped_gemm(a, k, w, "e4m3", sw, ids, E, a_dtype="e4m3", a_scale=sa)
    for t in range(T):
        for j in range(1, k):
            np.testing.assert_array_equal(C[t * k + j], C[t * k])
    # the same rows with token 0's scales in place of token 1's: token 1's outputs change
    sa2 = sa.copy()
    sa2[1] = sa[0]
    C2, _ = gemm.grouped_gemm(a, k, w, "e4m3", sw, ids, E, a_dtype="e4m3", a_scale=sa2)
    assert not np.array_equal(C2[k:2 * k], C[k:2 * k])
    np.testing.assert_array_equal(C2[:k], C[:k])


@pytest.mark.parametrize("a_row_div", ["top_k", 1])
@pytest.mark.parametrize("seed", [0, 1])
def test_mxfp8_activations_fraction_brute_force(a_row_div, seed):
    rng = np.random.default_rng(200 + seed)
    T, k, E, N, K = 4, 2, 3, 3, 64   # N, K, T and the row count all differ
    d = k if a_row_div == "top_k" else 1
    R = T * k // d
    ids = _routing(T, k, E, 20 + seed).reshape(-1).copy()
    ids[rng.integers(0, ids.size)] = -1  # one unrouted slot
    codes = [c for c in range(256) if (c & 0x7F) != 0x7F]
    a = rng.choice(codes, size=(R, K)).astype(np.uint8)
    sa = rng.integers(118, 137, (R, K // 32), dtype=np.uint8)
    w = rng.choice(codes, size=(E, N, K)).astype(np.uint8)
    sw = rng.integers(118, 137, (E, N, K // 32), dtype=np.uint8)
    a_elem = torch.from_numpy(a).view(torch.float8_e4m3fn).double().numpy()
    w_elem = torch.from_numpy(w).view(torch.float8_e4m3fn).double().numpy()
    a_vals = [[_frac(a_elem[r, kk]) * Fraction(2) ** (int(sa[r, kk // 32]) - 127) for kk in range(K)]
              for r in range(R)]
    w_vals = [[[_frac(w_elem[e, n, kk]) * Fraction(2) ** (int(sw[e, n, kk // 32]) - 127) for kk in range(K)]
               for n in range(N)] for e in range(E)]
    expect = _fraction_gemm(a_vals, d, w_vals, ids.tolist(), E, None)
    C, routed = gemm.grouped_gemm(a, d, w, "e4m3", sw, ids, E, a_dtype="e4m3", a_scale=sa)
    assert sorted(np.nonzero(routed)[0].tolist()) == sorted(expect)
    for s, row in expect.items():
        for n in range(N):
            exact = row[n]
            got = Fraction(float(C[s, n]))
            assert abs(got - exact) <= Fraction(1, 2 ** 45) * (1 + abs(exact)), (s, n)
