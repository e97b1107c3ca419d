"""Pins for the oracle's weight gradient: the aiter page's analytical
constant-input check, linearity and zero-padded-token guard, plus an exact
Fraction brute force and a scalar-loop cross-check on tiny shapes."""

from fractions import Fraction

import numpy as np
import torch

from oracle import wgrad


def _bf16_bits(vals):
    t = torch.tensor(np.asarray(vals, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _vals(bits):
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()


def _routing(T, k, E, seed):
    rng = np.random.default_rng(seed)
    return np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)


def test_constant_input():
    # x == a, grad == g -> dW[e] = c_e * g * a (c_e = slots routed to e)
    T, k, E, N, K, a, g = 13, 3, 6, 5, 7, 0.75, -1.5
    ids = _routing(T, k, E, 0)
    x = np.full((T, K), _bf16_bits([a])[0], dtype=np.uint16)
    gr = np.full((T * k, N), _bf16_bits([g])[0], dtype=np.uint16)
    dw = wgrad.wgrad(x, gr, ids, k, E)
    counts = np.bincount(ids.reshape(-1), minlength=E)
    for e in range(E):
        np.testing.assert_array_equal(dw[e], np.full((N, K), counts[e] * g * a))


def test_empty_expert_is_zero():
    ids = np.array([[0, 1], [1, 0]])
    x = _bf16_bits(np.ones((2, 4)))
    gr = _bf16_bits(np.ones((4, 3)))
    dw = wgrad.wgrad(x, gr, ids, 2, 3)
    assert np.all(dw[2] == 0) and np.all(dw[0] == 2)


def test_linearity_in_grad():
    rng = np.random.default_rng(1)
    T, k, E, N, K = 20, 2, 4, 6, 8
    ids = _routing(T, k, E, 1)
    x = _bf16_bits(rng.standard_normal((T, K)))
    g1 = rng.integers(-4, 5, (T * k, N)).astype(np.float64)
    g2 = rng.integers(-4, 5, (T * k, N)).astype(np.float64)
    d1 = wgrad.wgrad(x, _bf16_bits(g1), ids, k, E)
    d2 = wgrad.wgrad(x, _bf16_bits(g2), ids, k, E)
    d3 = wgrad.wgrad(x, _bf16_bits(2 * g1 - g2), ids, k, E)
    np.testing.assert_allclose(d3, 2 * d1 - d2, rtol=1e-12, atol=1e-12)


def test_zero_grad_and_unrouted_slots_contribute_nothing():
    rng = np.random.default_rng(2)
    T, k, E, N, K = 10, 2, 4, 5, 6
    ids = _routing(T, k, E, 2)
    x = _bf16_bits(rng.standard_normal((T, K)))
    gr = _bf16_bits(rng.standard_normal((T * k, N)))
    base = wgrad.wgrad(x, gr, ids, k, E)
    # zero-padded tokens: extra tokens whose grad rows are zero
    x2 = np.concatenate([x, _bf16_bits(rng.standard_normal((3, K)))])
    ids2 = np.concatenate([ids, _routing(3, k, E, 9)])
    gr2 = np.concatenate([gr, _bf16_bits(np.zeros((3 * k, N)))])
    np.testing.assert_array_equal(wgrad.wgrad(x2, gr2, ids2, k, E), base)
    # unrouted slots (ids outside [0, E)) with non-zero grad
    ids3 = np.concatenate([ids, np.full((3, k), E)])
    gr3 = np.concatenate([gr, _bf16_bits(np.ones((3 * k, N)))])
    np.testing.assert_array_equal(wgrad.wgrad(x2, gr3, ids3, k, E), base)


def test_fraction_brute_force_and_scalar_loop():
    rng = np.random.default_rng(3)
    T, k, E, N, K = 6, 2, 3, 4, 5
    ids = _routing(T, k, E, 3)
    x = _bf16_bits(rng.standard_normal((T, K)))
    gr = _bf16_bits(rng.standard_normal((T * k, N)))
    xv, gv = _vals(x), _vals(gr)
    flat = ids.reshape(-1)
    dw = wgrad.wgrad(x, gr, ids, k, E)
    for e in range(E):
        for n in range(N):
            for kk in range(K):
                exact = sum((Fraction(float(gv[s, n])) * Fraction(float(xv[s // k, kk]))
                             for s in range(T * k) if flat[s] == e), Fraction(0))
                assert abs(Fraction(float(dw[e, n, kk])) - exact) <= Fraction(1, 2 ** 48) * (1 + abs(exact))
    # scalar loop in float64, the same sum in slot order
    loop = np.zeros((E, N, K))
    for s in range(T * k):
        loop[flat[s]] += np.outer(gv[s], xv[s // k])
    np.testing.assert_allclose(dw, loop, rtol=1e-13, atol=1e-13)


def test_expert_subset():
    rng = np.random.default_rng(4)
    T, k, E, N, K = 8, 2, 5, 3, 4
    ids = _routing(T, k, E, 4)
    x = _bf16_bits(rng.standard_normal((T, K)))
    gr = _bf16_bits(rng.standard_normal((T * k, N)))
    full = wgrad.wgrad(x, gr, ids, k, E)
    np.testing.assert_array_equal(wgrad.wgrad(x, gr, ids, k, E, experts=[4, 1]), full[[4, 1]])
