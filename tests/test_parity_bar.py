"""The parity bar of a top-k combine (tests/helpers.py, combine_scale): it
admits what storing C and then y in bf16 does to y, also where the weighted
sum cancels most of its terms, and still rejects the mistakes a
combine can make (a dropped term, weights read per slot in the wrong order,
a slot taken from the wrong token)."""

import numpy as np
import torch

from helpers import REL, combine_scale
from oracle import gemm as ogemm


def _bf16(a):
    return torch.from_numpy(a).to(torch.bfloat16).double().numpy()


def _case(seed, T=64, k=7, N=96):
    rng = np.random.default_rng(seed)
    w = rng.uniform(0.05, 0.4, size=(T, k))
    c = rng.normal(0, 1, size=(T * k, N)) * 300.0
    # cancellation: the last term of each token undoes most of the others
    c3 = c.reshape(T, k, N)
    c3[:, -1] = -(np.einsum("tj,tjn->tn", w[:, :-1], c3[:, :-1]) / w[:, -1:]) + rng.normal(0, 1, (T, N))
    return c3.reshape(T * k, N), w


def _err(y, ref):
    return np.abs(y - ref).max()


def test_bf16_stored_c_is_inside_the_bar_and_outside_the_plain_one():
    c, w = _case(5)
    k = w.shape[1]
    ref = ogemm.combine(c, w, k)
    # the GPU's combine: C rounded to bf16 when stored, y rounded when stored
    y = _bf16(ogemm.combine(_bf16(c), w, k))
    err = _err(y, ref)
    assert err <= REL * combine_scale(c, w, k)
    # against |y| alone the same, correct, result would fail: the case is one
    # the plain bar cannot hold
    assert err > REL * np.abs(ref).max()


def test_two_roundings_just_above_a_power_of_two():
    # C rounds down by nearly half a unit (64.249 -> 64, 64.749 -> 64.5), the
    # combine lands on 64.25, a tie that y's own store takes down to 64: y is
    # 0.499 below 64.499, 7.7e-3 of it, past the plain bar and inside this one
    c = np.array([[64.249], [64.749]])
    w = np.array([[0.5, 0.5]])
    ref = ogemm.combine(c, w, 2)
    y = _bf16(ogemm.combine(_bf16(c), w, 2))
    assert y[0, 0] == 64.0
    err = _err(y, ref)
    assert REL * np.abs(ref).max() < err <= REL * combine_scale(c, w, 2)


def test_combine_mistakes_fail_the_bar():
    c, w = _case(6, T=16, k=4, N=32)
    c = c * 0 + np.random.default_rng(7).normal(0, 1, c.shape)   # no cancellation here
    T, k = w.shape
    ref = ogemm.combine(c, w, k)
    bar = REL * combine_scale(c, w, k)
    c3 = c.reshape(T, k, -1)
    for j in range(k):                                   # one term dropped
        y = ref - w[:, j:j + 1] * c3[:, j]
        assert _err(y, ref) > bar, j
    y = ogemm.combine(c, w[:, ::-1], k)                  # weights in reverse slot order
    assert _err(y, ref) > bar
    y = ogemm.combine(np.roll(c, k, axis=0), w, k)       # slots of the neighbouring token
    assert _err(y, ref) > bar


def test_scale_ignores_nan_rows_and_empty_inputs():
    c = np.array([[1.0, -2.0], [3.0, 4.0], [np.nan, 1.0], [2.0, 2.0]])
    w = np.array([[0.5, 0.25], [1.0, 1.0]])
    # token 0: 1.25 + 1.25 and 2 + 0; token 1: NaN and 3 + 3
    assert combine_scale(c, w, 2) == 6.0
    assert combine_scale(np.zeros((0, 8)), np.zeros((0, 2)), 2) == 0.0
