"""Pins the K-block layout definition (oracle.layout) to a per-element loop
over its index formula: code (e, n, k) of the rows layout must sit at
[e, k // 64, n, k % 64] (bytes of two E2M1 codes: [e, k // 64, n, (k % 64) // 2]),
scale byte (e, n, b) at [e, b // 2, n, b % 2], everything else zero."""

import numpy as np
import pytest

from oracle import layout


@pytest.mark.parametrize("w_dtype", ["bf16", "e4m3", "e2m1x2"])
@pytest.mark.parametrize("K", [64, 96, 192, 224])
def test_pack_kblock_matches_index_formula(w_dtype, K):
    rng = np.random.default_rng(K)
    E, N = 3, 5
    U = K // 2 if w_dtype == "e2m1x2" else K
    dt = np.uint16 if w_dtype == "bf16" else np.uint8
    w = rng.integers(1, np.iinfo(dt).max, size=(E, N, U), dtype=dt)  # nonzero: zeros mark the padding
    s = rng.integers(1, 255, size=(E, N, K // 32), dtype=np.uint8)
    pw, ps = layout.pack_kblock(w, w_dtype, s)
    nblk = -(-K // 64)
    assert pw.shape == (E, nblk, N, layout.row_units(w_dtype)) and ps.shape == (E, nblk, N, 2)
    seen = np.zeros(pw.shape, dtype=bool)
    for e in range(E):
        for n in range(N):
            for k in range(K):
                if w_dtype == "e2m1x2":
                    if k % 2:
                        continue
                    pos = (e, k // 64, n, (k % 64) // 2)
                    val = w[e, n, k // 2]
                else:
                    pos = (e, k // 64, n, k % 64)
                    val = w[e, n, k]
                assert pw[pos] == val
                seen[pos] = True
    assert np.all(pw[~seen] == 0)
    sseen = np.zeros(ps.shape, dtype=bool)
    for e in range(E):
        for n in range(N):
            for b in range(K // 32):
                assert ps[e, b // 2, n, b % 2] == s[e, n, b]
                sseen[e, b // 2, n, b % 2] = True
    assert np.all(ps[~sseen] == 0)


def test_pack_kblock_without_scales():
    w = np.arange(2 * 3 * 128, dtype=np.uint16).reshape(2, 3, 128)
    pw, ps = layout.pack_kblock(w, "bf16")
    assert ps is None
    assert np.array_equal(pw[:, 1, :, :], w[:, :, 64:])
