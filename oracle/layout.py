"""Definition of the library's K-block weight layout (oracle; test
infrastructure only).

Not a step of the method: the pages' kernels read expert weights row by row,
[E][N][K]. The library also accepts the same codes regrouped so that, for
every 64-element K block, all N rows' pieces of that block lie back to back:
    packed[e, kb, n, j] = rows[e, n, kb*R + j]     (j < R, kb*R + j < row length)
with R = 64 storage units per row per block (elements; 32 bytes of two E2M1
codes), zero where the last block runs past K; and the E8M0 scale bytes
    packed_scale[e, kb, n, i] = scale[e, n, 2*kb + i]   (zero past K/32).
This module writes that definition out with numpy slicing; the test pins it
against a per-element loop over the index formula.
"""

import numpy as np


def row_units(w_dtype):
    """Storage units per row per 64-element K block."""
    return 32 if w_dtype == "e2m1x2" else 64


def pack_kblock(w, w_dtype, scale=None):
    """Rows-layout codes w [E, N, U] (U = K, or K/2 bytes for e2m1x2) and
    scales [E, N, K/32] -> (packed codes [E, ceil(K/64), N, R],
    packed scales [E, ceil(K/64), N, 2] or None)."""
    w = np.asarray(w)
    E, N, U = w.shape
    R = row_units(w_dtype)
    nblk = -(-U // R)
    out = np.zeros((E, nblk, N, R), dtype=w.dtype)
    for kb in range(nblk):
        piece = w[:, :, kb * R:(kb + 1) * R]
        out[:, kb, :, :piece.shape[2]] = piece
    sout = None
    if scale is not None:
        scale = np.asarray(scale)
        nsb = scale.shape[2]
        sout = np.zeros((E, nblk, N, 2), dtype=scale.dtype)
        for kb in range(nblk):
            for i in range(2):
                if 2 * kb + i < nsb:
                    sout[:, kb, :, i] = scale[:, :, 2 * kb + i]
    return out, sout
