"""Pins for the oracle's routing (moe_align): a hand-worked example, brute
force with Python's sorted() on tiny inputs, and the structural invariants the
aiter page fixes (homogeneous blocks, -1 sentinel blocks past the used ones)."""

import numpy as np
import pytest

from oracle import align


def test_hand_worked_example():
    # T=3 tokens, top_k=2, E=4 experts, BLOCK_M=4.
    # slots: s0->2, s1->0, s2->0, s3->3, s4->3, s5->2
    # counts 2,0,2,2 -> padded 4,0,4,4 -> offsets 0,4,4,8, P=12.
    # max_blocks = (6 + min(4,6)*3) // 4 = 4, so 16 positions, PAD = 6.
    ids = np.array([[2, 0], [0, 3], [3, 2]])
    s, e, p = align.moe_align(ids, 4, 4)
    assert s.tolist() == [1, 2, 6, 6, 0, 5, 6, 6, 3, 4, 6, 6, 6, 6, 6, 6]
    assert e.tolist() == [0, 2, 3, -1]
    assert p == 12


def _brute(ids, E, B):
    flat = [int(v) for v in np.asarray(ids).reshape(-1)]
    S = len(flat)
    pairs = sorted((v, s) for s, v in enumerate(flat) if 0 <= v < E)
    nb = (S + min(E, S) * (B - 1)) // B
    out = [S] * (nb * B)
    blocks = [-1] * nb
    pos = 0
    for ex in range(E):
        mine = [s for (v, s) in pairs if v == ex]
        for r, s in enumerate(mine):
            out[pos + r] = s
        padded = -(-len(mine) // B) * B
        for b in range(pos // B, (pos + padded) // B):
            blocks[b] = ex
        pos += padded
    return out, blocks, pos


@pytest.mark.parametrize("seed", range(40))
def test_brute_force_tiny(seed):
    rng = np.random.default_rng(seed)
    T = int(rng.integers(0, 12))
    k = int(rng.integers(1, 4))
    E = int(rng.integers(1, 9))
    B = int(rng.choice([1, 2, 3, 4, 8, 16]))
    ids = rng.integers(-1, E + 2, size=(T, k))  # includes out-of-range ids
    s, e, p = align.moe_align(ids, E, B)
    bs, be, bp = _brute(ids, E, B)
    assert s.tolist() == bs
    assert e.tolist() == be
    assert p == bp


@pytest.mark.parametrize("T,k,E,B", [(64, 2, 8, 16), (300, 6, 128, 16), (2048, 4, 128, 64), (4096, 8, 256, 32)])
def test_invariants(T, k, E, B):
    rng = np.random.default_rng(T + E)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    S = T * k
    s, e, P = align.moe_align(ids, E, B)
    nb = align.max_blocks(S, E, B)
    assert s.size == nb * B and e.size == nb
    flat = ids.reshape(-1)
    real = s[s < S]
    # every routed slot exactly once
    assert np.array_equal(np.sort(real), np.arange(S))
    assert np.all(s[s >= S] == S)
    assert P % B == 0 and P <= nb * B
    # blocks are homogeneous and ascending in slot order; sentinels past P
    assert np.all(e[P // B:] == -1) and np.all(e[:P // B] >= 0)
    for b in range(P // B):
        blk = s[b * B:(b + 1) * B]
        r = blk[blk < S]
        assert np.all(flat[r] == e[b])
    # per-expert segments: ascending, padded by less than B
    counts = np.bincount(flat, minlength=E)
    for ex in range(E):
        seg_blocks = np.nonzero(e == ex)[0]
        assert seg_blocks.size * B - counts[ex] in range(0, B)
        if seg_blocks.size:
            seg = s[seg_blocks[0] * B:(seg_blocks[-1] + 1) * B]
            r = seg[seg < S]
            assert np.all(np.diff(r) > 0) and r.size == counts[ex]
    # expert segments appear in expert order
    used = e[:P // B]
    assert np.all(np.diff(used) >= 0)


def test_empty_input():
    s, e, p = align.moe_align(np.zeros((0, 4), dtype=np.int64), 8, 16)
    assert s.size == 0 and e.size == 0 and p == 0


def test_max_blocks_bound_is_tight():
    # every expert gets exactly one slot -> each wastes B-1 positions
    E, B = 8, 16
    ids = np.arange(E).reshape(E, 1)
    s, e, p = align.moe_align(ids, E, B)
    assert p == E * B == align.max_blocks(E, E, B) * B
    assert np.all(e >= 0)  # no sentinel block is guaranteed
