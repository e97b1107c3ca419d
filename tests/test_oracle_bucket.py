"""Pins for the oracle's token-dimension bucketing: the properties and the
count that the TensorRT-LLM page prints, checked exhaustively."""

import numpy as np
import pytest

from oracle import bucket


@pytest.fixture(scope="module")
def table(page_facts):
    lo, hi = page_facts["bucket"]["exhaustive_range"]
    m = np.arange(lo, hi + 1)
    b = np.array([bucket.bucket_round_up(int(v)) for v in m])
    return m, b


def test_round_up_bound(table, page_facts):
    m, b = table
    frac = page_facts["bucket"]["max_pad_fraction"]
    assert np.all(b >= m)
    # (b - m) / m <= 1/8, in integers: 8 b <= 9 m
    assert np.all(8 * b <= 9 * m)
    assert ((b - m) / m).max() <= frac


def test_fixed_point_and_monotonic(table):
    m, b = table
    bb = np.array([bucket.bucket_round_up(int(v)) for v in b])
    np.testing.assert_array_equal(bb, b)
    assert np.all(np.diff(b) >= 0)


def test_eight_per_octave(table, page_facts):
    m, b = table
    per = page_facts["bucket"]["buckets_per_octave"]
    values = np.unique(b)
    for p in range(3, 16):  # octaves [8, 16) ... [32768, 65536)
        inside = values[(values >= 2 ** p) & (values < 2 ** (p + 1))]
        assert inside.size == per, (p, inside)


def test_enumeration_is_closure(page_facts):
    mx = page_facts["bucket"]["max_num_tokens"]
    en = bucket.bucket_enumerate(mx)
    assert en == sorted(set(en))
    # the closure: values reached by some m <= mx, found by brute force
    reached = set()
    for m in range(1, mx + 1):
        reached.add(bucket.bucket_round_up(m))
    assert set(en) == reached
    # every member is a fixed point
    assert all(bucket.bucket_round_up(v) == v for v in en)


def test_printed_bucket_count(page_facts):
    f = page_facts["bucket"]
    assert len(bucket.buckets_up_to(f["max_num_tokens"])) == f["buckets_up_to_max"]
    # the closure holds one more value: the bucket of the counts above the
    # largest bucket <= 20000 (18433..20000 -> 20480)
    en = bucket.bucket_enumerate(f["max_num_tokens"])
    assert len(en) == f["buckets_up_to_max"] + 1
    assert en[-1] == 20480


def test_small_and_edge_values():
    assert bucket.bucket_round_up(0) == 0
    assert [bucket.bucket_round_up(m) for m in range(1, 17)] == list(range(1, 17))
    assert bucket.bucket_round_up(17) == 18
    assert bucket.bucket_round_up(6554) == 6656
    assert bucket.bucket_round_up(8192) == 8192
    assert bucket.bucket_round_up(8193) == 9216
    with pytest.raises(ValueError):
        bucket.bucket_round_up(-1)


def test_gpt_oss_token_range_buckets():
    # token counts uniform in [6554, 8192] land on four buckets
    got = sorted({bucket.bucket_round_up(m) for m in range(6554, 8193)})
    assert got == [6656, 7168, 7680, 8192]
