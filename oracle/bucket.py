"""Token-dimension bucketing (oracle; test infrastructure only).

Source: TensorRT-LLM PR #15311 "Bound Triton MoE JIT specializations via
token-dim bucketing and warmup", Description: the MoE token dimension is
padded up to geometric buckets, eight per power-of-two octave, with at most
12.5% padding, which makes the set of padded sizes finite (97 buckets for
max_num_tokens = 20000); Test Coverage: round-up by at most 12.5%, fixed
point, monotonic, enumeration equal to the closure.

The page states only these properties. The reading taken here (the plainest
rule that has all of them): a bucket is an integer with at most four
significant bits. Below 16 every integer qualifies; from 16 up, round m up to
a multiple of 2^(bitlen(m) - 4), which leaves eight values in each octave
[2^p, 2^(p+1)).
"""


def bucket_round_up(m):
    """Smallest bucket >= m. bucket(0) = 0; negative m is an error.

    Pinned: tests/test_oracle_bucket.py (exhaustive properties on [1, 65536]
    and the printed count of 97 buckets up to 20000).
    """
    m = int(m)
    if m < 0:
        raise ValueError("token count must be >= 0")
    if m < 16:
        return m
    step = 1 << (m.bit_length() - 4)
    return ((m + step - 1) // step) * step


def bucket_enumerate(max_tokens):
    """Sorted closure {bucket(m) : 1 <= m <= max_tokens}: every padded size
    that a token count up to max_tokens can produce (it may contain one value
    above max_tokens, the bucket of the largest counts)."""
    return sorted({bucket_round_up(m) for m in range(1, int(max_tokens) + 1)})


def buckets_up_to(max_tokens):
    """Sorted buckets b with 1 <= b <= max_tokens (the page's count of 97 for
    20000 counts these)."""
    return [b for b in bucket_enumerate(max_tokens) if b <= max_tokens]
