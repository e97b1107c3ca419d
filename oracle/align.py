"""Routing: sort (token, slot) pairs by expert and pad each expert to BLOCK_M
(oracle; test infrastructure only).

Sources: ROCm/aiter PR #5310 "Add MoE GEMM variants and weight-gradient
kernel", Summary (moe_wgrad consumes sorted_token_ids / expert_ids from
moe_align_block_size) and the second review (the block list is sized above the
real block count; padded blocks carry expert id -1 and must exit at once);
torchada PR #115 "tune the Nemotron MTP decode row on S5000 with a checked-in
recipe", "Follow-up on this table" (moe_align_block_size is the routing op
that runs before the fused MoE kernel).

Readings where the pages are silent:
  * slot s = t * top_k + j indexes the flattened topk_ids [T, top_k];
  * PAD = S (the number of slots) marks a padded position;
  * inside one expert, slots appear in ascending order (a stable sort), so the
    output is unique;
  * expert ids outside [0, E) are not routed anywhere;
  * the block list has max_blocks = floor((S + min(E, S) * (B - 1)) / B)
    entries, enough for any routing of S slots; entries past the used blocks
    hold -1.
"""

import numpy as np


def max_blocks(num_slots, num_experts, block_m):
    """Upper bound on the number of BLOCK_M blocks any routing can use."""
    S, E, B = int(num_slots), int(num_experts), int(block_m)
    return (S + min(E, S) * (B - 1)) // B


def moe_align(topk_ids, num_experts, block_m):
    """Return (sorted_token_ids, expert_ids, num_tokens_post_pad).

    For expert e: c_e = #slots routed to e, p_e = ceil(c_e / B) * B,
    o_e = sum of p_e' over e' < e, P = sum of all p_e.
    sorted_token_ids[o_e + r] is the r-th smallest slot routed to e (r < c_e);
    every other position of the [max_blocks * B] array is PAD = S.
    expert_ids[b] = e for o_e / B <= b < (o_e + p_e) / B, and -1 from P / B on.

    Pinned: tests/test_oracle_align.py (brute force with Python's sorted() on
    tiny inputs, structural invariants, a hand-worked example).
    """
    ids = np.asarray(topk_ids).reshape(-1).astype(np.int64)
    S = ids.size
    E, B = int(num_experts), int(block_m)
    nb = max_blocks(S, E, B)
    pad = S
    sorted_ids = np.full(nb * B, pad, dtype=np.int64)
    expert_ids = np.full(nb, -1, dtype=np.int64)
    offset = 0
    slots = np.arange(S, dtype=np.int64)
    for e in range(E):
        mine = slots[ids == e]  # ascending slot order: stable
        c = mine.size
        p = -(-c // B) * B
        sorted_ids[offset:offset + c] = mine
        expert_ids[offset // B:(offset + p) // B] = e
        offset += p
    return sorted_ids, expert_ids, offset
