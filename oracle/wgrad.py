"""Expert weight gradient (oracle; test infrastructure only).

Source: ROCm/aiter PR #5310 "Add MoE GEMM variants and weight-gradient
kernel", Summary (moe_wgrad: dW[e] = sum over the tokens routed to e of
grad[t]^T x input[t], over the sorted_token_ids / expert_ids of
moe_align_block_size, replacing a sort + pad + bmm) and Tests & Benchmarks
(analytical constant-input check, linearity, zero-padded-token guard).

Readings: grad is indexed by slot s = t * top_k + j and the input by token
s // top_k; no routing-weight factor; padded slots contribute nothing; dW is
overwritten, and an expert with no slots gets zeros.

The plain definition: dW[e] = G_e^T X_e, G_e the grad rows of e's slots and
X_e the input rows of their tokens, as one float64 matrix product per expert.
A full-size dW in float64 does not fit in host memory, so callers pick experts.
"""

import numpy as np

from .formats import bf16_to_f64


def wgrad_expert(x, grad, topk_ids, top_k, expert):
    """dW[expert] [N, K] in float64.

    x: bf16 bit patterns [T, K]; grad: bf16 bit patterns [S, N];
    topk_ids: [T, top_k] (or flat [S]).
    Pinned: tests/test_oracle_wgrad.py (constant input, linearity,
    zero-grad and out-of-range slots, Fraction brute force, scalar loop).
    """
    ids = np.asarray(topk_ids).reshape(-1).astype(np.int64)
    slots = np.nonzero(ids == int(expert))[0]
    N = grad.shape[1]
    K = x.shape[1]
    if slots.size == 0:
        return np.zeros((N, K), dtype=np.float64)
    g = bf16_to_f64(grad[slots])            # [M_e, N]
    xe = bf16_to_f64(x[slots // top_k])     # [M_e, K]
    return g.T @ xe


def wgrad(x, grad, topk_ids, top_k, num_experts, experts=None):
    """dW for the listed experts (all by default): float64 [len(experts), N, K]."""
    if experts is None:
        experts = range(int(num_experts))
    return np.stack([wgrad_expert(x, grad, topk_ids, top_k, e) for e in experts])
