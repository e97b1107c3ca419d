"""The W4A16 MXFP4 expert layer and the bf16 squared-ReLU decode layer as
compositions (oracle; test infrastructure only).

Source: TensorRT-LLM PR #15311 "Bound Triton MoE JIT specializations via
token-dim bucketing and warmup", Description: W4A16 MXFP4 grouped GEMMs with
bf16 activations; the token dimension is padded to a bucket before the grouped
GEMMs and sliced back afterwards; rows are independent, so padded rows cannot
change real tokens' outputs. The layer is gate+up GEMM -> SwiGLU -> down GEMM
-> top-k combine, with nothing rounded in between.
"""

import numpy as np

from .gemm import grouped_gemm, combine


def w4a16_layer(x, topk_ids, topk_w, top_k, num_experts,
                w1, s1, b1, w2, s2, b2, slots=None):
    """Return (h, c2, y) in float64.

    x bf16 bits [T, K]; w1 E2M1 bytes [E, 2I, K/2] with scales s1 [E, 2I, K/32];
    w2 E2M1 bytes [E, H, I/2] with s2 [E, H, I/32]; b1, b2 bf16 bits or None.
    h [S, I], c2 [S, H], y [T, H]. With `slots`, only those slots of h and c2
    are computed and y is not formed (returned as None).
    Pinned: tests/test_oracle_layer.py (padded == unpadded on real rows, and
    the composition equals its pinned parts).
    """
    h, routed = grouped_gemm(x, top_k, w1, "e2m1x2", s1, topk_ids, num_experts,
                             bias=b1, epilogue="swiglu", slots=slots)
    # The down GEMM reads h over slot rows (a_row_div = 1), in float64, unrounded.
    c2, _ = grouped_gemm(h, 1, w2, "e2m1x2", s2, topk_ids, num_experts,
                         bias=b2, a_dtype="f64", slots=np.nonzero(routed)[0])
    y = None if slots is not None else combine(c2, topk_w, top_k)
    return h, c2, y


def relu2_layer(x, topk_ids, topk_w, top_k, num_experts, w1, b1, w2, b2):
    """The non-gated squared-ReLU MoE layer of torchada PR #115's Nemotron
    shape ("Follow-up on this table": E=128, hidden 2688, N=1856, top-6,
    non-gated relu2, bf16): up GEMM -> relu2 -> down GEMM -> top-k combine,
    nothing rounded in between. Return (h, c2, y) in float64.

    x bf16 bits [T, H]; w1 bf16 bits [E, N, H]; w2 bf16 bits [E, H, N]; b1,
    b2 bf16 bits or None. h [S, N], c2 [S, H], y [T, H].
    Pinned: tests/test_oracle_layer.py (the composition equals its pinned
    parts; a constant-input closed form).
    """
    h, routed = grouped_gemm(x, top_k, w1, "bf16", None, topk_ids, num_experts, bias=b1, epilogue="relu2")
    c2, _ = grouped_gemm(h, 1, w2, "bf16", None, topk_ids, num_experts, bias=b2, a_dtype="f64",
                         slots=np.nonzero(routed)[0])
    return h, c2, combine(c2, topk_w, top_k)
