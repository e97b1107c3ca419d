"""Routed grouped GEMM, SwiGLU and top-k combine (oracle; test infrastructure
only).

Sources: ROCm/aiter PR #5310 "Add MoE GEMM variants and weight-gradient
kernel", Summary (moe_gemm_mxfp8: every expert's GEMM over its own tokens in
one launch; E8M0 microscales, one per 32 K-elements, applied per K-iteration;
optional per-expert bias), Notes (BLOCK_K equals the scale block; int64 expert
offsets) and the second review (bias indexed with explicit strides);
TensorRT-LLM PR #15311, Description (W4A16 MXFP4: bf16 activations against
MXFP4 weights; rows are independent); torchada PR #115, What it does (bf16
fused-MoE decode at M <= 32, same math). SwiGLU and the top-k combine are named
by the method's description but defined on none of the pages; the textbook
forms are used: silu(z) = z / (1 + e^-z), h = silu(gate) * up with gate the
first N/2 output columns and up the last N/2, y[t] = sum_j w[t, j] * C[t*k + j].

Definition (for every routed slot s, e = topk_ids[s] in [0, E)):
    pre[s] = A[s // a_row_div] . W_hat[e]^T + bias[e]
    W_hat[e][n, k] = dec(W[e, n, k]) * 2^(scale[e, n, k // 32] - 127)
computed per expert as a gathered dense float64 product (the plain
"sort + pad + bmm" form). Nothing is rounded.
"""

import numpy as np

from .formats import bf16_to_f64, e4m3_to_f64, e2m1_to_f64, e2m1x2_unpack, e8m0_to_f64

QUANT_BLOCK = 32


def _apply_block_scale(values, scale_codes):
    """values [R, K] * 2^(scale[R, K // 32] - 127)."""
    s = e8m0_to_f64(scale_codes)  # [R, K/32]
    return values * np.repeat(s, QUANT_BLOCK, axis=-1)[..., :values.shape[-1]]


def dequant_expert(w_codes, w_dtype, w_scale=None):
    """One expert's weights [N, K] (codes) -> float64 W_hat [N, K].

    w_dtype: "bf16" (uint16 bit patterns, no scale), "e4m3" (uint8 codes,
    scale [N, K/32]) or "e2m1x2" (uint8 bytes [N, K/2], two codes per byte,
    scale [N, K/32]).
    Pinned: tests/test_oracle_gemm.py (constant-input closed form, brute force).
    """
    if w_dtype == "bf16":
        return bf16_to_f64(w_codes)
    if w_dtype == "e4m3":
        return _apply_block_scale(e4m3_to_f64(w_codes), w_scale)
    if w_dtype == "e2m1x2":
        return _apply_block_scale(e2m1_to_f64(e2m1x2_unpack(w_codes)), w_scale)
    raise ValueError(f"unknown weight dtype {w_dtype}")


def dequant_act(a_codes, a_dtype, a_scale=None):
    """Activation rows -> float64: "bf16" (uint16 bit patterns), "e4m3"
    (uint8 codes with E8M0 scale [R, K/32], the both-operands-MXFP8 form) or
    "f64" (values already in float64, e.g. an earlier GEMM's unrounded output).

    Pinned (the "e4m3" form, through grouped_gemm with a_scale indexed by
    the activation row s // a_row_div): tests/test_oracle_gemm.py (constant
    codes with scales that vary per row and per K block, a Fraction triple
    loop decoded by torch's float8_e4m3fn, one scale row per token).
    """
    if a_dtype == "f64":
        return np.asarray(a_codes, dtype=np.float64)
    if a_dtype == "bf16":
        return bf16_to_f64(a_codes)
    if a_dtype == "e4m3":
        return _apply_block_scale(e4m3_to_f64(a_codes), a_scale)
    raise ValueError(f"unknown activation dtype {a_dtype}")


def silu(z):
    """silu(z) = z / (1 + e^-z); for very negative z this tends to -0.

    Pinned: tests/test_oracle_gemm.py (silu(0) = 0, silu(ln 3) = 0.75 ln 3,
    silu(z) - silu(-z) = z).
    """
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def relu2(pre):
    """The non-gated squared ReLU of torchada PR #115's Nemotron decode shape
    ("Follow-up on this table": the recipe records a non-gated relu2 layer):
    h = max(pre, 0)^2, elementwise, same width.

    Pinned: tests/test_oracle_gemm.py (closed forms on both sides of 0).
    """
    pre = np.asarray(pre, dtype=np.float64)
    return np.where(pre > 0, pre * pre, 0.0)


def swiglu(pre):
    """pre [R, N] -> h [R, N/2] with h[:, j] = silu(pre[:, j]) * pre[:, N/2 + j]."""
    n = pre.shape[-1]
    if n % 2:
        raise ValueError("SwiGLU needs an even number of columns")
    half = n // 2
    return silu(pre[..., :half]) * pre[..., half:]


def grouped_gemm(a, a_row_div, w, w_dtype, w_scale, topk_ids, num_experts,
                 bias=None, epilogue="none", a_dtype="bf16", a_scale=None,
                 slots=None):
    """Routed grouped GEMM.

    a        activation codes [R, K] (bf16 bit patterns, or E4M3 codes with a_scale)
    a_row_div  slot s reads activation row s // a_row_div (top_k for a GEMM
               over token rows, 1 for a GEMM over slot rows)
    w        weight codes [E, N, K] ("bf16", "e4m3") or [E, N, K/2] ("e2m1x2")
    w_scale  E8M0 bytes [E, N, K/32] (None for bf16)
    topk_ids routing [T, top_k] (or flat [S])
    bias     bf16 bit patterns [E, N] or None (added before the epilogue)
    epilogue "none", "swiglu" (output width N/2) or "relu2" (max(pre, 0)^2)
    slots    optional subset of slots to compute (for sampled checks)

    Returns (C, routed): C float64 [S, N_out] (rows of unrouted or unrequested
    slots are zero) and the boolean mask of rows computed.
    Pinned: tests/test_oracle_gemm.py.
    """
    ids = np.asarray(topk_ids).reshape(-1).astype(np.int64)
    S = ids.size
    E = int(num_experts)
    N = w.shape[1]
    n_out = N // 2 if epilogue == "swiglu" else N
    C = np.zeros((S, n_out), dtype=np.float64)
    want = np.zeros(S, dtype=bool)
    if slots is None:
        want[:] = True
    else:
        want[np.asarray(slots, dtype=np.int64)] = True
    routed = want & (ids >= 0) & (ids < E)
    all_slots = np.arange(S, dtype=np.int64)
    for e in np.unique(ids[routed]):
        rows = all_slots[routed & (ids == e)]
        w_hat = dequant_expert(w[e], w_dtype, None if w_scale is None else w_scale[e])
        a_rows = dequant_act(a[rows // a_row_div], a_dtype,
                             None if a_scale is None else a_scale[rows // a_row_div])
        pre = a_rows @ w_hat.T
        if bias is not None:
            pre = pre + bf16_to_f64(bias[e])[None, :]
        if epilogue == "swiglu":
            pre = swiglu(pre)
        elif epilogue == "relu2":
            pre = relu2(pre)
        elif epilogue != "none":
            raise ValueError(f"unknown epilogue {epilogue}")
        C[rows] = pre
    return C, routed


def combine(c, topk_w, top_k):
    """y[t] = sum_{j < top_k} w[t, j] * c[t * top_k + j], j ascending.

    c float64 [S, N]; topk_w [T, top_k]. Pinned: tests/test_oracle_gemm.py.
    """
    w = np.asarray(topk_w, dtype=np.float64).reshape(-1, top_k)
    T = w.shape[0]
    c = np.asarray(c, dtype=np.float64).reshape(T, top_k, -1)
    y = np.zeros((T, c.shape[-1]), dtype=np.float64)
    for j in range(top_k):
        y += w[:, j:j + 1] * c[:, j, :]
    return y


def build_block_mapping(group_sizes, block_m, max_blocks):
    """The expert block mapping of a group_sizes interface (ROCm/aiter PR
    #5310, Notes: _build_block_mapping shared by the GEMM wrappers; second
    review: block_expert_ids / block_token_offsets / block_token_ends, -1
    sentinels in the padded tail). Expert e owns rows [o_e, o_e + g_e) with
    o_e = g_0 + ... + g_{e-1}, cut into ceil(g_e / block_m) blocks in expert
    order; block i of e starts at o_e + i * block_m and its segment ends at
    o_e + g_e. Blocks past the used ones: expert -1, offset = end = total rows.

    Returns (expert_ids, token_offsets, token_ends), int64 [max_blocks].
    Pinned: tests/test_oracle_gemm.py (hand-worked example, empty groups,
    every row in exactly one block).
    """
    g = np.asarray(group_sizes, dtype=np.int64)
    total = int(g.sum())
    eid = np.full(max_blocks, -1, dtype=np.int64)
    beg = np.full(max_blocks, total, dtype=np.int64)
    end = np.full(max_blocks, total, dtype=np.int64)
    b, o = 0, 0
    for e, n in enumerate(g):
        for i in range(-(-int(n) // block_m)):
            assert b < max_blocks, "max_blocks too small"
            eid[b], beg[b], end[b] = e, o + i * block_m, o + n
            b += 1
        o += int(n)
    return eid, beg, end


def grouped_gemm_per_token(a_codes, a_scale, w, w_scale, group_sizes, bias=None):
    """Per-token-scaled FP8 grouped GEMM over expert-contiguous rows (ROCm/
    aiter PR #5310, Summary: moe_gemm_per_token, per-token activation scales
    and per-expert weight scales applied after the FP8 dot product, a
    group_sizes interface; Tests & Benchmarks: a bias variant):
        C[r, n] = (sum_k dec(A[r, k]) dec(W[e, n, k])) * a_scale[r] * w_scale[e] + bias[e, n]
    for the rows r of expert e's segment. a_codes E4M3 [R, K]; a_scale
    float [R]; w E4M3 [E, N, K]; w_scale float [E]; bias bf16 bits [E, N] or
    None. Returns float64 [R, N].
    Pinned: tests/test_oracle_gemm.py (constant input, a scalar loop on a tiny
    case, empty groups).
    """
    g = np.asarray(group_sizes, dtype=np.int64)
    a_s = np.asarray(a_scale, dtype=np.float64)
    w_s = np.asarray(w_scale, dtype=np.float64)
    R = int(g.sum())
    C = np.zeros((R, w.shape[1]), dtype=np.float64)
    o = 0
    for e, n in enumerate(g):
        if n:
            rows = slice(o, o + int(n))
            acc = e4m3_to_f64(a_codes[rows]) @ e4m3_to_f64(w[e]).T
            C[rows] = acc * a_s[rows, None] * w_s[e]
            if bias is not None:
                C[rows] += bf16_to_f64(bias[e])[None, :]
        o += int(n)
    return C
