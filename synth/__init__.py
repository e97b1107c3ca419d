"""Seeded synthetic inputs shaped like the pages' workloads.

Shared by the tests (which hand the same tensors to the HIP library and to the
float64 oracle), by bench.py and by the smoke check. This module draws random
numbers and encodes them into the input formats; it holds none of the method's
arithmetic (no decoding, routing sort, GEMM, activation, combine or gradient).

Every tensor comes from its own torch.Generator seeded from (seed, tag), so a
tensor's values do not depend on which other tensors were drawn. Generation
runs on the requested device; the same seed gives the same values on one
device type.

Stand-ins for the pages' workloads (their models, weights and serving traces
are not available): gpt-oss-shaped W4A16 MXFP4 layer, Nemotron-shaped bf16
decode, DSv4-shaped MXFP8 grouped GEMM and weight gradient, all at the shapes
the pages give, with synthetic values.
"""

import hashlib

import torch

__all__ = [
    "gen", "bf16_normal", "e4m3_normal", "e2m1_uniform", "e8m0_uniform",
    "softmax_topk_routing", "zipf_topk_routing", "uniform_topk_routing",
    "gemm_case", "config1", "config2", "config3", "config4", "config5", "nemotron_layer",
    "bits", "draw_token_counts", "f32_uniform", "zipf_group_sizes", "per_token_case", "config_per_token",
]


def gen(seed, tag, device="cpu"):
    """A torch.Generator on `device` seeded from (seed, tag)."""
    h = hashlib.sha256(f"{int(seed)}/{tag}".encode()).digest()
    g = torch.Generator(device=device)
    g.manual_seed(int.from_bytes(h[:8], "little") & ((1 << 63) - 1))
    return g


def bf16_normal(shape, std, seed, tag, device="cpu"):
    """N(0, std^2) rounded to bfloat16 (round-to-nearest-even)."""
    g = gen(seed, tag, device)
    return (torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std).to(torch.bfloat16)


def e4m3_normal(shape, std, seed, tag, device="cpu", chunk_dim0=True):
    """OCP E4M3 (FN) codes (uint8) of N(0, std^2) samples, cast by torch.

    Generated one slice of dim 0 at a time so the fp32 staging stays small.
    """
    g = gen(seed, tag, device)
    out = torch.empty(shape, dtype=torch.uint8, device=device)
    if not chunk_dim0 or len(shape) == 1:
        x = torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std
        return x.to(torch.float8_e4m3fn).view(torch.uint8)
    for i in range(shape[0]):
        x = torch.randn(shape[1:], generator=g, device=device, dtype=torch.float32) * std
        out[i] = x.to(torch.float8_e4m3fn).view(torch.uint8)
    return out


def e2m1_uniform(shape_bytes, seed, tag, device="cpu"):
    """Packed E2M1 bytes, both nibbles uniform over all 16 codes."""
    g = gen(seed, tag, device)
    return torch.randint(0, 256, shape_bytes, generator=g, device=device, dtype=torch.int32).to(torch.uint8)


def e8m0_uniform(shape, lo, hi, seed, tag, device="cpu"):
    """E8M0 scale bytes uniform in [lo, hi] (inclusive)."""
    g = gen(seed, tag, device)
    return torch.randint(lo, hi + 1, shape, generator=g, device=device, dtype=torch.int32).to(torch.uint8)


def softmax_topk_routing(T, E, k, seed, tag="route", device="cpu"):
    """Router stand-in: logits ~ N(0, 1) [T, E], p = softmax over E,
    ids = top-k of p (descending), weights = p[ids] (not renormalised)."""
    g = gen(seed, tag, device)
    logits = torch.randn((T, E), generator=g, device=device, dtype=torch.float32)
    p = torch.softmax(logits, dim=-1)
    w, ids = torch.topk(p, k, dim=-1)
    return ids.to(torch.int32).contiguous(), w.contiguous()


def zipf_topk_routing(T, E, k, s, n_empty, seed, tag="route", device="cpu"):
    """Skewed routing: expert perm[r-1] has probability proportional to r^-s
    (r = 1..E) except the n_empty lowest-ranked experts, which get 0; each
    token draws k distinct experts with probability proportional to p
    (Gumbel top-k). Weights are p of the chosen experts, renormalised."""
    g = gen(seed, tag, device)
    perm = torch.randperm(E, generator=g, device=device)
    ranks = torch.empty(E, dtype=torch.float64, device=device)
    ranks[perm] = torch.arange(1, E + 1, dtype=torch.float64, device=device)
    p = ranks.pow(-s)
    if n_empty:
        p[perm[E - n_empty:]] = 0.0
    p = p / p.sum()
    u = torch.rand((T, E), generator=g, device=device, dtype=torch.float64).clamp_min(1e-300)
    keys = torch.log(p)[None, :] - torch.log(-torch.log(u))
    _, ids = torch.topk(keys, k, dim=-1)
    w = p[ids]
    w = (w / w.sum(-1, keepdim=True)).to(torch.float32)
    return ids.to(torch.int32).contiguous(), w.contiguous()


def uniform_topk_routing(T, E, k, seed, tag="route", device="cpu"):
    """Each token's k experts uniform without replacement; weights 1/k."""
    g = gen(seed, tag, device)
    u = torch.rand((T, E), generator=g, device=device)
    ids = torch.argsort(u, dim=-1)[:, :k]
    w = torch.full((T, k), 1.0 / k, dtype=torch.float32, device=device)
    return ids.to(torch.int32).contiguous(), w


def gemm_case(T, k, E, N, K, w_dtype, seed, bias=False, a_rows=None,
              scale_lo=123, scale_hi=129, w_std=1.0, device="cpu"):
    """A generic routed-GEMM input set.

    a_rows: number of activation rows (T for a GEMM over tokens, T*k for a
    GEMM over slots); w_dtype "bf16" (N(0, w_std^2)), "e4m3" (cast of
    N(0, w_std^2)) or "e2m1x2" (uniform codes); scales uniform in
    [scale_lo, scale_hi] for the MX types.
    """
    a_rows = T if a_rows is None else a_rows
    d = {"T": T, "k": k, "E": E, "N": N, "K": K, "w_dtype": w_dtype}
    d["x"] = bf16_normal((a_rows, K), 1.0, seed, "x", device)
    if w_dtype == "bf16":
        d["w"] = bf16_normal((E, N, K), w_std, seed, "w", device)
        d["w_scale"] = None
    elif w_dtype == "e4m3":
        d["w"] = e4m3_normal((E, N, K), w_std, seed, "w", device)
        d["w_scale"] = e8m0_uniform((E, N, K // 32), scale_lo, scale_hi, seed, "ws", device)
    elif w_dtype == "e2m1x2":
        d["w"] = e2m1_uniform((E, N, K // 2), seed, "w", device)
        d["w_scale"] = e8m0_uniform((E, N, K // 32), scale_lo, scale_hi, seed, "ws", device)
    else:
        raise ValueError(w_dtype)
    d["bias"] = bf16_normal((E, N), 1.0, seed, "bias", device) if bias else None
    d["ids"], d["topk_w"] = softmax_topk_routing(T, E, k, seed, "route", device)
    return d


def config1(seed=1001, device="cpu"):
    """Tiny MXFP8 up-projection: T=64, E=8, top-2 of softmax(N(0,1) logits),
    x bf16 N(0,1) [64, 256], W E4M3 cast of N(0,1) [8, 512, 256], E8M0 scales
    per 32 along K with exponents uniform in [-4, 2] (bytes 123..129)."""
    return gemm_case(64, 2, 8, 512, 256, "e4m3", seed, device=device)


def config2(M, seed=1002, K=2048, device="cpu"):
    """Decode: E=128, N=1856, K=2048, top-6, M tokens; W bf16 N(0, 0.02^2),
    x bf16 N(0, 1)."""
    d = {"T": M, "k": 6, "E": 128, "N": 1856, "K": K, "w_dtype": "bf16", "w_scale": None, "bias": None}
    d["w"] = bf16_normal((128, 1856, K), 0.02, seed, "w", device)
    d["x"] = bf16_normal((M, K), 1.0, seed, f"x{M}", device)
    d["ids"], d["topk_w"] = softmax_topk_routing(M, 128, 6, seed, f"route{M}", device)
    return d


def nemotron_layer(M, seed=1006, device="cpu", E=128, H=2688, N=1856, k=6, bias=False, weights=True):
    """The Nemotron-shaped non-gated squared-ReLU decode layer: E=128, top-6,
    hidden H=2688, up N=1856 -> relu2 -> down H; W1 bf16 N(0, 0.02^2)
    [E, N, H], W2 bf16 N(0, 0.02^2) [E, H, N], x bf16 N(0, 1) [M, H],
    softmax top-k routing; optional bf16 N(0, 1) biases. weights=False
    leaves out W1 and W2 (the same draws of x and the routing)."""
    d = {"T": M, "k": k, "E": E, "H": H, "N": N}
    d["x"] = bf16_normal((M, H), 1.0, seed, f"x{M}", device)
    d["w1"] = bf16_normal((E, N, H), 0.02, seed, "w1", device) if weights else None
    d["w2"] = bf16_normal((E, H, N), 0.02, seed, "w2", device) if weights else None
    d["b1"] = bf16_normal((E, N), 1.0, seed, "b1", device) if bias else None
    d["b2"] = bf16_normal((E, H), 1.0, seed, "b2", device) if bias else None
    d["ids"], d["topk_w"] = softmax_topk_routing(M, E, k, seed, f"route{M}", device)
    return d


def config3(T_pad, seed=1003, bias=False, device="cpu", E=128, H=2880, I=2880):
    """W4A16 MXFP4 layer, gpt-oss-shaped: E=128, top-4, hidden H=2880,
    gate+up N=2I=5760 -> SwiGLU -> down N=H, K=I. Inputs are drawn for T_pad
    token rows (the bucketed size); a run over T real tokens uses the first T
    rows, and the rows [T, T_pad) are the padding (their activations are set
    to zero by the caller). E2M1 codes uniform; E8M0 bytes uniform in 118..121.
    """
    d = {"T": T_pad, "k": 4, "E": E, "H": H, "I": I}
    d["x"] = bf16_normal((T_pad, H), 1.0, seed, "x", device)
    d["w1"] = e2m1_uniform((E, 2 * I, H // 2), seed, "w1", device)
    d["s1"] = e8m0_uniform((E, 2 * I, H // 32), 118, 121, seed, "s1", device)
    d["w2"] = e2m1_uniform((E, H, I // 2), seed, "w2", device)
    d["s2"] = e8m0_uniform((E, H, I // 32), 118, 121, seed, "s2", device)
    d["b1"] = bf16_normal((E, 2 * I), 1.0, seed, "b1", device) if bias else None
    d["b2"] = bf16_normal((E, H), 1.0, seed, "b2", device) if bias else None
    d["ids"], d["topk_w"] = softmax_topk_routing(T_pad, E, 4, seed, "route", device)
    return d


def config4(seed=1004, bias=False, device="cpu", T=4096, E=256, N=4096, K=7168, n_empty=16):
    """MXFP8 grouped GEMM, DSv4-shaped: E=256, top-8, K=7168, N=4096, T=4096,
    Zipf(1.1) routing over a seeded expert order with the n_empty
    lowest-ranked experts never chosen; x bf16 N(0,1); W E4M3 cast of N(0,1)
    with E8M0 bytes uniform in 123..129; optional bias bf16 N(0,1)."""
    d = {"T": T, "k": 8, "E": E, "N": N, "K": K, "w_dtype": "e4m3"}
    d["x"] = bf16_normal((T, K), 1.0, seed, "x", device)
    d["w"] = e4m3_normal((E, N, K), 1.0, seed, "w", device)
    d["w_scale"] = e8m0_uniform((E, N, K // 32), 123, 129, seed, "ws", device)
    d["bias"] = bf16_normal((E, N), 1.0, seed, "bias", device) if bias else None
    d["ids"], d["topk_w"] = zipf_topk_routing(T, E, 8, 1.1, n_empty, seed, "route", device)
    return d


def config5(seed=1005, device="cpu", T=16384, E=256, N=2048, K=7168, k=8):
    """Weight gradient: E=256, top-8, T=16384, x bf16 N(0,1) [T, 7168],
    grad bf16 N(0,1) [8T, 2048], each token's 8 experts uniform without
    replacement."""
    d = {"T": T, "k": k, "E": E, "N": N, "K": K}
    d["x"] = bf16_normal((T, K), 1.0, seed, "x", device)
    d["grad"] = bf16_normal((T * k, N), 1.0, seed, "grad", device)
    d["ids"], d["topk_w"] = uniform_topk_routing(T, E, k, seed, "route", device)
    return d


def f32_uniform(shape, lo, hi, seed, tag, device="cpu"):
    """float32 uniform in [lo, hi)."""
    g = gen(seed, tag, device)
    return torch.rand(shape, generator=g, device=device, dtype=torch.float32) * (hi - lo) + lo


def zipf_group_sizes(T, E, k, s, n_empty, seed, tag="route", device="cpu"):
    """Per-expert row counts (int32 [E], summing to T * k) of the slots of
    zipf_topk_routing(T, E, k, s, n_empty): the rows of a grouped GEMM over
    T tokens' k distinct experts, grouped by expert."""
    ids, _ = zipf_topk_routing(T, E, k, s, n_empty, seed, tag, device)
    return torch.bincount(ids.reshape(-1).to(torch.int64), minlength=E).to(torch.int32)


def per_token_case(group_sizes, N, K, seed, bias=False, device="cpu"):
    """Inputs of the per-token-scaled FP8 grouped GEMM: A E4M3 codes of
    N(0, 1) [R, K] with R = sum(group_sizes), per-row scales uniform in
    [0.5, 2), W E4M3 codes of N(0, 1) [E, N, K], per-expert scales uniform
    in [0.5, 2), optional bias bf16 N(0, 1) [E, N]."""
    gs = torch.as_tensor(group_sizes, dtype=torch.int32).to(device)
    E, R = gs.numel(), int(gs.sum())
    d = {"E": E, "N": N, "K": K, "R": R, "group_sizes": gs}
    d["a"] = e4m3_normal((R, K), 1.0, seed, "a", device, chunk_dim0=False)
    d["a_scale"] = f32_uniform((R,), 0.5, 2.0, seed, "as", device)
    d["w"] = e4m3_normal((E, N, K), 1.0, seed, "w", device)
    d["w_scale"] = f32_uniform((E,), 0.5, 2.0, seed, "wsc", device)
    d["bias"] = bf16_normal((E, N), 1.0, seed, "bias", device) if bias else None
    return d


def config_per_token(seed=1007, bias=False, device="cpu", T=4096, E=256, N=4096, K=7168, n_empty=16):
    """Per-token FP8 grouped GEMM, DSv4-shaped like the MXFP8 workload: E=256,
    K=7168, N=4096, R = 4096 tokens x top-8 = 32768 rows grouped by expert,
    the group sizes those of Zipf(1.1) top-8 routing (the n_empty
    lowest-ranked experts empty)."""
    return per_token_case(zipf_group_sizes(T, E, 8, 1.1, n_empty, seed, device=device), N, K, seed, bias, device)


def bits(t):
    """A torch tensor -> numpy array of its raw encoding (bf16 -> uint16,
    uint8 stays uint8, int32 stays int32, float32 stays float32)."""
    import numpy as np
    if t is None:
        return None
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def draw_token_counts(n, lo, hi, seed, tag="T"):
    """n token counts uniform in [lo, hi] (the varied serving lengths)."""
    g = gen(seed, tag, "cpu")
    return [int(v) for v in torch.randint(lo, hi + 1, (n,), generator=g)]

