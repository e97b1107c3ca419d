"""moe_align + moe_grouped_gemm on random valid shapes (fixed seeds): every
weight encoding, both weight layouts, the three epilogues, bias on and off,
GEMMs over token rows and over slot rows, decode and large-M token counts,
checked in full against the float64 oracle (max|gpu - oracle| <= 5e-3 *
max|oracle|; for a top-k combine, 5e-3 * the size of its weighted terms plus
its own); likewise the MXFP8-activation and per-token GEMMs, the weight
gradient and the fused decode layer (its C and y)."""

import numpy as np
import pytest
import torch

import synth
from helpers import assert_parity, bf16_to_f64, combine_scale, host, need_gpu
from oracle import gemm as ogemm

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _case(seed):
    rng = np.random.default_rng(1000 + seed)
    wd = ("e2m1x2", "e4m3", "bf16")[seed % 3]
    T = int(rng.integers(1, 33)) if seed % 2 else int(rng.integers(33, 400))
    E = int(rng.integers(1, 24))
    k = int(rng.integers(1, min(E, 8) + 1))
    K = 32 * int(rng.integers(1, 40))
    epilogue = ("none", "swiglu", "relu2")[int(rng.integers(0, 3))]
    N = int(rng.integers(1, 700))
    if epilogue == "swiglu":
        N = 2 * max(1, N // 2)
    return dict(wd=wd, T=T, E=E, k=k, K=K, N=N, epilogue=epilogue, bias=bool(rng.integers(0, 2)),
                packed=bool(rng.integers(0, 2)), over_slots=bool(rng.integers(0, 2)))


@pytest.mark.parametrize("seed", range(36))
def test_grouped_gemm_random_shapes(seed):
    import mixture_experts_grouped_moe_amd as moe
    c = _case(seed)
    print("case", seed, c, flush=True)
    T, k, E, N, K, wd = c["T"], c["k"], c["E"], c["N"], c["K"], c["wd"]
    a_rows, a_row_div = (T * k, 1) if c["over_slots"] else (T, k)
    w_std = {"bf16": 0.05, "e4m3": 0.5, "e2m1x2": 1.0}[wd]
    d = synth.gemm_case(T, k, E, N, K, wd, seed=seed, bias=c["bias"], a_rows=a_rows, w_std=w_std, device="cuda")
    w = moe.moe_pack_weights(d["w"], wd, w_scale=d["w_scale"]) if c["packed"] else d["w"]
    routing = moe.moe_align(d["ids"], E, moe.moe_gemm_block_m(wd, T))
    n_out = N // 2 if c["epilogue"] == "swiglu" else N
    out = torch.full((T * k, n_out), float("nan"), dtype=torch.bfloat16, device="cuda")
    moe.moe_grouped_gemm(d["x"], w, wd, routing, T, k, E, a_row_div, w_scale=None if c["packed"] else d["w_scale"],
                         bias=d["bias"], epilogue=c["epilogue"], out=out)
    torch.cuda.synchronize()
    h = host(d)
    ref, routed = ogemm.grouped_gemm(h["x"], a_row_div, h["w"], wd, h["w_scale"], h["ids"], E,
                                     bias=h["bias"], epilogue=c["epilogue"])
    assert routed.all()
    assert_parity(bf16_to_f64(out), ref, what=f"case {seed}")


@pytest.mark.parametrize("seed", range(24))
def test_mxfp8_activation_gemm_random_shapes(seed):
    # E4M3 activation codes with E8M0 scales (the scaled fp8 MFMA kernel):
    # the same random shapes, activations drawn directly as codes and scales
    import mixture_experts_grouped_moe_amd as moe
    c = _case(3 * seed + 1)
    print("case", seed, c, flush=True)
    T, k, E, N, K = c["T"], c["k"], c["E"], c["N"], c["K"]
    a_rows, a_row_div = (T * k, 1) if c["over_slots"] else (T, k)
    d = synth.gemm_case(T, k, E, N, K, "e4m3", seed=seed, bias=c["bias"], a_rows=a_rows, w_std=0.5, device="cuda")
    a_codes = synth.e4m3_normal((a_rows, K), 1.0, seed, "xq")
    a_scales = synth.e8m0_uniform((a_rows, K // 32), 120, 130, seed, "xs")
    w = moe.moe_pack_weights(d["w"], "e4m3", w_scale=d["w_scale"]) if c["packed"] else d["w"]
    routing = moe.moe_align(d["ids"], E, moe.moe_gemm_block_m("e4m3", T, moe.MOE_E4M3))
    n_out = N // 2 if c["epilogue"] == "swiglu" else N
    out = torch.full((T * k, n_out), float("nan"), dtype=torch.bfloat16, device="cuda")
    moe.moe_grouped_gemm(a_codes.cuda(), w, "e4m3", routing, T, k, E, a_row_div,
                         w_scale=None if c["packed"] else d["w_scale"], bias=d["bias"], epilogue=c["epilogue"],
                         out=out, a_scale=a_scales.cuda())
    torch.cuda.synchronize()
    h = host(d)
    ref, routed = ogemm.grouped_gemm(synth.bits(a_codes), a_row_div, h["w"], "e4m3", h["w_scale"], h["ids"], E,
                                     bias=h["bias"], epilogue=c["epilogue"], a_dtype="e4m3",
                                     a_scale=synth.bits(a_scales))
    assert routed.all()
    assert_parity(bf16_to_f64(out), ref, what=f"mxfp8 activations, case {seed}")


@pytest.mark.parametrize("seed", range(24))
def test_per_token_gemm_random_groups(seed):
    # the group_sizes interface: random expert counts (about a third of the
    # groups empty), random N, K a multiple of 16, bias and packed weights
    # (K a multiple of 32) at random
    import mixture_experts_grouped_moe_amd as moe
    rng = np.random.default_rng(2000 + seed)
    E = int(rng.integers(1, 40))
    gs = [0 if rng.random() < 0.3 else int(rng.integers(1, 300)) for _ in range(E)]
    N = int(rng.integers(1, 1100))
    K = 16 * int(rng.integers(1, 80))
    bias = bool(rng.integers(0, 2))
    packed = K % 32 == 0 and bool(rng.integers(0, 2))
    print("case", seed, dict(E=E, R=sum(gs), N=N, K=K, bias=bias, packed=packed), flush=True)
    d = synth.per_token_case(gs, N, K, seed, bias=bias, device="cuda")
    w = moe.moe_pack_weights(d["w"], "e4m3") if packed else d["w"]
    mapping = moe.moe_block_mapping(d["group_sizes"], d["R"])
    out = moe.moe_grouped_gemm_per_token(d["a"], d["a_scale"], w, d["w_scale"], mapping, bias=d["bias"])
    torch.cuda.synchronize()
    h = {k: synth.bits(v) if isinstance(v, torch.Tensor) else v for k, v in d.items()}
    ref = ogemm.grouped_gemm_per_token(h["a"], h["a_scale"], h["w"], h["w_scale"], h["group_sizes"], bias=h["bias"])
    assert_parity(bf16_to_f64(out), ref, what=f"per-token case {seed}")


@pytest.mark.parametrize("seed", range(20))
def test_wgrad_random_shapes(seed):
    # dW[e] = sum over e's slots of grad[s]^T x[s // k] on random shapes
    # (N and K multiples of 32, empty experts likely at large E), every
    # expert checked in full
    import mixture_experts_grouped_moe_amd as moe
    from oracle import wgrad as owgrad
    rng = np.random.default_rng(3000 + seed)
    E = int(rng.integers(1, 48))
    k = int(rng.integers(1, min(E, 8) + 1))
    T = int(rng.integers(1, 500))
    N, K = 32 * int(rng.integers(1, 12)), 32 * int(rng.integers(1, 12))
    print("case", seed, dict(T=T, k=k, E=E, N=N, K=K), flush=True)
    d = synth.config5(seed=seed, T=T, E=E, N=N, K=K, k=k, device="cuda")
    routing = moe.moe_align(d["ids"], E, moe.moe_wgrad_block_m())
    dw = torch.full((E, N, K), float("nan"), dtype=torch.float32, device="cuda")
    moe.moe_wgrad(d["x"], d["grad"], routing, T, k, E, out=dw)
    torch.cuda.synchronize()
    h = host(d)
    ref = owgrad.wgrad(h["x"], h["grad"], h["ids"], k, E)
    got = dw.cpu().double().numpy()
    for e in range(E):
        assert_parity(got[e], ref[e], what=f"wgrad case {seed}, expert {e}")


def _layer_case(seed):
    rng = np.random.default_rng(3000 + seed)
    wd = ("e2m1x2", "e4m3", "bf16")[seed % 3]
    K = 32 * int(rng.integers(1, 129))                 # up to 4096
    T = int(rng.integers(0, 33))                       # two passes over K when T x K > 76288
    E = int(rng.integers(1, 300))
    k = int(rng.integers(1, min(E, 8) + 1))
    N = int(rng.integers(1, 700))
    return dict(wd=wd, T=T, E=E, k=k, K=K, N=N, epilogue=("none", "relu2")[int(rng.integers(0, 2))],
                bias=bool(rng.integers(0, 2)), packed=bool(rng.integers(0, 2)))


@pytest.mark.parametrize("seed", range(34))
def test_decode_layer_random_shapes(seed):
    # the fused decode layer (routing, GEMM, combine in one launch) on random
    # shapes within its limits: y and C against the oracle
    import mixture_experts_grouped_moe_amd as moe
    c = _layer_case(seed)
    print("case", seed, c, flush=True)
    T, k, E, N, K, wd = c["T"], c["k"], c["E"], c["N"], c["K"], c["wd"]
    assert moe.moe_decode_layer_fits(T, k, E, K)
    w_std = {"bf16": 0.05, "e4m3": 0.5, "e2m1x2": 1.0}[wd]
    d = synth.gemm_case(T, k, E, N, K, wd, seed=seed, bias=c["bias"], w_std=w_std, device="cuda")
    w = moe.moe_pack_weights(d["w"], wd, w_scale=d["w_scale"]) if c["packed"] else d["w"]
    C = torch.full((T * k, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    y = moe.moe_decode_layer(d["x"], d["ids"], d["topk_w"], w, wd, w_scale=None if c["packed"] else d["w_scale"],
                             bias=d["bias"], epilogue=c["epilogue"], c_out=C)
    torch.cuda.synchronize()
    assert tuple(y.shape) == (T, N)
    if T == 0:
        return
    h = host(d)
    ref, routed = ogemm.grouped_gemm(h["x"], k, h["w"], wd, h["w_scale"], h["ids"], E, bias=h["bias"],
                                     epilogue=c["epilogue"])
    assert routed.all()
    assert_parity(bf16_to_f64(C), ref, what=f"C case {seed}")
    assert_parity(bf16_to_f64(y), ogemm.combine(ref, h["topk_w"], k), scale=combine_scale(ref, h["topk_w"], k),
                  what=f"y case {seed}")
