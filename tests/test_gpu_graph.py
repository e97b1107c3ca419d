"""Every step of the path captured once in a HIP graph and replayed (the
benchmark times graph replays): each replay, with eager work and
synchronizations between replays, reproduces the eager run's bits. The
library issues no memset or allocation, so the captured graphs hold kernel
nodes only."""

import pytest
import torch

import synth
from helpers import need_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _moe():
    import mixture_experts_grouped_moe_amd as moe
    return moe


def _scrub(t):
    if t.dtype.is_floating_point:
        t.fill_(float("nan"))
    else:
        t.fill_(-7)


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def _replays_match(step, outputs, replays=3):
    step()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outputs]
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        step()
    torch.cuda.synchronize()
    for i in range(replays):
        for o in outputs:
            _scrub(o)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for j, (o, r) in enumerate(zip(outputs, ref)):
            assert torch.equal(_bits(o), _bits(r)), f"replay {i}: output {j} differs from the eager run"


def _routing(moe, T, k, E, bm):
    mb = moe.moe_align_max_blocks(T * k, E, bm)
    return (torch.empty(mb * bm, dtype=torch.int32, device="cuda"),
            torch.empty(mb, dtype=torch.int32, device="cuda"),
            torch.empty(1, dtype=torch.int32, device="cuda"))


def test_graph_fused_decode_layer():
    # the decode step in one launch (routing in LDS, GEMM, combine), its
    # expert outputs written too; e2m1 weights with bias
    moe = _moe()
    T, k, E, N, K = 9, 6, 32, 512, 1024
    d = synth.gemm_case(T, k, E, N, K, "e2m1x2", seed=23, bias=True, device="cuda")
    C = torch.empty((T * k, N), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")

    def step():
        moe.moe_decode_layer(d["x"], d["ids"], d["topk_w"], d["w"], "e2m1x2", w_scale=d["w_scale"],
                             bias=d["bias"], out=y, c_out=C)
    _replays_match(step, [C, y])


def test_graph_decode_step():
    moe = _moe()
    T, k, E, N, K = 7, 6, 32, 512, 1024
    d = synth.gemm_case(T, k, E, N, K, "bf16", seed=21, w_std=0.02, device="cuda")
    r = _routing(moe, T, k, E, moe.moe_gemm_block_m("bf16", T))
    C = torch.empty((T * k, N), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")

    def step():
        moe.moe_align(d["ids"], E, moe.moe_gemm_block_m("bf16", T), out=r)
        moe.moe_grouped_gemm(d["x"], d["w"], "bf16", r, T, k, E, k, out=C)
        moe.moe_combine(C, d["topk_w"], k, out=y)
    _replays_match(step, [*r, C, y])


def test_graph_w4a16_layer_step():
    moe = _moe()
    T, k, E, H, I = 160, 4, 8, 256, 192
    d = synth.config3(T, seed=22, bias=True, device="cuda", E=E, H=H, I=I)
    bm = moe.moe_gemm_block_m("e2m1x2", T)
    r = _routing(moe, T, k, E, bm)
    h = torch.empty((T * k, I), dtype=torch.bfloat16, device="cuda")
    c2 = torch.empty((T * k, H), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")

    def step():
        moe.moe_align(d["ids"], E, bm, out=r)
        moe.moe_grouped_gemm(d["x"], d["w1"], "e2m1x2", r, T, k, E, k, w_scale=d["s1"], bias=d["b1"],
                             epilogue="swiglu", out=h)
        moe.moe_grouped_gemm(h, d["w2"], "e2m1x2", r, T, k, E, 1, w_scale=d["s2"], bias=d["b2"], out=c2)
        moe.moe_combine(c2, d["topk_w"], k, out=y)
    _replays_match(step, [*r, h, c2, y])


@pytest.mark.parametrize("packed", [False, True])
def test_graph_mxfp8_activation_step(packed):
    # packed weights take the kernel's one-DMA weight-scale path
    moe = _moe()
    T, k, E, N, K = 100, 4, 8, 512, 192
    d = synth.gemm_case(T, k, E, N, K, "e4m3", seed=23, bias=True, w_std=0.5, device="cuda")
    w, ws = (moe.moe_pack_weights(d["w"], "e4m3", w_scale=d["w_scale"]), None) if packed else (d["w"], d["w_scale"])
    bm = moe.moe_gemm_block_m("e4m3", T, moe.MOE_E4M3)
    r = _routing(moe, T, k, E, bm)
    q = torch.empty((T, K), dtype=torch.uint8, device="cuda")
    qs = torch.empty((T, K // 32), dtype=torch.uint8, device="cuda")
    C = torch.empty((T * k, N), dtype=torch.bfloat16, device="cuda")

    def step():
        moe.moe_quantize_mxfp8(d["x"], out=q, out_scales=qs)
        moe.moe_align(d["ids"], E, bm, out=r)
        moe.moe_grouped_gemm(q, w, "e4m3", r, T, k, E, k, w_scale=ws, bias=d["bias"], out=C, a_scale=qs)
    _replays_match(step, [q, qs, *r, C])


def test_graph_per_token_step():
    moe = _moe()
    d = synth.per_token_case([70, 0, 5, 130, 1], 300, 256, 24, bias=True, device="cuda")
    bm = moe.moe_gemm_block_m("e4m3", d["R"], moe.MOE_E4M3)
    mb = moe.moe_align_max_blocks(d["R"], d["E"], bm)
    mapping = tuple(torch.empty(mb, dtype=torch.int32, device="cuda") for _ in range(3)) + \
        (torch.empty(1, dtype=torch.int32, device="cuda"),)
    C = torch.empty((d["R"], d["N"]), dtype=torch.bfloat16, device="cuda")

    def step():
        moe.moe_block_mapping(d["group_sizes"], d["R"], out=mapping)
        moe.moe_grouped_gemm_per_token(d["a"], d["a_scale"], d["w"], d["w_scale"], mapping, bias=d["bias"], out=C)
    _replays_match(step, [*mapping, C])


def test_graph_wgrad_step():
    moe = _moe()
    d = synth.config5(seed=25, T=256, E=16, N=128, K=256, k=4, device="cuda")
    r = _routing(moe, 256, 4, 16, moe.moe_wgrad_block_m())
    dw = torch.empty((16, 128, 256), dtype=torch.float32, device="cuda")

    def step():
        moe.moe_align(d["ids"], 16, moe.moe_wgrad_block_m(), out=r)
        moe.moe_wgrad(d["x"], d["grad"], r, 256, 4, 16, out=dw)
    _replays_match(step, [*r, dw])
