"""GPU parity of the grouped GEMM with MXFP8 activations (E4M3 codes + E8M0
per 32 along K) and MXFP8 weights, on the scaled fp8 MFMA, against the
float64 oracle: ragged N and K tails (K % 64 == 32), bias, SwiGLU, both
weight layouts, one token, a GEMM over slot rows, the bf16 -> MXFP8 -> GEMM
chain, and the MXFP8 workload at full size on sampled slots. Activation codes
and scales come from seeded generators or from the oracle's own conversion,
never from the GPU."""

import numpy as np
import pytest
import torch

import synth
from helpers import LazyRows, assert_parity, bf16_to_f64, host, need_gpu, to_dev
from oracle import gemm as ogemm
from oracle import quant as oquant

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _moe():
    import mixture_experts_grouped_moe_amd as moe
    return moe


CASES = [
    # T, k, E, N, K, epilogue, bias, packed weights, activation rows per slot (k: token rows, 1: slot rows)
    (64, 2, 8, 512, 256, "none", False, False, "k"),
    (200, 2, 4, 640, 320, "none", True, True, "k"),
    (150, 3, 5, 300, 288, "swiglu", True, False, "k"),
    (97, 2, 3, 200, 96, "none", False, True, "k"),
    (1, 2, 8, 640, 320, "swiglu", False, True, "k"),
    (7, 6, 16, 200, 352, "none", True, False, "k"),
    (100, 4, 8, 256, 192, "none", False, False, "1"),
    # packed weights: the N tile's scale bytes of a step in one 16-byte DMA
    # per lane (SwiGLU with N/2 a multiple of 8, edge tile of 8 h columns),
    # and the per-wave 2-byte scale DMAs where N/2 is not (N/2 = 100)
    (60, 4, 6, 1040, 352, "swiglu", False, True, "k"),
    (150, 3, 5, 200, 288, "swiglu", True, True, "k"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "T{}k{}E{}N{}K{}-{}-b{}-p{}-div{}".format(*c))
def test_f8_gemm_matches_oracle(case):
    _check(case)


@pytest.mark.parametrize("seed", range(12))
def test_packed_scale_pieces_random_shapes(seed):
    # packed weights with N a multiple of 16 (so N/2 is one of 8): the shapes
    # whose weight scale bytes of a step arrive as 16-byte pieces of 8 rows,
    # fetched by one wave; ragged N tiles, K tails, SwiGLU, bias, token and
    # slot rows
    rng = np.random.default_rng(7000 + seed)
    E = int(rng.integers(1, 41))
    k = int(rng.integers(1, min(E, 8) + 1))
    case = (int(rng.integers(1, 261)), k, E, 16 * int(rng.integers(1, 81)), 32 * int(rng.integers(1, 41)),
            ("none", "swiglu")[int(rng.integers(0, 2))], bool(rng.integers(0, 2)), True,
            ("k", "1")[int(rng.integers(0, 2))])
    print("case", seed, case, flush=True)
    _check(case)


def _check(case):
    moe = _moe()
    T, k, E, N, K, epi, bias, packed, div = case
    a_row_div = k if div == "k" else 1
    seed = T * 7 + N + K
    d = synth.gemm_case(T, k, E, N, K, "e4m3", seed=seed, bias=bias, w_std=0.5)
    a_rows = T if a_row_div == k else T * k
    a_codes = synth.e4m3_normal((a_rows, K), 1.0, seed, "xq")
    a_scales = synth.e8m0_uniform((a_rows, K // 32), 120, 130, seed, "xs")
    dd = to_dev(d)
    w = moe.moe_pack_weights(dd["w"], "e4m3", w_scale=dd["w_scale"]) if packed else dd["w"]
    bm = moe.moe_gemm_block_m("e4m3", T, moe.MOE_E4M3)
    routing = moe.moe_align(dd["ids"], E, bm)
    n_out = N // 2 if epi == "swiglu" else N
    out = torch.full((T * k, n_out), float("nan"), dtype=torch.bfloat16, device="cuda")
    moe.moe_grouped_gemm(a_codes.cuda(), w, "e4m3", routing, T, k, E, a_row_div,
                         w_scale=None if packed else dd["w_scale"], bias=dd["bias"], epilogue=epi, out=out,
                         a_scale=a_scales.cuda())
    torch.cuda.synchronize()
    h = host(d)
    ref, routed = ogemm.grouped_gemm(synth.bits(a_codes), a_row_div, h["w"], "e4m3", h["w_scale"], h["ids"], E,
                                     bias=h["bias"], epilogue=epi, a_dtype="e4m3", a_scale=synth.bits(a_scales))
    assert routed.all()
    assert_parity(bf16_to_f64(out), ref, what=f"f8 {case}")


@pytest.mark.parametrize("epi", ["none", "swiglu"])
def test_scale_load_paths_same_bits(epi):
    # the same packed weights with their scale bytes 16-byte aligned (one
    # 16-byte DMA per step for the tile), at a 2-byte offset (a 2-byte DMA
    # per lane from every wave) and at a 1-byte offset (byte DMAs): only the
    # way the bytes reach LDS differs, so C must be the same bits
    moe = _moe()
    T, k, E, N, K = 150, 4, 8, 1040, 352
    d = synth.gemm_case(T, k, E, N, K, "e4m3", seed=91, bias=True, w_std=0.5)
    a_codes = synth.e4m3_normal((T, K), 1.0, 91, "xq").cuda()
    a_scales = synth.e8m0_uniform((T, K // 32), 120, 130, 91, "xs").cuda()
    dd = to_dev(d)
    pw = moe.moe_pack_weights(dd["w"], "e4m3", w_scale=dd["w_scale"])
    routing = moe.moe_align(dd["ids"], E, moe.moe_gemm_block_m("e4m3", T, moe.MOE_E4M3))
    n_out = N // 2 if epi == "swiglu" else N
    outs = []
    for off in (0, 2, 1):
        buf = torch.zeros(pw.scales.numel() + 64, dtype=torch.uint8, device="cuda")
        sc = buf[off:off + pw.scales.numel()].view(pw.scales.shape)
        sc.copy_(pw.scales)
        w = moe.PackedWeights(pw.codes, sc, "e4m3", N, K)
        out = torch.full((T * k, n_out), float("nan"), dtype=torch.bfloat16, device="cuda")
        moe.moe_grouped_gemm(a_codes, w, "e4m3", routing, T, k, E, k, bias=dd["bias"], epilogue=epi, out=out,
                             a_scale=a_scales)
        outs.append(out)
    torch.cuda.synchronize()
    assert not torch.isnan(outs[0]).all()
    for off, o in zip((2, 1), outs[1:]):
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16)), f"scale bytes at offset {off}"


def test_bf16_to_mxfp8_to_gemm_chain():
    # the GPU path quantizes bf16 activations and runs the MXFP8 x MXFP8 GEMM;
    # the oracle converts the same bf16 values itself and multiplies in float64
    moe = _moe()
    T, k, E, N, K = 300, 4, 16, 1056, 352
    d = synth.gemm_case(T, k, E, N, K, "e4m3", seed=77, bias=True, w_std=0.5)
    dd = to_dev(d)
    q, s = moe.moe_quantize_mxfp8(dd["x"])
    routing = moe.moe_align(dd["ids"], E, moe.moe_gemm_block_m("e4m3", T, moe.MOE_E4M3))
    out = moe.moe_grouped_gemm(q, dd["w"], "e4m3", routing, T, k, E, k, w_scale=dd["w_scale"], bias=dd["bias"],
                               a_scale=s)
    torch.cuda.synchronize()
    h = host(d)
    ref_q, ref_s = oquant.mx_quantize_e4m3(bf16_to_f64(d["x"]))
    ref, routed = ogemm.grouped_gemm(ref_q, k, h["w"], "e4m3", h["w_scale"], h["ids"], E, bias=h["bias"],
                                     a_dtype="e4m3", a_scale=ref_s)
    assert routed.all()
    assert_parity(bf16_to_f64(out), ref, what="bf16 -> mxfp8 -> gemm")


def test_mxfp8_workload_full_size_sampled():
    # The MXFP8 workload (E=256, top-8, K=7168, N=4096, T=4096, Zipf routing)
    # with MXFP8 activations, in the launch configuration the benchmark times
    # (packed weights, activations converted on the GPU), checked on sampled
    # slots of the hottest, the highest-numbered routed and two more experts.
    moe = _moe()
    d = synth.config4(device="cuda")
    T, k, E = 4096, 8, 256
    pw = moe.moe_pack_weights(d["w"], "e4m3", w_scale=d["w_scale"])
    q, s = moe.moe_quantize_mxfp8(d["x"])
    routing = moe.moe_align(d["ids"], E, moe.moe_gemm_block_m("e4m3", T, moe.MOE_E4M3))
    C = torch.full((T * k, 4096), float("nan"), dtype=torch.bfloat16, device="cuda")
    moe.moe_grouped_gemm(q, pw, "e4m3", routing, T, k, E, k, out=C, a_scale=s)
    torch.cuda.synchronize()
    ids = synth.bits(d["ids"]).reshape(-1)
    counts = np.bincount(ids, minlength=E)
    routed = np.nonzero(counts)[0]
    experts = {int(np.argmax(counts)), int(routed.max()), int(routed[len(routed) // 3]),
               int(routed[2 * len(routed) // 3])}
    slots = []
    for e in sorted(experts):
        es = np.nonzero(ids == e)[0]
        slots += [int(es[0]), int(es[len(es) // 2]), int(es[-1])]
    slots = sorted(set(slots))
    rows = sorted({sl // k for sl in slots})
    ref_q = np.zeros((T, 7168), dtype=np.uint8)
    ref_s = np.zeros((T, 7168 // 32), dtype=np.uint8)
    ref_q[rows], ref_s[rows] = oquant.mx_quantize_e4m3(bf16_to_f64(d["x"][rows]))
    ref, routed_mask = ogemm.grouped_gemm(ref_q, k, LazyRows(d["w"]), "e4m3", LazyRows(d["w_scale"]), ids, E,
                                          a_dtype="e4m3", a_scale=ref_s, slots=slots)
    assert routed_mask[slots].all()
    assert_parity(bf16_to_f64(C[slots]), ref[slots], what="mxfp8 activations, sampled slots")
