"""The fused decode layer (moe_decode_layer: routing, the decode grouped GEMM
and the top-k combine in one launch) on the GPU. Its y and its expert outputs
C equal, bit for bit, those of moe_align -> moe_grouped_gemm -> moe_combine
on the same inputs, and both match the float64 oracle: every weight encoding,
with and without bias and the relu2 epilogue, K short of a pass and across
two passes, N not a multiple of 8, skewed and repeated routing, ids outside
[0, E), single-token calls (up to 8 slots, routed in registers), NaN scale
bytes, and the launch's limits (256 slots, 1024 experts,
K = 4096). Where the activations of all tokens exceed 76288 elements they
are staged in two passes over the halves of K and each output is summed per
pass; those cases are checked against the oracle, and against the three
launches within the parity bar."""

import numpy as np
import pytest
import torch

import synth
from helpers import assert_parity, bf16_to_f64, combine_scale, host, need_gpu, to_dev
from oracle import gemm as ogemm

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _moe():
    import mixture_experts_grouped_moe_amd as moe
    return moe


def _nan(rows, cols):
    return torch.full((rows, cols), float("nan"), dtype=torch.bfloat16, device="cuda")


def _unfused(dd, T, k, E, N, wd, epilogue):
    moe = _moe()
    routing = moe.moe_align(dd["ids"], E, moe.moe_gemm_block_m(wd, T))
    C = _nan(T * k, N)
    moe.moe_grouped_gemm(dd["x"], dd["w"], wd, routing, T, k, E, k, w_scale=dd["w_scale"], bias=dd["bias"],
                         epilogue=epilogue, out=C)
    y = moe.moe_combine(C, dd["topk_w"], k)
    return C, y


def _fused(dd, T, k, N, wd, epilogue):
    moe = _moe()
    C = _nan(T * k, N)
    y = moe.moe_decode_layer(dd["x"], dd["ids"], dd["topk_w"], dd["w"], wd, w_scale=dd["w_scale"],
                             bias=dd["bias"], epilogue=epilogue, c_out=C)
    return C, y


def _oracle(d, T, k, E, wd, epilogue):
    h = host(d)
    C, routed = ogemm.grouped_gemm(h["x"], k, h["w"], wd, h["w_scale"], h["ids"], E, bias=h["bias"],
                                   epilogue=epilogue)
    return C, routed, ogemm.combine(C, h["topk_w"], k), combine_scale(C, h["topk_w"], k)


def _same_bits(a, b, what):
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)), what


CASES = [
    # T, k, E, N, K, w_dtype, bias, epilogue
    (5, 6, 16, 200, 352, "bf16", True, "relu2"),      # K short of one 2048 pass
    (24, 6, 32, 264, 2688, "bf16", True, "relu2"),    # the Nemotron hidden size: two 2048-element passes
    (28, 6, 32, 264, 2688, "e4m3", True, "none"),     # M x K = 75264, near the on-chip maximum (76288)
    (32, 8, 64, 256, 2048, "bf16", False, "none"),    # 256 slots
    (16, 4, 32, 256, 4096, "e4m3", True, "none"),     # K = 4096 and M x K = 65536
    (28, 4, 16, 256, 2080, "e4m3", False, "relu2"),
    (7, 2, 8, 640, 320, "e2m1x2", True, "none"),
    (12, 4, 1024, 64, 256, "e2m1x2", False, "none"),  # 1024 experts
    (3, 1, 4, 128, 64, "bf16", False, "none"),        # top-1, K = 64
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "T{}k{}E{}N{}K{}{}{}{}".format(
    *c[:6], "b" if c[6] else "", c[7]))
def test_decode_layer_equals_three_launches_and_oracle(case):
    T, k, E, N, K, wd, bias, ep = case
    d = synth.gemm_case(T, k, E, N, K, wd, seed=T * 7 + N + K, bias=bias, w_std=0.5)
    dd = to_dev(d)
    C3, y3 = _unfused(dd, T, k, E, N, wd, ep)
    C1, y1 = _fused(dd, T, k, N, wd, ep)
    torch.cuda.synchronize()
    _same_bits(C1, C3, f"C {case}")
    _same_bits(y1, y3, f"y {case}")
    rC, routed, ry, ys = _oracle(d, T, k, E, wd, ep)
    assert routed.all()
    assert_parity(bf16_to_f64(C1), rC, what=f"C {case}")
    assert_parity(bf16_to_f64(y1), ry, scale=ys, what=f"y {case}")


@pytest.mark.parametrize("M", [1, 7, 14, 21, 28, 32])
def test_decode_shape_equals_three_launches(M):
    # the decode workload: E=128, N=1856, K=2048, top-6, bf16 weights; the
    # oracle checks 64 sampled output columns
    d = synth.config2(M, device="cuda")
    T, k, E, N = M, 6, 128, 1856
    C3, y3 = _unfused(d, T, k, E, N, "bf16", "none")
    C1, y1 = _fused(d, T, k, N, "bf16", "none")
    torch.cuda.synchronize()
    _same_bits(C1, C3, f"C M={M}")
    _same_bits(y1, y3, f"y M={M}")
    cols = np.sort(np.random.default_rng(M).choice(N, 64, replace=False))
    sub = dict(d, w=d["w"][:, torch.from_numpy(cols).cuda(), :].contiguous())
    rC, _, ry, ys = _oracle(sub, T, k, E, "bf16", "none")
    assert_parity(bf16_to_f64(C1)[:, cols], rC, what=f"C M={M}")
    assert_parity(bf16_to_f64(y1)[:, cols], ry, scale=ys, what=f"y M={M}")


def test_nemotron_up_projection_equals_three_launches():
    # hidden 2688 (two K passes) at M = 24, the largest token count whose
    # activations fit on chip at that K, with bias and relu2
    d = synth.nemotron_layer(24, device="cuda", bias=True)
    dd = {"x": d["x"], "ids": d["ids"], "topk_w": d["topk_w"], "w": d["w1"], "w_scale": None, "bias": d["b1"]}
    C3, y3 = _unfused(dd, 24, 6, 128, 1856, "bf16", "relu2")
    C1, y1 = _fused(dd, 24, 6, 1856, "bf16", "relu2")
    torch.cuda.synchronize()
    _same_bits(C1, C3, "C")
    _same_bits(y1, y3, "y")


def test_ragged_n_against_oracle():
    # N = 203: the last workgroup owns three live columns (moe_combine needs
    # N % 8 == 0, so the oracle alone is the reference here)
    T, k, E, N, K = 9, 3, 12, 203, 512
    d = synth.gemm_case(T, k, E, N, K, "e4m3", seed=31, bias=True, w_std=0.5)
    dd = to_dev(d)
    C1, y1 = _fused(dd, T, k, N, "e4m3", "relu2")
    torch.cuda.synchronize()
    rC, _, ry, ys = _oracle(d, T, k, E, "e4m3", "relu2")
    assert_parity(bf16_to_f64(C1), rC, what="C")
    assert_parity(bf16_to_f64(y1), ry, scale=ys, what="y")


@pytest.mark.parametrize("kind", ["zipf", "repeated"])
def test_skewed_and_repeated_routing(kind):
    # zipf: a few experts take most slots (long slot lists per expert);
    # repeated: a token names one expert several times
    T, k, E, N, K = 32, 6, 64, 256, 1024
    d = synth.gemm_case(T, k, E, N, K, "bf16", seed=41, w_std=0.5)
    if kind == "zipf":
        d["ids"], d["topk_w"] = synth.zipf_topk_routing(T, E, k, 1.5, 8, 41)
    else:
        g = torch.Generator().manual_seed(41)
        d["ids"] = torch.randint(0, 4, (T, k), generator=g, dtype=torch.int32)
    dd = to_dev(d)
    C3, y3 = _unfused(dd, T, k, E, N, "bf16", "none")
    C1, y1 = _fused(dd, T, k, N, "bf16", "none")
    torch.cuda.synchronize()
    _same_bits(C1, C3, "C")
    _same_bits(y1, y3, "y")
    rC, _, ry, ys = _oracle(d, T, k, E, "bf16", "none")
    assert_parity(bf16_to_f64(y1), ry, scale=ys, what="y")


def test_ids_outside_the_experts_contribute_zero():
    T, k, E, N, K = 6, 4, 16, 128, 256
    d = synth.gemm_case(T, k, E, N, K, "bf16", seed=51, bias=True, w_std=0.5)
    ids = d["ids"].clone()
    ids[0, 1], ids[3, 0], ids[5, 3] = -1, E, 1 << 30
    d["ids"] = ids
    dd = to_dev(d)
    C1, y1 = _fused(dd, T, k, N, "bf16", "none")
    torch.cuda.synchronize()
    rC, routed, ry, ys = _oracle(d, T, k, E, "bf16", "none")
    assert routed.sum() == T * k - 3
    got = bf16_to_f64(C1)
    assert np.isnan(got[~routed]).all()          # rows of unrouted slots are not written
    assert_parity(got[routed], rC[routed], what="C")
    assert_parity(bf16_to_f64(y1), ry, scale=ys, what="y")


SMALL_ROUTES = [
    # T, k, K, ids (one row per token), w_dtype, bias, epilogue; E = 8. Up
    # to 8 slots every wave routes in registers; 9 and more go through LDS.
    (1, 8, 2688, [[5, 1, 7, 0, 3, 2, 6, 4]], "bf16", True, "relu2"),    # 8 slots, all experts
    (1, 6, 1024, [[3, 3, 3, 3, 3, 3]], "e4m3", False, "none"),           # one expert named six times
    (2, 4, 2688, [[2, 0, 2, 1], [1, 2, 0, 0]], "e2m1x2", True, "none"),  # shared and repeated across tokens
    (1, 6, 2048, [[4, -1, 9, 1 << 30, 0, 9]], "bf16", True, "none"),     # ids outside [0, E) among repeats
    (1, 4, 4096, [[-1, 8, 8, -5]], "bf16", False, "none"),               # no slot routed
    (1, 1, 96, [[7]], "e4m3", True, "relu2"),                            # top-1, K short of a lane's piece
    (2, 4, 512, [[6, 6, 1, 0], [6, 1, 0, 1]], "e2m1x2", False, "none"),
    (3, 3, 2688, [[1, 0, 1], [7, 7, 7], [0, 2, 4]], "bf16", False, "relu2"),  # 9 slots: routed in LDS
]


@pytest.mark.parametrize("case", SMALL_ROUTES, ids=lambda c: "T{}k{}K{}{}".format(c[0], c[1], c[2], c[4]))
def test_few_slots_routed_in_registers(case):
    T, k, K, ids, wd, bias, ep = case
    E, N = 8, 256
    d = synth.gemm_case(T, k, E, N, K, wd, seed=T * 13 + k, bias=bias, w_std=0.5)
    d["ids"] = torch.tensor(ids, dtype=torch.int32)
    dd = to_dev(d)
    C1, y1 = _fused(dd, T, k, N, wd, ep)
    torch.cuda.synchronize()
    rC, routed, ry, ys = _oracle(d, T, k, E, wd, ep)
    got = bf16_to_f64(C1)
    assert np.isnan(got[~routed]).all()          # rows of unrouted slots are not written
    assert_parity(got[routed], rC[routed], what=f"C {case}")
    assert_parity(bf16_to_f64(y1), ry, scale=ys, what=f"y {case}")
    if routed.all():
        C3, y3 = _unfused(dd, T, k, E, N, wd, ep)
        torch.cuda.synchronize()
        _same_bits(C1, C3, f"C {case}")
        _same_bits(y1, y3, f"y {case}")
    if not routed.any():
        assert (bf16_to_f64(y1) == 0).all()


def test_repeated_calls_identical_and_empty():
    # the slots of an expert are grouped with LDS atomics, in any order; each
    # output is computed on its own, so every call gives the same bits
    moe = _moe()
    d = to_dev(synth.gemm_case(20, 6, 32, 256, 2048, "e2m1x2", seed=61, bias=True))
    ys = [moe.moe_decode_layer(d["x"], d["ids"], d["topk_w"], d["w"], "e2m1x2", w_scale=d["w_scale"],
                               bias=d["bias"]) for _ in range(4)]
    torch.cuda.synchronize()
    for y in ys[1:]:
        _same_bits(y, ys[0], "repeat")
    y0 = moe.moe_decode_layer(d["x"][:0], d["ids"][:0], d["topk_w"][:0], d["w"], "e2m1x2", w_scale=d["w_scale"])
    torch.cuda.synchronize()
    assert tuple(y0.shape) == (0, 256)


def test_outside_the_limits_is_refused():
    moe = _moe()
    assert not moe.moe_decode_layer_fits(4, 6, 8, 4128)
    d = to_dev(synth.gemm_case(4, 6, 8, 64, 4128, "bf16", seed=71))
    with pytest.raises(moe.MoeError, match="UNSUPPORTED"):
        moe.moe_decode_layer(d["x"], d["ids"], d["topk_w"], d["w"], "bf16")
    with pytest.raises(moe.MoeError, match="UNSUPPORTED"):
        moe.moe_decode_layer(d["x"][:4], d["ids"][:4], d["topk_w"][:4], d["w"], "bf16", epilogue="swiglu")


@pytest.mark.parametrize("wd", ["e4m3", "e2m1x2"])
def test_nan_scale_bytes_propagate_like_the_oracle(wd):
    # an E8M0 byte of 0xFF decodes to NaN: the C entries of the slots routed
    # to that expert in that column turn NaN, and so do the y entries of
    # their tokens; everything else stays finite (NaN positions must match)
    T, k, E, N, K = 8, 4, 12, 96, 256
    d = synth.gemm_case(T, k, E, N, K, wd, seed=81, w_std=0.5)
    e = int(d["ids"][0, 0])
    ws = d["w_scale"].clone()
    ws[e, 5, 3] = 0xFF       # expert e, weight row 5, K block 3
    ws[e, 40, :] = 0xFF      # expert e, weight row 40, every block
    d["w_scale"] = ws
    dd = to_dev(d)
    C1, y1 = _fused(dd, T, k, N, wd, "none")
    torch.cuda.synchronize()
    rC, _, ry, ys = _oracle(d, T, k, E, wd, "none")
    got_c, got_y = bf16_to_f64(C1), bf16_to_f64(y1)
    assert np.isnan(got_c[:, 5]).any() and np.isnan(got_y[0, 40])
    assert_parity(got_c, rC, what="C")
    assert_parity(got_y, ry, scale=ys, what="y")


SPLIT_CASES = [
    # T, k, E, N, K, w_dtype, bias, epilogue: M x K > 76288, two passes over the halves of K
    (29, 6, 32, 264, 2688, "bf16", True, "relu2"),     # the Nemotron hidden size past 28 tokens
    (32, 8, 64, 256, 4096, "e4m3", True, "none"),      # the largest: 256 slots, K = 4096
    (32, 6, 16, 200, 2688, "e2m1x2", False, "none"),   # halves of 1344
    (32, 2, 8, 72, 2400, "bf16", False, "relu2"),      # unequal halves: 1216 + 1184
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=lambda c: "T{}k{}E{}N{}K{}{}{}{}".format(
    *c[:6], "b" if c[6] else "", c[7]))
def test_two_pass_layer_against_oracle_and_three_launches(case):
    T, k, E, N, K, wd, bias, ep = case
    moe = _moe()
    assert moe.moe_decode_layer_fits(T, k, E, K) and T * K > 76288
    d = synth.gemm_case(T, k, E, N, K, wd, seed=T * 11 + N + K, bias=bias, w_std=0.5)
    dd = to_dev(d)
    C3, y3 = _unfused(dd, T, k, E, N, wd, ep)
    C1, y1 = _fused(dd, T, k, N, wd, ep)
    torch.cuda.synchronize()
    rC, routed, ry, ys = _oracle(d, T, k, E, wd, ep)
    assert routed.all()
    assert_parity(bf16_to_f64(C1), rC, what=f"C {case}")
    assert_parity(bf16_to_f64(y1), ry, scale=ys, what=f"y {case}")
    # the three launches sum each output over all of K at once: equal within
    # the bar (the per-pass grouping may move a last bit)
    assert_parity(bf16_to_f64(C1), bf16_to_f64(C3), what=f"C vs three launches {case}")
    assert_parity(bf16_to_f64(y1), bf16_to_f64(y3), what=f"y vs three launches {case}")


@pytest.mark.parametrize("M", [28, 32])
def test_nemotron_up_projection_at_28_and_32_tokens(M):
    # the page's recipe shape (hidden 2688, N 1856, E 128, top-6): 28 tokens
    # are the most whose activations fit on chip at once (the bits of the
    # three launches), 32 take two passes (within the bar); the oracle
    # checks 64 sampled columns
    d = synth.nemotron_layer(M, device="cuda", bias=True)
    dd = {"x": d["x"], "ids": d["ids"], "topk_w": d["topk_w"], "w": d["w1"], "w_scale": None, "bias": d["b1"]}
    C3, y3 = _unfused(dd, M, 6, 128, 1856, "bf16", "relu2")
    C1, y1 = _fused(dd, M, 6, 1856, "bf16", "relu2")
    torch.cuda.synchronize()
    if M == 28:
        _same_bits(C1, C3, "C")
        _same_bits(y1, y3, "y")
    else:
        assert_parity(bf16_to_f64(y1), bf16_to_f64(y3), what="y vs three launches")
    cols = np.sort(np.random.default_rng(28).choice(1856, 64, replace=False))
    sub = dict(dd, w=d["w1"][:, torch.from_numpy(cols).cuda(), :].contiguous(),
               bias=d["b1"][:, torch.from_numpy(cols).cuda()].contiguous())
    rC, _, ry, ys = _oracle(sub, M, 6, 128, "bf16", "relu2")
    assert_parity(bf16_to_f64(C1)[:, cols], rC, what="C")
