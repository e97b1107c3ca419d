"""GPU parity of moe_grouped_gemm (large-M and decode variants) and
moe_combine against the float64 oracle.

Small cases span several tiles and ragged tails in M, N and K; every weight
encoding, bias and SwiGLU combination is covered. The parity bar is
max|gpu - oracle| <= 5e-3 * max|oracle| per output tensor."""

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


def run_gemm(d, a_row_div=None, epilogue="none", poison=True):
    """Run align + grouped GEMM on the device tensors of d; return C (device)."""
    moe = _moe()
    T, k, E = d["T"], d["k"], d["E"]
    a_row_div = k if a_row_div is None else a_row_div
    bm = moe.moe_gemm_block_m(d["w_dtype"], T)
    routing = moe.moe_align(d["ids"], E, bm)
    n_out = d["N"] // 2 if epilogue == "swiglu" else d["N"]
    out = torch.full((T * k, n_out), float("nan") if poison else 0.0, dtype=torch.bfloat16, device="cuda")
    moe.moe_grouped_gemm(d["x"], d["w"], d["w_dtype"], routing, T, k, E, a_row_div,
                         w_scale=d["w_scale"], bias=d["bias"], epilogue=epilogue, out=out)
    torch.cuda.synchronize()
    return out


def oracle_gemm(h, a_row_div=None, epilogue="none", slots=None):
    k = h["k"]
    a_row_div = k if a_row_div is None else a_row_div
    C, routed = ogemm.grouped_gemm(h["x"], a_row_div, h["w"], h["w_dtype"], h["w_scale"], h["ids"], h["E"],
                                   bias=h["bias"], epilogue=epilogue, slots=slots)
    return C, routed


CASES = [
    # T, k, E, N, K, w_dtype  (spans tiles, ragged N and K tails, decode and large M)
    (200, 2, 4, 640, 320, "e2m1x2"),
    (300, 4, 16, 1056, 256, "e2m1x2"),
    (200, 2, 4, 640, 352, "e4m3"),
    (150, 3, 5, 300, 288, "e4m3"),
    (200, 2, 4, 640, 320, "bf16"),
    (97, 2, 3, 200, 96, "bf16"),
    (1, 2, 8, 640, 320, "e2m1x2"),
    (7, 6, 16, 200, 352, "e4m3"),
    (32, 4, 16, 1056, 2080, "bf16"),
    (33, 4, 16, 1056, 2080, "bf16"),
]


@pytest.mark.parametrize("bias", [False, True])
@pytest.mark.parametrize("epilogue", ["none", "swiglu"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "T{}k{}E{}N{}K{}{}".format(*c))
def test_gemm_parity_small(case, epilogue, bias):
    T, k, E, N, K, wd = case
    d = synth.gemm_case(T, k, E, N, K, wd, seed=T + N + K, bias=bias, w_std=0.5)
    h = host(d)
    C = run_gemm(to_dev(d), epilogue=epilogue)
    ref, routed = oracle_gemm(h, epilogue=epilogue)
    assert routed.all()
    assert_parity(bf16_to_f64(C), ref, what=f"{case} {epilogue} bias={bias}")


@pytest.mark.parametrize("wd", ["e2m1x2", "e4m3", "bf16"])
def test_gemm_over_slot_rows(wd):
    # second-GEMM form: A indexed by slot (a_row_div = 1)
    T, k, E, N, K = 120, 4, 8, 256, 192
    d = synth.gemm_case(T, k, E, N, K, wd, seed=5, bias=True, a_rows=T * k, w_std=0.5)
    C = run_gemm(to_dev(d), a_row_div=1)
    ref, _ = oracle_gemm(host(d), a_row_div=1)
    assert_parity(bf16_to_f64(C), ref)


def test_config1_and_combine():
    moe = _moe()
    d = synth.config1()
    h = host(d)
    dd = to_dev(d)
    C = run_gemm(dd)
    ref, _ = oracle_gemm(h)
    assert_parity(bf16_to_f64(C), ref, what="config1 C")
    y = moe.moe_combine(C, dd["topk_w"], 2)
    torch.cuda.synchronize()
    assert_parity(bf16_to_f64(y), ogemm.combine(ref, h["topk_w"], 2), scale=combine_scale(ref, h["topk_w"], 2),
                  what="config1 y")


@pytest.mark.parametrize("M", [1, 7, 14, 21, 28])
def test_config2_decode(M):
    d = synth.config2(M, device="cuda")
    C = run_gemm(d)
    ref, _ = oracle_gemm(host(d))
    assert_parity(bf16_to_f64(C), ref, what=f"decode M={M}")


def test_decode_and_large_variants_agree_on_threshold():
    moe = _moe()
    assert moe.moe_gemm_block_m("bf16", 32) != moe.moe_gemm_block_m("bf16", 33)
    assert moe.moe_bucket_round_up(32) == 32


def test_unrouted_slots_left_untouched():
    T, k, E, N, K = 40, 2, 4, 128, 64
    d = synth.gemm_case(T, k, E, N, K, "e4m3", seed=9)
    ids = d["ids"].clone()
    ids[3, 1] = E      # out of range: not routed
    ids[10, 0] = -1
    d["ids"] = ids
    C = run_gemm(to_dev(d))
    Cn = bf16_to_f64(C)
    assert np.isnan(Cn[3 * k + 1]).all() and np.isnan(Cn[10 * k]).all()
    ref, routed = oracle_gemm(host(d))
    assert_parity(Cn[routed], ref[routed])


def test_e8m0_edge_codes():
    # E8M0 0x00 = 2^-127, 0x01 = 2^-126, 0xFE = 2^127, 0xFF = NaN. Each group of
    # weight rows uses one edge code on one 32-wide K block (weight code 1.0
    # there, 0 elsewhere) against activations sized so results stay finite,
    # and each group is checked on its own scale.
    T, k, E, N, K = 64, 1, 1, 128, 128
    d = synth.gemm_case(T, k, E, N, K, "e4m3", seed=11)
    x = torch.zeros((T, K), dtype=torch.bfloat16)
    x[:, 0:32], x[:, 32:64], x[:, 64:96] = 2.0 ** 100, 1.0, 2.0 ** -100
    w = torch.zeros((E, N, K), dtype=torch.uint8)
    sc = torch.full((E, N, K // 32), 127, dtype=torch.uint8)
    groups = {"0x00": (slice(0, 32), 0, 0x00), "0x01": (slice(32, 64), 0, 0x01),
              "0xFE": (slice(64, 96), 2, 0xFE), "0xFF": (slice(96, 128), 3, 0xFF)}
    for rows, blk, code in groups.values():
        w[:, rows, blk * 32:(blk + 1) * 32] = 0x38  # 1.0
        sc[:, rows, blk] = code
    d.update(w=w, w_scale=sc, x=x)
    got = bf16_to_f64(run_gemm(to_dev(d)))
    ref, _ = oracle_gemm(host(d))
    assert np.isnan(got[:, 96:]).all() and np.isnan(ref[:, 96:]).all()
    for name, (rows, _, _) in list(groups.items())[:3]:
        assert_parity(got[:, rows], ref[:, rows], what=f"E8M0 {name}")


def test_bias_noncontiguous_strides():
    T, k, E, N, K = 100, 2, 4, 256, 128
    d = synth.gemm_case(T, k, E, N, K, "e2m1x2", seed=12)
    big = synth.bf16_normal((N, 2 * E), 1.0, 12, "bigbias")  # [N, 2E]
    view = big.t()[0::2]                                      # [E, N], strides (2, 2E)
    assert view.shape == (E, N) and not view.is_contiguous()
    d["bias"] = view
    dd = to_dev(d)
    dd["bias"] = big.cuda().t()[0::2]
    assert dd["bias"].stride() == (2, 2 * E)
    C = run_gemm(dd)
    h = host(d)
    h["bias"] = synth.bits(view.contiguous())
    ref, _ = oracle_gemm(h)
    assert_parity(bf16_to_f64(C), ref, what="strided bias")


@pytest.mark.parametrize("wd", ["e2m1x2", "e4m3", "bf16"])
def test_deterministic(wd):
    d = to_dev(synth.gemm_case(300, 4, 16, 512, 256, wd, seed=13, bias=True))
    a = run_gemm(d, epilogue="swiglu")
    b = run_gemm(d, epilogue="swiglu")
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_empty_token_guard():
    moe = _moe()
    d = to_dev(synth.gemm_case(0, 2, 4, 128, 64, "e4m3", seed=14))
    routing = moe.moe_align(d["ids"], 4, moe.moe_gemm_block_m("e4m3", 0))
    out = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    moe.moe_grouped_gemm(d["x"], d["w"], "e4m3", routing, 0, 2, 4, 2, w_scale=d["w_scale"], out=out)
    y = moe.moe_combine(out, d["topk_w"], 2)
    torch.cuda.synchronize()
    assert y.shape == (0, 128)


class _Cols:
    """Rows `cols` of each expert's [N, ...] weights (or scales), fetched from
    the device per expert: the oracle applied to a subset of weight rows
    gives exactly those output columns, as every output column depends on its
    own weight row only."""

    def __init__(self, t, cols):
        self.t, self.cols = t, torch.as_tensor(np.asarray(cols, dtype=np.int64), device=t.device)
        self.shape = (t.shape[0], len(cols)) + tuple(t.shape[2:])

    def __getitem__(self, e):
        return synth.bits(self.t[int(e)].index_select(0, self.cols))


@pytest.mark.parametrize("bias", [False, True])
def test_config4_mxfp8_full_size_sampled(bias):
    # The MXFP8 workload at its full size (E=256, top-8, K=7168, N=4096,
    # T=4096, Zipf routing with 16 empty experts) in the launch configuration
    # the benchmark times (packed weights): one slot of every routed expert
    # (its first, middle or last slot in turn; expert 255's weights start past
    # 2^31 elements), plus the first / middle / last slot of the hottest
    # expert, each on 96 output columns spread over every N tile (both edges
    # of each 512-row tile among them).
    moe = _moe()
    d = synth.config4(device="cuda", bias=bias)
    T, k, E, N = 4096, 8, 256, 4096
    pw = moe.moe_pack_weights(d["w"], "e4m3", w_scale=d["w_scale"])
    bm = moe.moe_gemm_block_m("e4m3", T)
    routing = moe.moe_align(d["ids"], E, bm)
    C = torch.full((T * k, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    moe.moe_grouped_gemm(d["x"], pw, "e4m3", routing, T, k, E, k, bias=d["bias"], out=C)
    torch.cuda.synchronize()
    ids = synth.bits(d["ids"]).reshape(-1)
    counts = np.bincount(ids, minlength=E)
    routed = np.nonzero(counts)[0]
    assert routed.size == E - 16 and routed.max() == 255
    slots = []
    for i, e in enumerate(routed):
        es = np.nonzero(ids == e)[0]
        slots.append(int(es[(0, len(es) // 2, -1)[i % 3]]))
    hot = np.nonzero(ids == int(np.argmax(counts)))[0]
    slots = sorted(set(slots + [int(hot[0]), int(hot[len(hot) // 2]), int(hot[-1])]))
    rng = np.random.default_rng(7)
    cols = sorted(set([0, N - 1] + [t * 512 + o for t in range(N // 512) for o in (0, 511)] +
                      rng.choice(N, 60, replace=False).tolist()))
    bias_cols = None if d["bias"] is None else synth.bits(d["bias"])[:, cols]
    ref, routed_mask = ogemm.grouped_gemm(synth.bits(d["x"]), k, _Cols(d["w"], cols), "e4m3",
                                          _Cols(d["w_scale"], cols), ids, E, bias=bias_cols, slots=slots)
    assert routed_mask[slots].all()
    got = bf16_to_f64(C[slots][:, cols])
    assert_parity(got, ref[slots], what=f"config4 one slot per routed expert (bias={bias})")


def test_bf16_packed_swiglu_large_sampled():
    # bf16 weights at a gate+up shape (N = 5760 -> 2880 SwiGLU columns,
    # K = 2880) in the packed layout, many routing blocks per expert: the
    # two-stage bf16 kernel checked on first / middle / last slots of three
    # experts
    moe = _moe()
    from helpers import LazyRows
    T, k, E, N, K = 2048, 4, 32, 5760, 2880
    d = synth.gemm_case(T, k, E, N, K, "bf16", seed=31, bias=True, w_std=0.02, device="cuda")
    pw = moe.moe_pack_weights(d["w"], "bf16")
    routing = moe.moe_align(d["ids"], E, moe.moe_gemm_block_m("bf16", T))
    C = torch.full((T * k, N // 2), float("nan"), dtype=torch.bfloat16, device="cuda")
    moe.moe_grouped_gemm(d["x"], pw, "bf16", routing, T, k, E, k, bias=d["bias"], epilogue="swiglu", out=C)
    torch.cuda.synchronize()
    ids = synth.bits(d["ids"]).reshape(-1)
    counts = np.bincount(ids, minlength=E)
    slots = []
    for e in (int(np.argmax(counts)), int(np.argmin(np.where(counts > 0, counts, 1 << 30))), E - 1):
        es = np.nonzero(ids == e)[0]
        if es.size:
            slots += [int(es[0]), int(es[len(es) // 2]), int(es[-1])]
    slots = sorted(set(slots))
    ref, routed_mask = ogemm.grouped_gemm(synth.bits(d["x"]), k, LazyRows(d["w"]), "bf16", None, ids, E,
                                          bias=synth.bits(d["bias"]), epilogue="swiglu", slots=slots)
    assert routed_mask[slots].all()
    assert_parity(bf16_to_f64(C[slots]), ref[slots], what="bf16 packed SwiGLU sampled slots")
