"""GPU parity of the group_sizes interface: the expert block mapping (bit-exact
against the oracle) and the per-token-scaled FP8 grouped GEMM (E4M3 operands,
one fp32 scale per activation row and one per expert, applied after the fp8
dot product) against the float64 oracle: ragged N and K tails, bias, empty
groups, a one-row group, both weight layouts, the constant-input roundtrip,
rows no group covers, and the DSv4-shaped workload at full size on sampled
rows."""

import numpy as np
import pytest
import torch

import synth
from helpers import LazyRows, assert_parity, bf16_to_f64, need_gpu
from oracle import gemm as ogemm

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _moe():
    import mixture_experts_grouped_moe_amd as moe
    return moe


def _mapping_on_gpu(gs, rows, bm):
    moe = _moe()
    eids, offs, ends, total = moe.moe_block_mapping(torch.as_tensor(gs, dtype=torch.int32).cuda(), rows, bm)
    torch.cuda.synchronize()
    return [synth.bits(t) for t in (eids, offs, ends)], int(total.item())


MAP_CASES = [
    ("hand", [3, 0, 5, 1], 2),
    ("zeros", [0, 7, 0, 0, 64, 65, 0, 1], 64),
    ("one", [1000], 64),
    ("empty", [0, 0, 0], 64),
    ("bm1", [2, 0, 3], 1),
    ("e1024", "rand1024", 16),
    ("zipf", "zipf", 64),
]


@pytest.mark.parametrize("case", MAP_CASES, ids=lambda c: c[0])
def test_block_mapping_matches_oracle(case):
    moe = _moe()
    _, gs, bm = case
    if gs == "rand1024":
        gs = synth.bits(torch.randint(0, 40, (1024,), generator=synth.gen(5, "gs"), dtype=torch.int32)).tolist()
    elif gs == "zipf":
        gs = synth.bits(synth.zipf_group_sizes(4096, 256, 8, 1.1, 16, 1007)).tolist()
    rows = int(sum(gs))
    (eids, offs, ends), total = _mapping_on_gpu(gs, rows, bm)
    mb = moe.moe_align_max_blocks(rows, len(gs), bm)
    assert eids.shape == (mb,)
    r_e, r_o, r_n = ogemm.build_block_mapping(gs, bm, mb)
    np.testing.assert_array_equal(eids, r_e)
    np.testing.assert_array_equal(offs, r_o)
    np.testing.assert_array_equal(ends, r_n)
    assert total == rows


def test_block_mapping_counts_off_rows():
    # counts summing to fewer rows than the buffers: the oracle's mapping of
    # those counts; counts past the rows or negative: no block names a row at
    # or past `rows`, negative counts count as zero, total reports the sum
    moe = _moe()
    gs = [5, 0, 9]
    (eids, offs, ends), total = _mapping_on_gpu(gs, 20, 4)
    r = ogemm.build_block_mapping(gs, 4, moe.moe_align_max_blocks(20, 3, 4))
    for got, ref in zip((eids, offs, ends), r):
        np.testing.assert_array_equal(got, ref)
    assert total == 14
    (eids, offs, ends), total = _mapping_on_gpu([6, -3, 9], 10, 4)
    assert total == 15
    used = eids >= 0
    assert (offs[used] < 10).all() and (ends <= 10).all() and (offs <= ends).all()
    assert eids[used].tolist() == [0, 0, 2]
    assert offs[used].tolist() == [0, 4, 6] and ends[used].tolist() == [6, 6, 10]


def _run(d, packed=False, out=None):
    moe = _moe()
    w = moe.moe_pack_weights(d["w"], "e4m3") if packed else d["w"]
    mapping = moe.moe_block_mapping(d["group_sizes"], d["R"])
    return moe.moe_grouped_gemm_per_token(d["a"], d["a_scale"], w, d["w_scale"], mapping, bias=d["bias"], out=out)


def _oracle(d):
    h = {k: synth.bits(v) if isinstance(v, torch.Tensor) else v for k, v in d.items()}
    return ogemm.grouped_gemm_per_token(h["a"], h["a_scale"], h["w"], h["w_scale"], h["group_sizes"],
                                        bias=h["bias"])


GEMM_CASES = [
    # group sizes, N, K, bias, packed weights
    ([70, 0, 5, 130, 1], 200, 96, True, False),
    ([64, 64, 64], 512, 256, False, True),
    ([1], 640, 80, False, False),
    ([0, 0, 300, 0], 1056, 352, True, True),
    ("rand16", 300, 512, False, False),
    ([129, 63, 0, 2], 1030, 1040, True, False),
]


@pytest.mark.parametrize("case", GEMM_CASES, ids=lambda c: "g{}-N{}-K{}-b{}-p{}".format(
    c[0] if isinstance(c[0], str) else len(c[0]), *c[1:]))
def test_per_token_gemm_matches_oracle(case):
    gs, N, K, bias, packed = case
    if gs == "rand16":
        gs = synth.bits(torch.randint(0, 130, (16,), generator=synth.gen(6, "gs"), dtype=torch.int32)).tolist()
    seed = N + K + len(gs)
    d = synth.per_token_case(gs, N, K, seed, bias=bias, device="cuda")
    out = torch.full((d["R"], N), float("nan"), dtype=torch.bfloat16, device="cuda")
    _run(d, packed, out)
    torch.cuda.synchronize()
    assert_parity(bf16_to_f64(out), _oracle(d), what=f"per-token {case}")


def test_packed_equals_rows_layout_bitwise():
    d = synth.per_token_case([100, 0, 37, 250], 700, 320, 11, bias=True, device="cuda")
    a = _run(d, packed=False)
    b = _run(d, packed=True)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_constant_input_roundtrip():
    # A = W = 1.0 (E4M3 0x38), power-of-two scales: every output is
    # K * a_scale[r] * w_scale[e] + bias[e] (exact in fp32) rounded once to bf16
    moe = _moe()
    gs, N, K = [3, 0, 2], 96, 128
    a = torch.full((5, K), 0x38, dtype=torch.uint8, device="cuda")
    w = torch.full((3, N, K), 0x38, dtype=torch.uint8, device="cuda")
    a_s = torch.tensor([1.0, 0.5, 2.0, 0.25, 4.0], device="cuda")
    w_s = torch.tensor([0.5, 8.0, 2.0], device="cuda")
    bias = torch.tensor([[1.0] * N, [0.0] * N, [-2.0] * N], dtype=torch.bfloat16, device="cuda")
    mapping = moe.moe_block_mapping(torch.tensor(gs, dtype=torch.int32, device="cuda"), 5)
    out = moe.moe_grouped_gemm_per_token(a, a_s, w, w_s, mapping, bias=bias)
    torch.cuda.synchronize()
    owner = [0, 0, 0, 2, 2]
    expect = torch.tensor([K * a_s[r].item() * w_s[owner[r]].item() + bias[owner[r], 0].item() for r in range(5)])
    assert expect.tolist() == [65.0, 33.0, 129.0, 62.0, 1022.0]
    assert torch.equal(out.cpu(), expect[:, None].expand(5, N).to(torch.bfloat16))


def test_empty_and_uncovered_rows():
    moe = _moe()
    # no rows at all: nothing to do, no error
    d0 = synth.per_token_case([0, 0], 64, 64, 3, device="cuda")
    out0 = _run(d0)
    assert out0.shape == (0, 64)
    # counts covering 40 of 50 rows: rows 40..49 are not written
    d = synth.per_token_case([25, 0, 15], 128, 64, 4, device="cuda")
    a = torch.cat([d["a"], d["a"][:10]])
    a_s = torch.cat([d["a_scale"], d["a_scale"][:10]])
    out = torch.full((50, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    mapping = moe.moe_block_mapping(d["group_sizes"], 50)
    moe.moe_grouped_gemm_per_token(a, a_s, d["w"], d["w_scale"], mapping, out=out)
    torch.cuda.synchronize()
    assert int(mapping[3].item()) == 40
    assert torch.isnan(out[40:].float()).all()
    assert_parity(bf16_to_f64(out[:40]), _oracle(d), what="covered rows")


def test_per_token_workload_full_size_sampled():
    # The DSv4-shaped per-token workload (E=256, K=7168, N=4096, 32768 rows
    # grouped by Zipf top-8 counts) in the launch configuration the benchmark
    # times (packed weights), checked on sampled rows of the hottest, the
    # highest-numbered non-empty and two more experts.
    moe = _moe()
    d = synth.config_per_token(device="cuda")
    w = moe.moe_pack_weights(d["w"], "e4m3")
    mapping = moe.moe_block_mapping(d["group_sizes"], d["R"])
    C = torch.full((d["R"], d["N"]), float("nan"), dtype=torch.bfloat16, device="cuda")
    moe.moe_grouped_gemm_per_token(d["a"], d["a_scale"], w, d["w_scale"], mapping, out=C)
    torch.cuda.synchronize()
    gs = synth.bits(d["group_sizes"]).astype(np.int64)
    offs = np.concatenate([[0], np.cumsum(gs)])
    live = np.nonzero(gs)[0]
    experts = sorted({int(np.argmax(gs)), int(live.max()), int(live[len(live) // 3]),
                      int(live[2 * len(live) // 3])})
    rows, sub_gs = [], np.zeros_like(gs)
    for e in experts:
        pick = sorted({int(offs[e]), int(offs[e] + gs[e] // 2), int(offs[e + 1] - 1)})
        rows += pick
        sub_gs[e] = len(pick)
    rows_t = torch.tensor(rows, device="cuda")
    ref = ogemm.grouped_gemm_per_token(synth.bits(d["a"][rows_t]), synth.bits(d["a_scale"][rows_t]),
                                       LazyRows(d["w"]), synth.bits(d["w_scale"]), sub_gs)
    assert_parity(bf16_to_f64(C[rows_t]), ref, what="per-token workload, sampled rows")
    assert not torch.isnan(C.float()).any()
