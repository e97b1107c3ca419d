"""GPU edge cases against the float64 oracle:

* E8M0 edge bytes (0x00 = 2^-127, 0x01 = 2^-126, 0xFE = 2^127, 0xFF = NaN;
  ROCm/aiter PR #5310, second review) on the decode kernel and on both
  operands of the scaled fp8 MFMA, where an activation byte of 0x00 or 0x01
  meets a weight byte of 0xFE so that the product of the two scales is 2^0 or
  2^1: a scale flushed to zero would show as a zero output;
* routing blocks that name an expert id at or past num_experts (weights are
  allocated for one more expert, so memory stays in bounds either way): their
  rows must be left untouched by every GEMM kernel;
* the weight gradient when a workgroup takes a second dW tile after an N / K
  edge tile (more tiles than workgroups, N and K not multiples of 256).
"""

import numpy as np
import pytest
import torch

import synth
from helpers import assert_parity, bf16_to_f64, host, need_gpu, to_dev
from oracle import align as oalign
from oracle import gemm as ogemm
from oracle import wgrad as owgrad

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _moe():
    import mixture_experts_grouped_moe_amd as moe
    return moe


# ---------------------------------------------------------------- E8M0 edges

@pytest.mark.parametrize("w_dtype", ["e4m3", "e2m1x2"])
def test_e8m0_edge_codes_decode(w_dtype):
    # 16 tokens (the decode kernel). Each group of 32 weight rows carries one
    # edge byte on one K block, weight code 1.0 there and 0 elsewhere, against
    # activations sized so the group's outputs are finite (2^100 * 2^-127,
    # 1 * 2^-126, 2^-100 * 2^127) or NaN (0xFF).
    moe = _moe()
    T, k, E, N, K = 16, 1, 1, 128, 128
    d = synth.gemm_case(T, k, E, N, K, w_dtype, seed=41)
    x = torch.zeros((T, K), dtype=torch.bfloat16)
    x[:, 0:32], x[:, 32:64], x[:, 64:96] = 2.0 ** 100, 1.0, 2.0 ** -100
    one = 0x38 if w_dtype == "e4m3" else 0x22  # 1.0 (two E2M1 codes of 1.0 per byte)
    kk = K if w_dtype == "e4m3" else K // 2
    per_blk = 32 if w_dtype == "e4m3" else 16
    w = torch.zeros((E, N, kk), dtype=torch.uint8)
    sc = torch.full((E, N, K // 32), 127, dtype=torch.uint8)
    groups = {"0x00": (slice(0, 32), 0, 0x00), "0x01": (slice(32, 64), 1, 0x01),
              "0xFE": (slice(64, 96), 2, 0xFE), "0xFF": (slice(96, 128), 3, 0xFF)}
    for rows, blk, code in groups.values():
        w[:, rows, blk * per_blk:(blk + 1) * per_blk] = one
        sc[:, rows, blk] = code
    d.update(w=w, w_scale=sc, x=x)
    dd = to_dev(d)
    assert moe.moe_gemm_block_m(w_dtype, T) == 8  # the decode variant
    routing = moe.moe_align(dd["ids"], E, moe.moe_gemm_block_m(w_dtype, T))
    out = torch.full((T, N), 7.0, dtype=torch.bfloat16, device="cuda")
    moe.moe_grouped_gemm(dd["x"], dd["w"], w_dtype, routing, T, k, E, k, w_scale=dd["w_scale"], out=out)
    torch.cuda.synchronize()
    got = bf16_to_f64(out)
    h = host(d)
    ref, _ = ogemm.grouped_gemm(h["x"], k, h["w"], w_dtype, h["w_scale"], h["ids"], E)
    assert np.isnan(got[:, 96:]).all() and np.isnan(ref[:, 96:]).all()
    for name, (rows, _, _) in list(groups.items())[:3]:
        assert_parity(got[:, rows], ref[:, rows], what=f"decode E8M0 {name}")
    # each finite group's value is exact: 32 * 2^(100-127), 32 * 2^-126, 32 * 2^(127-100)
    np.testing.assert_array_equal(got[:, 0:32], 32 * 2.0 ** -27)
    np.testing.assert_array_equal(got[:, 32:64], 32 * 2.0 ** -126)
    np.testing.assert_array_equal(got[:, 64:96], 32 * 2.0 ** 27)


def test_e8m0_edge_codes_scaled_fp8_both_operands():
    # MXFP8 activations x MXFP8 weights on the scaled fp8 MFMA, E8M0 bytes fed
    # to the instruction as they are. Token group g has activation code 1.0
    # on K block g only; the weight rows carry code 1.0 on every block:
    #   block 0: activation byte 0x00 (2^-127) x weight byte 0xFE (2^127) -> 32
    #   block 1: activation byte 0x01 (2^-126) x weight byte 0xFE          -> 64
    #   block 2: activation byte 0xFE          x weight byte 0x00 / 0x01   -> 32 / 64
    #   block 3: activation byte 0xFF (NaN)                                -> NaN rows
    # weight rows 96..127 carry 0xFF on block 3 as well (NaN columns). Every
    # other activation byte is 127 with code 0, whose products are 0.
    moe = _moe()
    T, k, E, N, K = 64, 1, 1, 128, 128
    a = torch.zeros((T, K), dtype=torch.uint8)
    sa = torch.full((T, K // 32), 127, dtype=torch.uint8)
    a_byte = [0x00, 0x01, 0xFE, 0xFF]
    for g in range(4):
        a[16 * g:16 * (g + 1), 32 * g:32 * (g + 1)] = 0x38
        sa[16 * g:16 * (g + 1), g] = a_byte[g]
    w = torch.full((E, N, K), 0x38, dtype=torch.uint8)
    sw = torch.full((E, N, K // 32), 127, dtype=torch.uint8)
    sw[:, :, 0] = 0xFE
    sw[:, :, 1] = 0xFE
    sw[:, :64, 2] = 0x00
    sw[:, 64:, 2] = 0x01
    sw[:, 96:, 3] = 0xFF
    ids = torch.zeros((T, k), dtype=torch.int32)
    routing = moe.moe_align(ids.cuda(), E, moe.moe_gemm_block_m("e4m3", T, moe.MOE_E4M3))
    out = torch.full((T, N), 7.0, dtype=torch.bfloat16, device="cuda")
    moe.moe_grouped_gemm(a.cuda(), w.cuda(), "e4m3", routing, T, k, E, k, w_scale=sw.cuda(), out=out,
                         a_scale=sa.cuda())
    torch.cuda.synchronize()
    got = bf16_to_f64(out)
    ref, _ = ogemm.grouped_gemm(synth.bits(a), k, synth.bits(w), "e4m3", synth.bits(sw), synth.bits(ids), E,
                                a_dtype="e4m3", a_scale=synth.bits(sa))
    assert_parity(got, ref, what="scaled fp8 E8M0 edges")
    # the exact values the two scales give (none of them may flush to 0)
    np.testing.assert_array_equal(got[0:16, :96], 32.0)
    np.testing.assert_array_equal(got[16:32, :96], 64.0)
    np.testing.assert_array_equal(got[32:48, :64], 32.0)
    np.testing.assert_array_equal(got[32:48, 64:96], 64.0)
    assert np.isnan(got[48:64]).all() and np.isnan(got[:, 96:]).all()


# ---------------------------------------------------------------- ids past E

def _routing_with_extra_expert_first(moe, ids_host, E, bm, dev="cuda"):
    """moe_align's routing for E + 1 experts (the oracle's, so it is known
    exactly) with the blocks of expert E moved to the front of the block
    list: a GEMM told num_experts = E must skip them wherever they sit."""
    S = ids_host.size
    sorted_ids, eids, post = oalign.moe_align(ids_host, E + 1, bm)
    eids = np.asarray(eids).copy()
    mb = eids.size
    assert mb == moe.moe_align_max_blocks(S, E + 1, bm)
    sorted_ids = np.asarray(sorted_ids).reshape(mb, bm).copy()
    extra = np.nonzero(eids == E)[0]
    assert extra.size > 0
    # every used block lies inside the range the GEMM reads for E experts
    assert post // bm <= moe.moe_align_max_blocks(S, E, bm)
    order = np.concatenate([extra, np.setdiff1d(np.arange(mb), extra)])
    eids, sorted_ids = eids[order], sorted_ids[order].reshape(-1)
    to = lambda v: torch.from_numpy(np.ascontiguousarray(v).astype(np.int32)).to(dev)
    return (to(sorted_ids), to(eids), to(np.array([post]))), extra.size


@pytest.mark.parametrize("variant", ["decode", "large", "scaled_fp8"])
def test_blocks_naming_an_expert_past_E_are_skipped(variant):
    moe = _moe()
    T = 16 if variant == "decode" else 160
    k, E, N, K = 2, 6, 256, 128
    w_dtype = "e4m3"
    d = synth.gemm_case(T, k, E + 1, N, K, w_dtype, seed=43)  # weights for E + 1 experts
    ids = synth.bits(d["ids"]).reshape(-1)
    ids[::5] = E  # every fifth slot goes to expert E
    d["ids"] = torch.from_numpy(ids.reshape(T, k).astype(np.int32))
    a_f8 = variant == "scaled_fp8"
    bm = moe.moe_gemm_block_m(w_dtype, T, moe.MOE_E4M3 if a_f8 else moe.MOE_BF16)
    routing, n_extra = _routing_with_extra_expert_first(moe, ids, E, bm)
    assert n_extra >= 1
    # the GEMM reads only the blocks moe_align can fill for E experts; every
    # block of expert E was moved into that range
    assert routing[1].numel() >= moe.moe_align_max_blocks(T * k, E, bm)
    dd = to_dev(d)
    out = torch.full((T * k, N), 7.0, dtype=torch.bfloat16, device="cuda")
    if a_f8:
        a = synth.e4m3_normal((T, K), 1.0, 43, "xq")
        sa = synth.e8m0_uniform((T, K // 32), 122, 128, 43, "xs")
        moe.moe_grouped_gemm(a.cuda(), dd["w"], w_dtype, routing, T, k, E, k, w_scale=dd["w_scale"], out=out,
                             a_scale=sa.cuda())
        h = host(d)
        ref, routed = ogemm.grouped_gemm(synth.bits(a), k, h["w"], w_dtype, h["w_scale"], ids, E,
                                         a_dtype="e4m3", a_scale=synth.bits(sa))
    else:
        moe.moe_grouped_gemm(dd["x"], dd["w"], w_dtype, routing, T, k, E, k, w_scale=dd["w_scale"], out=out)
        h = host(d)
        ref, routed = ogemm.grouped_gemm(h["x"], k, h["w"], w_dtype, h["w_scale"], ids, E)
    torch.cuda.synchronize()
    got = bf16_to_f64(out)
    assert (ids == E).sum() > 0 and not routed[ids == E].any()
    np.testing.assert_array_equal(got[ids == E], 7.0)  # untouched
    assert_parity(got[routed], ref[routed], what=f"{variant}: routed rows")


# ---------------------------------------------------------------- wgrad tiles

def _run_wgrad(d):
    moe = _moe()
    routing = moe.moe_align(d["ids"], d["E"], moe.moe_wgrad_block_m())
    dw = torch.full((d["E"], d["N"], d["K"]), float("nan"), dtype=torch.float32, device="cuda")
    moe.moe_wgrad(d["x"], d["grad"], routing, d["T"], d["k"], d["E"], out=dw)
    torch.cuda.synchronize()
    return dw


def test_wgrad_second_tile_after_an_edge_tile():
    # N = K = 288: every expert has 2 x 2 tiles, three of them edge tiles; 96
    # experts give 384 tiles, more than the persistent grid's workgroups, so
    # workgroups go on to a second tile right after storing an edge tile.
    # Every expert is checked in full.
    d = synth.config5(seed=45, T=2000, E=96, N=288, K=288, k=4, device="cuda")
    dw = _run_wgrad(d)
    h = host(d)
    ref = owgrad.wgrad(h["x"], h["grad"], h["ids"], 4, 96)
    for e in range(96):
        assert_parity(dw[e].cpu().double().numpy(), ref[e], what=f"expert {e}")
    # a second call gives the same bits
    dw2 = _run_wgrad(d)
    assert torch.equal(dw.view(torch.int32), dw2.view(torch.int32))


def test_wgrad_down_projection_shape_sampled():
    # a gpt-oss-shaped down-projection gradient: E = 128, N = K = 2880
    # (12 x 12 tiles per expert, edge tiles in both directions, 18432 tiles),
    # top-4 over 4096 tokens; eight experts checked in full, 0 and 127 among them
    d = synth.config5(seed=46, T=4096, E=128, N=2880, K=2880, k=4, device="cuda")
    dw = _run_wgrad(d)
    h = host(d)
    for e in (0, 1, 37, 64, 90, 111, 126, 127):
        ref = owgrad.wgrad_expert(h["x"], h["grad"], h["ids"], 4, e)
        assert_parity(dw[e].cpu().double().numpy(), ref, what=f"expert {e}")
