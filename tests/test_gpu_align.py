"""GPU parity of moe_align: bit-exact against the oracle on the routings of
every workload and on edge cases (no tokens, empty experts, out-of-range ids,
sentinel blocks), and identical bits run to run."""

import numpy as np
import pytest
import torch

import synth
from helpers import need_gpu
from oracle import align as oalign

pytestmark = pytest.mark.gpu


def _run(ids_np, E, B, extra_blocks=0):
    import mixture_experts_grouped_moe_amd as moe
    ids = torch.from_numpy(np.ascontiguousarray(ids_np, dtype=np.int32)).cuda()
    T, k = ids_np.shape
    mb = moe.moe_align_max_blocks(T * k, E, B) + extra_blocks
    out = (torch.full((mb * B,), -7, dtype=torch.int32, device="cuda"),
           torch.full((mb,), -7, dtype=torch.int32, device="cuda"),
           torch.full((1,), -7, dtype=torch.int32, device="cuda"))
    s, e, p = moe.moe_align(ids, E, B, out=out)
    torch.cuda.synchronize()
    return s.cpu().numpy(), e.cpu().numpy(), int(p.item())


def _check(ids_np, E, B, extra_blocks=0):
    s, e, p = _run(ids_np, E, B, extra_blocks)
    rs, re_, rp = oalign.moe_align(ids_np, E, B)
    S = ids_np.size
    if extra_blocks:  # a longer block list: the extra blocks are sentinels / PAD
        rs = np.concatenate([rs, np.full(extra_blocks * B, S)])
        re_ = np.concatenate([re_, np.full(extra_blocks, -1)])
    assert p == rp
    np.testing.assert_array_equal(e, re_)
    np.testing.assert_array_equal(s, rs)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


@pytest.mark.parametrize("B", [8, 16, 32, 64, 128])
def test_config1_routing(B):
    d = synth.config1()
    _check(synth.bits(d["ids"]), 8, B)


@pytest.mark.parametrize("M", [1, 7, 14, 21, 28])
def test_config2_routing(M):
    d = synth.config2(M)
    _check(synth.bits(d["ids"]), 128, 8)


@pytest.mark.parametrize("T", [6554, 8192])
def test_config3_routing(T):
    ids, _ = synth.softmax_topk_routing(T, 128, 4, 1003)
    _check(synth.bits(ids), 128, 64)


def test_config4_routing_zipf_with_empty_experts():
    ids, _ = synth.zipf_topk_routing(4096, 256, 8, 1.1, 16, 1004)
    ids_np = synth.bits(ids)
    assert (np.bincount(ids_np.reshape(-1), minlength=256) == 0).sum() == 16
    _check(ids_np, 256, 64)


def test_config5_routing():
    ids, _ = synth.uniform_topk_routing(16384, 256, 8, 1005)
    _check(synth.bits(ids), 256, 64)


def test_no_tokens():
    _check(np.zeros((0, 4), dtype=np.int32), 16, 64, extra_blocks=3)


def test_out_of_range_ids_are_not_routed():
    rng = np.random.default_rng(0)
    ids = rng.integers(-3, 40, size=(500, 3)).astype(np.int32)
    _check(ids, 32, 16)


@pytest.mark.parametrize("seed", range(6))
def test_random_small(seed):
    rng = np.random.default_rng(seed)
    T = int(rng.integers(1, 3000))
    E = int(rng.integers(1, 300))
    k = int(rng.integers(1, min(E, 8) + 1))
    B = int(rng.choice([1, 4, 8, 16, 64, 256]))
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    _check(ids, E, B, extra_blocks=int(rng.integers(0, 3)))


def test_max_experts_and_single_expert():
    rng = np.random.default_rng(1)
    _check(rng.integers(0, 1024, size=(2000, 2)).astype(np.int32), 1024, 16)
    _check(np.zeros((3000, 1), dtype=np.int32), 1, 64)


def test_deterministic():
    ids, _ = synth.uniform_topk_routing(16384, 256, 8, 7)
    a = _run(synth.bits(ids), 256, 64)
    b = _run(synth.bits(ids), 256, 64)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


@pytest.mark.parametrize("S", [63, 64, 65, 511, 512, 513, 959, 960, 961, 1023, 1024, 1025, 8191])
def test_run_boundaries(S):
    # the slots split into one run per 64 slots, at most 16 runs: slot counts
    # on either side of a run edge, with block sizes on both sides of the
    # per-thread / per-wave padding switch (32), one heavy expert spanning runs
    rng = np.random.default_rng(S)
    for E, B in ((3, 1), (128, 32), (128, 33), (1024, 64)):
        ids = rng.integers(0, E, size=(S, 1)).astype(np.int32)
        ids[S // 3: S // 3 + S // 4, 0] = E - 1
        _check(ids, E, B, extra_blocks=1)


@pytest.mark.parametrize("S", [16383, 16384, 16385, 24577, 65535, 131071, 200003])
def test_workgroup_boundaries(S):
    # above 8192 slots the routing runs on one workgroup per 8192 slots (at
    # most 16), each counting every run and scattering its own 16: slot
    # counts on either side of a workgroup count's edge, the cap, padding
    # below and above 32 rows, ids outside [0, E), and one heavy expert whose
    # slots span several workgroups' runs
    rng = np.random.default_rng(S)
    for E, B in ((5, 8), (256, 64), (1024, 32)):
        ids = rng.integers(-2, E + 2, size=(S, 1)).astype(np.int32)
        ids[S // 5: S // 5 + S // 3, 0] = E - 1
        _check(ids, E, B, extra_blocks=2)
