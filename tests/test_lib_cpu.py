"""CPU tests of the C-ABI library: it loads, exports every symbol the header
declares, its host helpers agree with the oracle, and every argument check
rejects bad calls before anything reaches a GPU (all calls here are invalid
on purpose, so none of them launches a kernel)."""

import ctypes
import os
import re

import numpy as np
import pytest

from oracle import align as oalign
from oracle import bucket as obucket

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

moe = pytest.importorskip("mixture_experts_grouped_moe_amd")
L = moe.lib

OK, INVALID, UNSUPPORTED = 0, 1, 2
FAKE = ctypes.c_void_p(0x100000)  # never dereferenced: every call below is rejected first


@pytest.fixture
def no_device():
    """The rejection tests pass fake pointers; keep them off any machine with a
    GPU, where a check that wrongly let a call through would launch a kernel."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("argument-rejection tests run on hosts without a GPU")


def _declared_symbols():
    text = open(os.path.join(ROOT, "include", "moe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    syms = _declared_symbols()
    assert len(syms) == 20, syms
    for name in syms:
        assert hasattr(L, name), name


def test_bucket_matches_oracle_exhaustively():
    for m in range(0, 65537):
        assert moe.moe_bucket_round_up(m) == obucket.bucket_round_up(m)
    assert moe.moe_bucket_round_up(-5) == -1


@pytest.mark.parametrize("mx", [1, 15, 16, 17, 1000, 20000, 65536])
def test_enumerate_matches_oracle(mx):
    assert moe.moe_bucket_enumerate(mx) == obucket.bucket_enumerate(mx)


def test_enumerate_capacity_query():
    assert L.moe_bucket_enumerate(20000, None, 0) == 98
    assert L.moe_bucket_enumerate(-1, None, 0) == -1
    assert moe.moe_bucket_enumerate(0) == []


def test_max_blocks_matches_oracle():
    rng = np.random.default_rng(0)
    for _ in range(200):
        S, E, B = int(rng.integers(0, 10 ** 6)), int(rng.integers(1, 1025)), int(rng.integers(1, 257))
        assert moe.moe_align_max_blocks(S, E, B) == oalign.max_blocks(S, E, B)
    assert moe.moe_align_max_blocks(-1, 4, 4) == -1


def test_block_m_rule():
    for wd in ("bf16", "e4m3", "e2m1x2"):
        small = {moe.moe_gemm_block_m(wd, t) for t in range(0, 33)}
        large = {moe.moe_gemm_block_m(wd, t) for t in (33, 100, 6554, 8192, 32768)}
        assert len(small) == 1 and len(large) == 1 and small != large
    # the decode threshold is a bucket, so padding never switches variants
    assert moe.moe_decode_max_tokens() == 32 == moe.moe_bucket_round_up(32)
    for t in range(1, 2000):
        assert (t <= 32) == (moe.moe_bucket_round_up(t) <= 32)
    # MXFP8 activations run one kernel (one block size) at every token count, with E4M3 weights only
    f8 = {L.moe_gemm_block_m(moe.MOE_E4M3, moe.MOE_E4M3, t) for t in (0, 1, 32, 33, 4096)}
    assert len(f8) == 1 and f8.pop() in (64, 128)
    assert L.moe_gemm_block_m(moe.MOE_E4M3, moe.MOE_E2M1X2, 100) == -1
    assert L.moe_gemm_block_m(moe.MOE_E4M3, moe.MOE_BF16, 100) == -1
    assert L.moe_gemm_block_m(moe.MOE_BF16, 99, 100) == -1


def test_padding_policy():
    # padding is exact only for bf16 activations x MXFP4 weights without
    # dynamic activation scales; the flag is ignored everywhere else
    codes = [moe.MOE_BF16, moe.MOE_FP32, moe.MOE_E4M3, moe.MOE_E2M1X2, moe.MOE_E8M0]
    for a in codes:
        for w in codes:
            for dyn in (0, 1):
                want = a == moe.MOE_BF16 and w == moe.MOE_E2M1X2 and dyn == 0
                assert moe.moe_padding_supported(a, w, dyn) == want


def test_status_strings():
    assert L.moe_status_string(0) == b"MOE_OK"
    assert L.moe_status_string(1) == b"MOE_ERR_INVALID_ARGUMENT"
    assert L.moe_status_string(99) == b"MOE_ERR_UNKNOWN"


def _align(ids=FAKE, T=10, k=2, E=8, B=16, s=FAKE, e=FAKE, p=FAKE, mb=None):
    if mb is None:
        mb = moe.moe_align_max_blocks(T * k, E, B) if T >= 0 else 0
    return L.moe_align(ids, T, k, E, B, s, e, p, mb, None)


def test_align_rejects(no_device):
    assert _align(T=-1) == INVALID
    assert _align(k=0) == INVALID
    assert _align(k=9, E=8) == INVALID
    assert _align(E=2000, k=2) == UNSUPPORTED
    assert _align(B=0) == INVALID
    assert _align(B=300) == INVALID
    assert _align(mb=1) == INVALID
    assert _align(ids=None) == INVALID
    assert _align(p=None) == INVALID
    assert _align(s=None) == INVALID
    # slot counts within 2^16 of 2^31 are refused before any launch
    assert _align(T=(2 ** 31 - 2 ** 16) // 2 + 1, k=2, E=8, B=1) == INVALID
    assert b"2^16" in L.moe_last_error()


def _gemm_args(**kw):
    g = moe.MoeGemmArgs()
    T, k, E, N, K = kw.pop("T", 100), kw.pop("k", 2), kw.pop("E", 8), kw.pop("N", 256), kw.pop("K", 128)
    wd = kw.pop("w_dtype", moe.MOE_E2M1X2)
    g.num_tokens, g.top_k, g.num_experts, g.n, g.k = T, k, E, N, K
    g.a_dtype, g.a_row_div, g.a, g.a_ld = moe.MOE_BF16, k, 0x100000, K
    wld = K // 2 if wd == moe.MOE_E2M1X2 else K
    g.w_dtype, g.w, g.w_stride_e, g.w_ld = wd, 0x100000, N * wld, wld
    g.w_scale, g.w_scale_stride_e, g.w_scale_ld = 0x100000, N * (K // 32), K // 32
    g.epilogue, g.c, g.c_ld = 0, 0x100000, N
    g.sorted_token_ids = g.expert_ids = g.num_tokens_post_pad = 0x100000
    g.block_m = L.moe_gemm_block_m(moe.MOE_BF16, wd, T)
    g.max_blocks = moe.moe_align_max_blocks(T * k, E, g.block_m)
    for key, v in kw.items():
        setattr(g, key, v)
    return g


def _gemm(**kw):
    return L.moe_grouped_gemm(ctypes.byref(_gemm_args(**kw)), None)


def test_grouped_gemm_rejects_mxfp8_activations(no_device):
    def g8(**kw):
        args = _gemm_args(w_dtype=moe.MOE_E4M3)
        args.a_dtype, args.a_ld, args.a_scale, args.a_scale_ld = moe.MOE_E4M3, args.k, 0x100000, args.k // 32
        args.block_m = L.moe_gemm_block_m(moe.MOE_E4M3, moe.MOE_E4M3, args.num_tokens)
        args.max_blocks = moe.moe_align_max_blocks(args.num_tokens * args.top_k, args.num_experts, args.block_m)
        for key, v in kw.items():
            setattr(args, key, v)
        return L.moe_grouped_gemm(ctypes.byref(args), None)

    assert g8(a_scale=None) == INVALID               # scales required
    assert g8(a_scale_ld=3) == INVALID               # fewer than k / 32
    assert g8(a_ld=136) == INVALID                   # not a multiple of 16 bytes
    assert g8(w_dtype=moe.MOE_E2M1X2, w_ld=64, w_stride_e=256 * 64) == UNSUPPORTED
    assert g8(a_dtype=moe.MOE_FP32) == UNSUPPORTED


def test_grouped_gemm_rejects(no_device):
    assert L.moe_grouped_gemm(None, None) == INVALID
    assert _gemm(K=100) == INVALID                 # K % 32
    assert _gemm(K=0) == INVALID
    assert _gemm(N=255, epilogue=1) == INVALID     # odd N with SwiGLU
    assert _gemm(epilogue=7) == INVALID
    assert _gemm(block_m=32) == INVALID            # not the variant's block_m
    assert _gemm(max_blocks=1) == INVALID
    assert _gemm(a_row_div=3) == INVALID
    assert _gemm(a_ld=64) == INVALID               # < K
    assert _gemm(a_ld=130) == INVALID              # not a multiple of 8
    assert _gemm(w_ld=16) == INVALID
    assert _gemm(w_stride_e=10) == INVALID
    assert _gemm(w_scale=0) == INVALID
    assert _gemm(w_scale_ld=1) == INVALID
    assert _gemm(c_ld=100) == INVALID              # < N
    assert _gemm(c=0x100001) == INVALID            # odd address
    assert _gemm(c=0) == INVALID
    assert _gemm(a=0x100004) == INVALID            # misaligned
    assert _gemm(top_k=9, E=8) == INVALID
    assert _gemm(a_dtype=moe.MOE_E4M3) == UNSUPPORTED
    assert _gemm(w_dtype=moe.MOE_FP32) == UNSUPPORTED
    assert _gemm(num_tokens=-1) == INVALID
    assert _gemm(bias=0x100000, bias_stride_e=-1) == INVALID
    assert _gemm(w_layout=2) == INVALID
    assert _gemm(w_stride_e=256 * 64 + 8) == INVALID   # not a multiple of 16 bytes
    # K-block layout: w_ld is the K-block stride (>= n * 32 bytes for E2M1 pairs)
    assert _gemm(w_layout=moe.MOE_LAYOUT_KBLOCK) == INVALID                 # rows-layout strides
    assert _gemm(w_layout=moe.MOE_LAYOUT_KBLOCK, w_ld=256 * 32, w_stride_e=2 * 256 * 32 - 16,
                 w_scale_ld=512, w_scale_stride_e=1024) == INVALID            # expert stride too small
    assert _gemm(w_layout=moe.MOE_LAYOUT_KBLOCK, w_ld=256 * 32, w_stride_e=2 * 256 * 32,
                 w_scale_ld=500, w_scale_stride_e=1024) == INVALID            # scale block stride < 2n


def test_decode_layer_fits():
    f = moe.moe_decode_layer_fits
    assert f(28, 6, 128, 2048) and f(32, 8, 1024, 2048) and f(0, 6, 128, 2048)
    assert f(24, 6, 128, 2688) and f(28, 6, 128, 2688)       # one pass, two passes of K
    assert f(32, 8, 128, 4096) and not f(1, 6, 128, 4128)    # K <= 4096
    assert not f(33, 1, 128, 256)                            # beyond the decode bucket
    assert not f(32, 9, 128, 256)                            # 288 slots
    assert not f(1, 6, 1025, 256)
    assert not f(1, 6, 128, 100) and not f(-1, 6, 128, 256) and not f(1, 0, 128, 256)


def _dl(ids=FAKE, tw=FAKE, y=FAKE, y_ld=None, **kw):
    for key, v in (("T", 7), ("k", 6), ("E", 128), ("N", 256), ("K", 2048)):
        kw.setdefault(key, v)
    g = _gemm_args(**kw)
    return L.moe_decode_layer(ctypes.byref(g), ids, tw, y, g.n if y_ld is None else y_ld, None)


def test_decode_layer_rejects(no_device):
    assert L.moe_decode_layer(None, FAKE, FAKE, FAKE, 256, None) == INVALID
    assert _dl(T=33) == UNSUPPORTED                  # beyond the decode bucket
    assert _dl(K=4128) == UNSUPPORTED                # K > 4096
    assert _dl(E=1025) == UNSUPPORTED
    assert _dl(T=32, k=9, E=16) == UNSUPPORTED       # 288 slots
    assert _dl(epilogue=1) == UNSUPPORTED            # SwiGLU
    assert _dl(a_dtype=moe.MOE_E4M3) == UNSUPPORTED
    assert _dl(w_dtype=moe.MOE_FP32) == UNSUPPORTED
    assert _dl(epilogue=7) == INVALID
    assert _dl(a_row_div=1) == INVALID               # A must hold token rows
    assert _dl(K=100) == INVALID
    assert _dl(num_tokens=-1) == INVALID
    assert _dl(k=9, E=8) == INVALID                  # top_k > E
    assert _dl(a_ld=2040) == INVALID                 # < K
    assert _dl(y_ld=100) == INVALID                  # < N
    assert _dl(c_ld=100) == INVALID                  # C given with c_ld < N
    assert _dl(w_ld=16) == INVALID
    assert _dl(w_scale=0) == INVALID
    assert _dl(ids=None) == INVALID
    assert _dl(tw=None) == INVALID
    assert _dl(y=None) == INVALID
    assert _dl(y=ctypes.c_void_p(0x100001)) == INVALID   # odd address
    assert _dl(a=0x100004) == INVALID                # misaligned
    assert _dl(bias=0x100000, bias_stride_e=-1) == INVALID


def test_packed_sizes():
    assert moe.moe_packed_sizes("e2m1x2", 256, 128) == (2 * 256 * 32, 2 * 256 * 2)
    assert moe.moe_packed_sizes("e4m3", 10, 96) == (2 * 10 * 64, 2 * 10 * 2)
    assert moe.moe_packed_sizes("bf16", 3, 64) == (3 * 64, 0)
    i64 = ctypes.c_int64
    assert L.moe_packed_sizes(moe.MOE_E4M3, 10, 100, ctypes.byref(i64()), None) == INVALID
    assert L.moe_packed_sizes(moe.MOE_FP32, 10, 64, None, None) == INVALID
    assert L.moe_packed_sizes(moe.MOE_E4M3, 0, 64, None, None) == INVALID


def test_pack_weights_rejects(no_device):
    p = L.moe_pack_weights
    E4 = moe.MOE_E4M3

    def call(wd=E4, E=2, n=16, k=128, w=FAKE, se=16 * 128, ld=128, s=FAKE, sse=16 * 4, sld=4,
             wo=ctypes.c_void_p(0x10000000), so=FAKE):
        return p(wd, E, n, k, w, se, ld, s, sse, sld, wo, so, None)

    assert call(k=100) == INVALID
    assert call(E=-1) == INVALID
    assert call(ld=64) == INVALID              # row shorter than k
    assert call(se=100) == INVALID
    assert call(ld=136) == INVALID             # not a multiple of 16 bytes
    assert call(s=None) == INVALID
    assert call(so=None) == INVALID
    assert call(sld=2) == INVALID
    assert call(w=None) == INVALID
    assert call(wo=FAKE) == INVALID            # output overlaps the input
    assert call(w=ctypes.c_void_p(0x100008)) == INVALID
    assert call(wd=moe.MOE_FP32) == INVALID


def test_block_mapping_rejects(no_device):
    def call(gs=FAKE, E=8, rows=100, bm=64, e=FAKE, o=FAKE, en=FAKE, mb=None, tot=None):
        if mb is None:
            mb = moe.moe_align_max_blocks(rows, E, bm) if rows >= 0 and 1 <= bm <= 256 else 1
        return L.moe_block_mapping(gs, E, rows, bm, e, o, en, mb, tot, None)

    assert call(E=0) == INVALID
    assert call(E=1025) == INVALID
    assert call(rows=-1) == INVALID
    assert call(rows=1 << 31) == INVALID
    assert call(bm=0) == INVALID
    assert call(bm=257) == INVALID
    assert call(mb=2) == INVALID               # fewer than the bound
    assert call(gs=None) == INVALID
    assert call(e=None) == INVALID
    assert call(o=None) == INVALID
    assert call(en=None) == INVALID


def _per_token(**kw):
    g = moe.MoePerTokenArgs()
    R, E, N, K = 300, 8, 256, 128
    g.rows, g.num_experts, g.n, g.k = R, E, N, K
    g.a, g.a_ld, g.a_scale = 0x100000, K, 0x100000
    g.w_layout, g.w, g.w_stride_e, g.w_ld, g.w_scale = moe.MOE_LAYOUT_ROWS, 0x100000, N * K, K, 0x100000
    g.c, g.c_ld = 0x100000, N
    g.block_expert_ids = g.block_token_offsets = g.block_token_ends = 0x100000
    g.block_m = L.moe_gemm_block_m(moe.MOE_E4M3, moe.MOE_E4M3, R)
    g.max_blocks = moe.moe_align_max_blocks(R, E, g.block_m)
    for key, v in kw.items():
        setattr(g, key, v)
    return L.moe_grouped_gemm_per_token(ctypes.byref(g), None)


def test_grouped_gemm_per_token_rejects(no_device):
    assert L.moe_grouped_gemm_per_token(None, None) == INVALID
    assert _per_token(rows=-1) == INVALID
    assert _per_token(num_experts=0) == INVALID
    assert _per_token(k=24, a_ld=32, w_ld=32, w_stride_e=256 * 32) == INVALID   # k % 16
    assert _per_token(a_ld=136) == INVALID             # not a multiple of 16 bytes
    assert _per_token(a_ld=64) == INVALID              # shorter than k
    assert _per_token(w_ld=120) == INVALID
    assert _per_token(w_stride_e=100) == INVALID
    assert _per_token(w_layout=7) == INVALID
    assert _per_token(k=48, a_ld=48, w_ld=48, w_stride_e=256 * 48, w_layout=moe.MOE_LAYOUT_KBLOCK) == INVALID
    assert L.moe_last_error().endswith(b"needs k % 32 == 0")
    assert _per_token(w_layout=moe.MOE_LAYOUT_KBLOCK, w_ld=256 * 64 - 16) == INVALID
    assert _per_token(c_ld=255) == INVALID
    assert _per_token(bias=0x100000, bias_stride_e=-1) == INVALID
    assert _per_token(block_m=32) == INVALID
    assert _per_token(max_blocks=3) == INVALID
    assert _per_token(a_scale=None) == INVALID
    assert _per_token(w_scale=None) == INVALID
    assert _per_token(block_token_ends=None) == INVALID
    assert _per_token(a_scale=0x100002) == INVALID     # not 4-byte aligned
    assert _per_token(a=0x100008) == INVALID           # not 16-byte aligned


def test_quantize_mxfp8_rejects(no_device):
    qz = L.moe_quantize_mxfp8
    Q = ctypes.c_void_p(0x10000000)

    def call(x=FAKE, x_ld=256, rows=10, k=256, q=Q, q_ld=256, s=FAKE, s_ld=8):
        return qz(x, x_ld, rows, k, q, q_ld, s, s_ld, None)

    assert call(rows=-1) == INVALID
    assert call(k=100) == INVALID              # not a multiple of 32
    assert call(k=0) == INVALID
    assert call(x_ld=128) == INVALID           # row shorter than k
    assert call(x_ld=260) == INVALID           # not a multiple of 8 elements
    assert call(q_ld=264) == INVALID           # not a multiple of 16 bytes
    assert call(s_ld=7) == INVALID             # fewer than k / 32 scales
    assert call(x=None) == INVALID
    assert call(s=None) == INVALID
    assert call(q=ctypes.c_void_p(0x10000008)) == INVALID  # not 16-byte aligned


def test_combine_rejects(no_device):
    c = L.moe_combine
    assert c(FAKE, 256, FAKE, -1, 2, 256, FAKE, 256, None) == INVALID
    assert c(FAKE, 256, FAKE, 10, 0, 256, FAKE, 256, None) == INVALID
    assert c(FAKE, 256, FAKE, 10, 2, 100, FAKE, 256, None) == INVALID
    assert c(FAKE, 100, FAKE, 10, 2, 256, FAKE, 256, None) == INVALID
    assert c(None, 256, FAKE, 10, 2, 256, FAKE, 256, None) == INVALID
    assert c(ctypes.c_void_p(0x100002), 256, FAKE, 10, 2, 256, FAKE, 256, None) == INVALID


def test_wgrad_rejects(no_device):
    w = L.moe_wgrad
    mb = moe.moe_align_max_blocks(80, 8, 64)
    args = dict(x=FAKE, xld=256, g=FAKE, gld=128, s=FAKE, e=FAKE, p=FAKE, T=10, k=8, E=8,
                n=128, kk=256, bm=64, mb=mb, dw=FAKE)

    def call(**kw):
        a = dict(args, **kw)
        return w(a["x"], a["xld"], a["g"], a["gld"], a["s"], a["e"], a["p"], a["T"], a["k"], a["E"],
                 a["n"], a["kk"], a["bm"], a["mb"], a["dw"], None)

    assert call(bm=32) == INVALID
    assert call(n=100) == INVALID
    assert call(kk=200) == INVALID
    assert call(k=9) == INVALID
    assert call(mb=0) == INVALID
    assert call(dw=None) == INVALID
    assert call(xld=100) == INVALID
    assert call(T=-1) == INVALID
    # no tokens: the kernel still runs (dW = 0) and reads the routing arrays when they have blocks
    assert call(T=0, x=None, g=None, e=None, mb=4) == INVALID
    assert call(T=0, x=None, g=None, s=None, mb=4) == INVALID


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "moe_copy", os.path.join(ROOT, "mixture_experts_grouped_moe_amd", "__init__.py"))
    mod = importlib.util.module_from_spec(spec)
    src = open(spec.origin).read().replace(
        'LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")',
        f'LIB_PATH = {str(tmp_path / "missing.so")!r}')
    with pytest.raises(ImportError):
        exec(compile(src, spec.origin, "exec"), mod.__dict__)


def test_max_blocks_bounds_the_used_blocks():
    # the grouped GEMM launches moe_align_max_blocks(S, E, B) routing blocks:
    # the oracle's used block count never exceeds it, and it is reached when
    # every touched expert needs one more block than S / B alone would give
    rng = np.random.default_rng(11)
    for _ in range(300):
        E = int(rng.integers(1, 300))
        k = int(rng.integers(1, min(E, 8) + 1))
        T = int(rng.integers(1, 400))
        B = int(rng.choice([1, 2, 8, 16, 64, 128, 256]))
        ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32).reshape(T, k)
        _, _, post_pad = oalign.moe_align(ids, E, B)
        assert post_pad % B == 0
        assert post_pad // B <= moe.moe_align_max_blocks(T * k, E, B)
    # tight case: E experts with one slot each
    E, B = 40, 16
    _, _, post_pad = oalign.moe_align(np.arange(E, dtype=np.int32).reshape(E, 1), E, B)
    assert post_pad // B == moe.moe_align_max_blocks(E, E, B) == E
