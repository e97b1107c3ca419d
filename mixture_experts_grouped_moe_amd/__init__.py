"""Python binding of libmoe, the C-ABI library of gfx950 HIP kernels for the
routed, block-scaled MoE expert layer.

The functions here have the names of the C entry points (include/moe.h) and
only marshal arguments: they check tensor shapes, dtypes and devices, take
raw device pointers and the current HIP stream from torch, and call the
library. Every step of the computation runs in the library's kernels; torch
supplies device memory and streams. Importing this module loads libmoe.so and
fails loudly when it has not been built (there is no fallback).
"""

import ctypes
import os

import torch

__all__ = [
    "MoeError", "lib", "MOE_BF16", "MOE_FP32", "MOE_E4M3", "MOE_E2M1X2", "MOE_E8M0",
    "moe_bucket_round_up", "moe_bucket_enumerate", "moe_padding_supported",
    "moe_align_max_blocks", "moe_gemm_block_m", "moe_wgrad_block_m", "moe_decode_max_tokens",
    "moe_align", "moe_grouped_gemm", "moe_grouped_gemm_prepare", "moe_combine", "moe_wgrad",
    "moe_quantize_mxfp8", "moe_block_mapping", "moe_grouped_gemm_per_token",
    "moe_grouped_gemm_per_token_prepare",
    "moe_pack_weights", "moe_packed_sizes", "PackedWeights", "MOE_LAYOUT_ROWS", "MOE_LAYOUT_KBLOCK",
    "moe_w4a16_layer", "moe_relu2_layer", "moe_decode_layer", "moe_decode_layer_prepare",
    "moe_decode_layer_fits",
    "LIB_PATH",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")

MOE_BF16, MOE_FP32, MOE_E4M3, MOE_E2M1X2, MOE_E8M0, MOE_I32 = 1, 2, 3, 4, 5, 6
MOE_LAYOUT_ROWS, MOE_LAYOUT_KBLOCK = 0, 1
_W_DTYPES = {"bf16": MOE_BF16, "e4m3": MOE_E4M3, "e2m1x2": MOE_E2M1X2}
_EPILOGUES = {"none": 0, "swiglu": 1, "relu2": 2}


class MoeError(RuntimeError):
    """A libmoe call returned an error status."""

    def __init__(self, status, message):
        super().__init__(f"{_status_name(status)}: {message}")
        self.status = status


class MoeGemmArgs(ctypes.Structure):
    """ctypes mirror of moe_gemm_args (include/moe.h)."""
    _fields_ = [
        ("num_tokens", ctypes.c_int64), ("top_k", ctypes.c_int32), ("num_experts", ctypes.c_int32),
        ("n", ctypes.c_int64), ("k", ctypes.c_int64),
        ("a_dtype", ctypes.c_int32), ("a_row_div", ctypes.c_int32),
        ("a", ctypes.c_void_p), ("a_ld", ctypes.c_int64),
        ("a_scale", ctypes.c_void_p), ("a_scale_ld", ctypes.c_int64),
        ("w_dtype", ctypes.c_int32), ("w_layout", ctypes.c_int32), ("w", ctypes.c_void_p),
        ("w_stride_e", ctypes.c_int64), ("w_ld", ctypes.c_int64),
        ("w_scale", ctypes.c_void_p), ("w_scale_stride_e", ctypes.c_int64), ("w_scale_ld", ctypes.c_int64),
        ("bias", ctypes.c_void_p), ("bias_stride_e", ctypes.c_int64), ("bias_stride_n", ctypes.c_int64),
        ("epilogue", ctypes.c_int32), ("c", ctypes.c_void_p), ("c_ld", ctypes.c_int64),
        ("sorted_token_ids", ctypes.c_void_p), ("expert_ids", ctypes.c_void_p),
        ("num_tokens_post_pad", ctypes.c_void_p),
        ("block_m", ctypes.c_int32), ("max_blocks", ctypes.c_int64),
    ]


class MoePerTokenArgs(ctypes.Structure):
    """ctypes mirror of moe_per_token_args (include/moe.h)."""
    _fields_ = [
        ("rows", ctypes.c_int64), ("num_experts", ctypes.c_int32),
        ("n", ctypes.c_int64), ("k", ctypes.c_int64),
        ("a", ctypes.c_void_p), ("a_ld", ctypes.c_int64), ("a_scale", ctypes.c_void_p),
        ("w_layout", ctypes.c_int32), ("w", ctypes.c_void_p),
        ("w_stride_e", ctypes.c_int64), ("w_ld", ctypes.c_int64), ("w_scale", ctypes.c_void_p),
        ("bias", ctypes.c_void_p), ("bias_stride_e", ctypes.c_int64), ("bias_stride_n", ctypes.c_int64),
        ("c", ctypes.c_void_p), ("c_ld", ctypes.c_int64),
        ("block_expert_ids", ctypes.c_void_p), ("block_token_offsets", ctypes.c_void_p),
        ("block_token_ends", ctypes.c_void_p),
        ("block_m", ctypes.c_int32), ("max_blocks", ctypes.c_int64),
    ]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it first with "
            "`python mixture_experts_grouped_moe_amd/_build.py` (or __graft_entry__.build())")
    L = ctypes.CDLL(LIB_PATH)
    i64, i32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
    sig = {
        "moe_bucket_round_up": (i64, [i64]),
        "moe_bucket_enumerate": (i64, [i64, ctypes.POINTER(i64), i64]),
        "moe_padding_supported": (i32, [i32, i32, i32]),
        "moe_align_max_blocks": (i64, [i64, i32, i32]),
        "moe_gemm_block_m": (i32, [i32, i32, i64]),
        "moe_wgrad_block_m": (i32, []),
        "moe_decode_max_tokens": (i64, []),
        "moe_status_string": (ctypes.c_char_p, [i32]),
        "moe_last_error": (ctypes.c_char_p, []),
        "moe_align": (i32, [vp, i64, i32, i32, i32, vp, vp, vp, i64, vp]),
        "moe_grouped_gemm": (i32, [ctypes.POINTER(MoeGemmArgs), vp]),
        "moe_combine": (i32, [vp, i64, vp, i64, i32, i64, vp, i64, vp]),
        "moe_quantize_mxfp8": (i32, [vp, i64, i64, i64, vp, i64, vp, i64, vp]),
        "moe_wgrad": (i32, [vp, i64, vp, i64, vp, vp, vp, i64, i32, i32, i64, i64, i32, i64, vp, vp]),
        "moe_pack_weights": (i32, [i32, i32, i64, i64, vp, i64, i64, vp, i64, i64, vp, vp, vp]),
        "moe_packed_sizes": (i32, [i32, i64, i64, ctypes.POINTER(i64), ctypes.POINTER(i64)]),
        "moe_block_mapping": (i32, [vp, i32, i64, i32, vp, vp, vp, i64, vp, vp]),
        "moe_grouped_gemm_per_token": (i32, [ctypes.POINTER(MoePerTokenArgs), vp]),
        "moe_decode_layer": (i32, [ctypes.POINTER(MoeGemmArgs), vp, vp, vp, i64, vp]),
        "moe_decode_layer_fits": (i32, [i64, i32, i32, i64]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    return L


lib = _load()


def _status_name(status):
    return lib.moe_status_string(int(status)).decode()


def _check(status):
    if status != 0:
        raise MoeError(status, lib.moe_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, name, dtype, dim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dim is not None and t.dim() != dim:
        raise ValueError(f"{name} must have {dim} dimensions, got {t.dim()}")
    if t.numel() and t.dim() and t.stride(-1) != 1:
        raise ValueError(f"{name} must be contiguous in its last dimension")


# ---------------------------------------------------------------- host helpers

def moe_bucket_round_up(m):
    """Token-dimension bucket of m (8 per power-of-two octave, <= 12.5% padding)."""
    return int(lib.moe_bucket_round_up(int(m)))


def moe_bucket_enumerate(max_tokens):
    """Sorted closure of the buckets of 1..max_tokens."""
    n = lib.moe_bucket_enumerate(int(max_tokens), None, 0)
    if n < 0:
        raise ValueError("max_tokens must be >= 0")
    buf = (ctypes.c_int64 * max(n, 1))()
    lib.moe_bucket_enumerate(int(max_tokens), buf, n)
    return [int(buf[i]) for i in range(n)]


def moe_padding_supported(a_dtype, w_dtype, dynamic_act_scale=False):
    return bool(lib.moe_padding_supported(int(a_dtype), int(w_dtype), int(bool(dynamic_act_scale))))


def moe_align_max_blocks(num_slots, num_experts, block_m):
    return int(lib.moe_align_max_blocks(int(num_slots), int(num_experts), int(block_m)))


def moe_gemm_block_m(w_dtype, num_tokens, a_dtype=MOE_BF16):
    w = _W_DTYPES.get(w_dtype, w_dtype)
    return int(lib.moe_gemm_block_m(int(a_dtype), int(w), int(num_tokens)))


def moe_wgrad_block_m():
    return int(lib.moe_wgrad_block_m())


def moe_decode_max_tokens():
    return int(lib.moe_decode_max_tokens())


def moe_packed_sizes(w_dtype, n, k):
    """Per-expert (storage units, scale bytes) of moe_pack_weights' output."""
    wu, sb = ctypes.c_int64(0), ctypes.c_int64(0)
    _check(lib.moe_packed_sizes(int(_W_DTYPES[w_dtype]), int(n), int(k), ctypes.byref(wu), ctypes.byref(sb)))
    return wu.value, sb.value


# ---------------------------------------------------------------- device calls

class PackedWeights:
    """Expert weights in the K-block layout (MOE_LAYOUT_KBLOCK of moe.h).

    codes: [E, ceil(K/64), N, R] (R = 64 elements, or 32 bytes of E2M1 pairs);
    scales: uint8 [E, ceil(K/64), N, 2] or None for bf16. n and k are the
    logical weight shape [E, N, K]. Accepted by moe_grouped_gemm in place of
    a rows-layout weight tensor (then w_scale is not passed).
    """

    def __init__(self, codes, scales, w_dtype, n, k):
        self.codes, self.scales, self.w_dtype, self.n, self.k = codes, scales, w_dtype, int(n), int(k)

    @property
    def num_experts(self):
        return self.codes.shape[0]


def moe_pack_weights(w, w_dtype, w_scale=None, stream=None):
    """Repack rows-layout weights [E, N, K] (and E8M0 scales [E, N, K/32])
    into the K-block layout; returns a PackedWeights. A copy, run once when
    the weights are loaded. E4M3 codes may come without scales (the weights
    of moe_grouped_gemm_per_token)."""
    wd = _W_DTYPES[w_dtype]
    _need(w, "w", torch.bfloat16 if w_dtype == "bf16" else torch.uint8, 3)
    E, N = w.shape[0], w.shape[1]
    K = w.shape[2] * (2 if w_dtype == "e2m1x2" else 1)
    nblk = (K + 63) // 64
    R = 32 if w_dtype == "e2m1x2" else 64
    codes = torch.empty((E, nblk, N, R), dtype=w.dtype, device=w.device)
    scales = None
    if w_dtype != "bf16" and not (w_dtype == "e4m3" and w_scale is None):
        _need(w_scale, "w_scale", torch.uint8, 3)
        if tuple(w_scale.shape) != (E, N, K // 32):
            raise ValueError(f"w_scale must be [E, N, K/32] = {(E, N, K // 32)}")
        scales = torch.empty((E, nblk, N, 2), dtype=torch.uint8, device=w.device)
    _check(lib.moe_pack_weights(wd, E, N, K, _ptr(w), w.stride(0), w.stride(1),
                                _ptr(w_scale), w_scale.stride(0) if scales is not None else 0,
                                w_scale.stride(1) if scales is not None else 0,
                                _ptr(codes), _ptr(scales), _stream(stream)))
    return PackedWeights(codes, scales, w_dtype, N, K)



def moe_align(topk_ids, num_experts, block_m, num_tokens=None, out=None, stream=None):
    """Sort slots by expert and pad each expert to block_m.

    topk_ids: int32 [T, top_k] on the device. Returns (sorted_token_ids,
    expert_ids, num_tokens_post_pad) as int32 device tensors; `out` may give
    preallocated ones. num_tokens (default T) routes only the first rows.
    """
    _need(topk_ids, "topk_ids", torch.int32, 2)
    if not topk_ids.is_contiguous():
        raise ValueError("topk_ids must be contiguous")
    T = topk_ids.shape[0] if num_tokens is None else int(num_tokens)
    if T > topk_ids.shape[0]:
        raise ValueError("num_tokens exceeds topk_ids rows")
    k = topk_ids.shape[1]
    mb = moe_align_max_blocks(T * k, num_experts, block_m)
    if out is None:
        dev = topk_ids.device
        out = (torch.empty(max(mb, 0) * block_m, dtype=torch.int32, device=dev),
               torch.empty(max(mb, 0), dtype=torch.int32, device=dev),
               torch.empty(1, dtype=torch.int32, device=dev))
    sorted_ids, expert_ids, post_pad = out
    max_blocks = expert_ids.numel()
    if sorted_ids.numel() < max_blocks * block_m:
        raise ValueError("sorted_token_ids is shorter than max_blocks * block_m")
    _check(lib.moe_align(_ptr(topk_ids), T, k, int(num_experts), int(block_m),
                         _ptr(sorted_ids), _ptr(expert_ids), _ptr(post_pad), max_blocks,
                         _stream(stream)))
    return sorted_ids, expert_ids, post_pad


def _weight_args(g, w, w_dtype, w_scale, bias, K):
    """Checks the weights, scales and bias of a routed GEMM and fills their
    fields of the MoeGemmArgs g. Returns (E, N, codes, scales)."""
    wd = _W_DTYPES[w_dtype]
    packed = isinstance(w, PackedWeights)
    if packed:
        if w.w_dtype != w_dtype or w.k != K:
            raise ValueError("packed weights do not match w_dtype / a's K")
        if w_scale is not None:
            raise ValueError("packed weights carry their own scales")
        E, N = w.num_experts, w.n
        w_t, w_scale = w.codes, w.scales
        _need(w_t, "w.codes", torch.bfloat16 if w_dtype == "bf16" else torch.uint8, 4)
    else:
        w_t = w
        _need(w_t, "w", torch.bfloat16 if w_dtype == "bf16" else torch.uint8, 3)
        E, N = w_t.shape[0], w_t.shape[1]
        if w_t.shape[2] * (2 if w_dtype == "e2m1x2" else 1) != K:
            raise ValueError("w's K does not match a's")
        if w_dtype != "bf16":
            _need(w_scale, "w_scale", torch.uint8, 3)
            if tuple(w_scale.shape) != (E, N, K // 32):
                raise ValueError(f"w_scale must be [E, N, K/32] = {(E, N, K // 32)}")
    if bias is not None:
        if bias.dtype != torch.bfloat16 or not bias.is_cuda or tuple(bias.shape) != (E, N):
            raise TypeError("bias must be a bf16 [E, N] device tensor")
    g.w_dtype, g.w, g.w_stride_e, g.w_ld = wd, w_t.data_ptr(), w_t.stride(0), w_t.stride(1)
    g.w_layout = MOE_LAYOUT_KBLOCK if packed else MOE_LAYOUT_ROWS
    if w_scale is not None:
        g.w_scale, g.w_scale_stride_e, g.w_scale_ld = w_scale.data_ptr(), w_scale.stride(0), w_scale.stride(1)
    if bias is not None:
        g.bias, g.bias_stride_e, g.bias_stride_n = bias.data_ptr(), bias.stride(0), bias.stride(1)
    return E, N, w_t, w_scale


def moe_grouped_gemm(a, w, w_dtype, routing, num_tokens, top_k, num_experts, a_row_div,
                     w_scale=None, bias=None, epilogue="none", out=None, block_m=None,
                     stream=None, a_scale=None):
    """See moe_grouped_gemm_prepare; this builds the call and runs it once."""
    call, out = moe_grouped_gemm_prepare(a, w, w_dtype, routing, num_tokens, top_k, num_experts, a_row_div,
                                         w_scale=w_scale, bias=bias, epilogue=epilogue, out=out,
                                         block_m=block_m, stream=stream, a_scale=a_scale)
    call()
    return out


def moe_grouped_gemm_prepare(a, w, w_dtype, routing, num_tokens, top_k, num_experts, a_row_div,
                             w_scale=None, bias=None, epilogue="none", out=None, block_m=None,
                             stream=None, a_scale=None):
    """Routed grouped GEMM: C[s] = epilogue(A[s // a_row_div] . W_hat[e]^T + bias[e]).

    a: bf16 [rows, K], or uint8 E4M3 codes [rows, K] with a_scale uint8 E8M0
    [rows, K/32] (MXFP8 activations, e.g. from moe_quantize_mxfp8; E4M3
    weights only); w: [E, N, K] bf16 / uint8 E4M3 codes, or uint8 [E, N, K/2]
    packed E2M1; w_scale: uint8 E8M0 [E, N, K/32]; bias: bf16 [E, N] (any
    strides); routing: the (sorted_token_ids, expert_ids, num_tokens_post_pad)
    of moe_align with block_m = moe_gemm_block_m(w_dtype, num_tokens).
    C is bf16 [num_tokens * top_k, N or N/2]; rows of unrouted slots are left
    as they were. Returns (call, C): call() launches the GEMM on the stream
    captured here, with the arguments checked and marshalled once (for tight
    loops and graph capture).
    """
    a_f8 = isinstance(a, torch.Tensor) and a.dtype == torch.uint8
    if a_f8:
        _need(a, "a", torch.uint8, 2)
        _need(a_scale, "a_scale", torch.uint8, 2)
        if w_dtype != "e4m3":
            raise ValueError("MXFP8 activations need e4m3 weights")
        if a_scale.shape[0] < a.shape[0] or a_scale.shape[1] < a.shape[1] // 32:
            raise ValueError("a_scale must be at least [rows, K/32]")
    else:
        _need(a, "a", torch.bfloat16, 2)
        if a_scale is not None:
            raise ValueError("a_scale is for uint8 (E4M3) activations")
    a_dt = MOE_E4M3 if a_f8 else MOE_BF16
    K = a.shape[1]
    S = int(num_tokens) * int(top_k)
    g = MoeGemmArgs()
    E, N, w_t, w_scale = _weight_args(g, w, w_dtype, w_scale, bias, K)
    if a.shape[0] * int(a_row_div) < S:
        raise ValueError("a has too few rows for num_tokens * top_k slots")
    ep = _EPILOGUES[epilogue]
    out_w = N // 2 if ep == 1 else N
    if out is None:
        out = torch.empty((S, out_w), dtype=torch.bfloat16, device=a.device)
    _need(out, "out", torch.bfloat16, 2)
    if out.shape[0] < S or out.shape[1] < out_w:
        raise ValueError(f"out must be at least [{S}, {out_w}]")
    sorted_ids, expert_ids, post_pad = routing
    bm = moe_gemm_block_m(w_dtype, num_tokens, a_dt) if block_m is None else block_m
    if sorted_ids.numel() < expert_ids.numel() * bm:
        raise ValueError("routing arrays do not match block_m")
    g.num_tokens, g.top_k, g.num_experts = int(num_tokens), int(top_k), int(num_experts)
    g.n, g.k = N, K
    g.a_dtype, g.a_row_div, g.a, g.a_ld = a_dt, int(a_row_div), a.data_ptr(), a.stride(0)
    if a_f8:
        g.a_scale, g.a_scale_ld = a_scale.data_ptr(), a_scale.stride(0)
    g.epilogue, g.c, g.c_ld = ep, out.data_ptr(), out.stride(0)
    g.sorted_token_ids, g.expert_ids = sorted_ids.data_ptr(), expert_ids.data_ptr()
    g.num_tokens_post_pad = post_pad.data_ptr()
    g.block_m, g.max_blocks = int(bm), expert_ids.numel()
    st = _stream(stream)
    ref = ctypes.byref(g)
    keep = (a, w_t, w_scale, bias, out, routing, a_scale)  # the call holds its tensors alive

    def call():
        _check(lib.moe_grouped_gemm(ref, st))
        return keep[4]
    call.args = g
    return call, out


def moe_block_mapping(group_sizes, rows, block_m=None, out=None, stream=None):
    """Expert block mapping of per-expert row counts (the group_sizes
    interface): rows of expert e are [o_e, o_e + g_e), cut into blocks of
    block_m (default: the per-token GEMM's) in expert order.

    group_sizes: int32 [E] on the device (summing to `rows`). Returns
    (block_expert_ids, block_token_offsets, block_token_ends, total_rows) as
    int32 device tensors, -1 / rows / rows past the used blocks; total_rows[0]
    is the sum of the counts, for callers that want to check it. `out` may
    give the four preallocated.
    """
    _need(group_sizes, "group_sizes", torch.int32, 1)
    if not group_sizes.is_contiguous():
        raise ValueError("group_sizes must be contiguous")
    E = group_sizes.shape[0]
    bm = moe_gemm_block_m("e4m3", rows, MOE_E4M3) if block_m is None else int(block_m)
    mb = moe_align_max_blocks(int(rows), E, bm)
    if out is None:
        dev = group_sizes.device
        out = tuple(torch.empty(max(mb, 0), dtype=torch.int32, device=dev) for _ in range(3)) + \
            (torch.empty(1, dtype=torch.int32, device=dev),)
    eids, offs, ends, total = out
    if not (eids.numel() == offs.numel() == ends.numel()):
        raise ValueError("the three mapping arrays must have one length")
    _check(lib.moe_block_mapping(_ptr(group_sizes), E, int(rows), bm, _ptr(eids), _ptr(offs), _ptr(ends),
                                 eids.numel(), _ptr(total), _stream(stream)))
    return eids, offs, ends, total


def moe_grouped_gemm_per_token(a, a_scale, w, w_scale, mapping, bias=None, out=None, stream=None):
    """See moe_grouped_gemm_per_token_prepare; this builds the call and runs it once."""
    call, out = moe_grouped_gemm_per_token_prepare(a, a_scale, w, w_scale, mapping, bias=bias, out=out,
                                                   stream=stream)
    call()
    return out


def moe_grouped_gemm_per_token_prepare(a, a_scale, w, w_scale, mapping, bias=None, out=None, stream=None):
    """Per-token-scaled FP8 grouped GEMM over expert-contiguous rows:
    C[r] = (dec(A[r]) . dec(W[e])^T) * a_scale[r] * w_scale[e] + bias[e].

    a: uint8 E4M3 codes [R, K]; a_scale: float32 [R]; w: uint8 E4M3 codes
    [E, N, K], or a PackedWeights of them (e4m3, no scales); w_scale: float32
    [E]; mapping: moe_block_mapping's result for these R rows; bias: bf16
    [E, N] (any strides). C is bf16 [R, N]. Returns (call, C) like
    moe_grouped_gemm_prepare.
    """
    _need(a, "a", torch.uint8, 2)
    _need(a_scale, "a_scale", torch.float32, 1)
    _need(w_scale, "w_scale", torch.float32, 1)
    R, K = a.shape
    if a_scale.numel() < R or not a_scale.is_contiguous() or not w_scale.is_contiguous():
        raise ValueError("a_scale must be a contiguous [R], w_scale a contiguous [E]")
    packed = isinstance(w, PackedWeights)
    if packed:
        if w.w_dtype != "e4m3" or w.scales is not None or w.k != K:
            raise ValueError("packed weights must be e4m3 codes without scales, with a's K")
        E, N, w_t = w.num_experts, w.n, w.codes
        _need(w_t, "w.codes", torch.uint8, 4)
    else:
        w_t = w
        _need(w_t, "w", torch.uint8, 3)
        E, N = w_t.shape[0], w_t.shape[1]
        if w_t.shape[2] != K:
            raise ValueError("w's K does not match a's")
    if w_scale.numel() < E:
        raise ValueError("w_scale must hold one scale per expert")
    if bias is not None:
        if bias.dtype != torch.bfloat16 or not bias.is_cuda or tuple(bias.shape) != (E, N):
            raise TypeError("bias must be a bf16 [E, N] device tensor")
    if out is None:
        out = torch.empty((R, N), dtype=torch.bfloat16, device=a.device)
    _need(out, "out", torch.bfloat16, 2)
    if out.shape[0] < R or out.shape[1] < N:
        raise ValueError(f"out must be at least [{R}, {N}]")
    eids, offs, ends = mapping[0], mapping[1], mapping[2]
    g = MoePerTokenArgs()
    g.rows, g.num_experts, g.n, g.k = R, E, N, K
    g.a, g.a_ld, g.a_scale = a.data_ptr(), a.stride(0), a_scale.data_ptr()
    g.w_layout = MOE_LAYOUT_KBLOCK if packed else MOE_LAYOUT_ROWS
    g.w, g.w_stride_e, g.w_ld, g.w_scale = w_t.data_ptr(), w_t.stride(0), w_t.stride(1), w_scale.data_ptr()
    if bias is not None:
        g.bias, g.bias_stride_e, g.bias_stride_n = bias.data_ptr(), bias.stride(0), bias.stride(1)
    g.c, g.c_ld = out.data_ptr(), out.stride(0)
    g.block_expert_ids, g.block_token_offsets, g.block_token_ends = eids.data_ptr(), offs.data_ptr(), ends.data_ptr()
    g.block_m, g.max_blocks = moe_gemm_block_m("e4m3", R, MOE_E4M3), eids.numel()
    st = _stream(stream)
    ref = ctypes.byref(g)
    keep = (a, a_scale, w_t, w_scale, bias, out, mapping)

    def call():
        _check(lib.moe_grouped_gemm_per_token(ref, st))
        return keep[5]
    call.args = g
    return call, out


def moe_combine(c, topk_w, top_k, num_tokens=None, out=None, stream=None):
    """y[t] = sum_j topk_w[t, j] * c[t * top_k + j] (fp32, bf16 out), t < num_tokens."""
    _need(c, "c", torch.bfloat16, 2)
    _need(topk_w, "topk_w", torch.float32, 2)
    if not topk_w.is_contiguous():
        raise ValueError("topk_w must be contiguous")
    T = topk_w.shape[0] if num_tokens is None else int(num_tokens)
    N = c.shape[1]
    if c.shape[0] < T * int(top_k) or topk_w.shape[0] < T or topk_w.shape[1] != int(top_k):
        raise ValueError("c / topk_w too small for num_tokens * top_k")
    if out is None:
        out = torch.empty((T, N), dtype=torch.bfloat16, device=c.device)
    _need(out, "out", torch.bfloat16, 2)
    _check(lib.moe_combine(_ptr(c), c.stride(0), _ptr(topk_w), T, int(top_k), N,
                           _ptr(out), out.stride(0), _stream(stream)))
    return out


def moe_decode_layer_fits(num_tokens, top_k, num_experts, k):
    """True when moe_decode_layer takes this many tokens, slots, experts and K."""
    return bool(lib.moe_decode_layer_fits(int(num_tokens), int(top_k), int(num_experts), int(k)))


def moe_decode_layer(x, topk_ids, topk_w, w, w_dtype, w_scale=None, bias=None, epilogue="none", out=None,
                     c_out=None, stream=None):
    """See moe_decode_layer_prepare; this builds the call and runs it once."""
    call, out = moe_decode_layer_prepare(x, topk_ids, topk_w, w, w_dtype, w_scale=w_scale, bias=bias,
                                         epilogue=epilogue, out=out, c_out=c_out, stream=stream)
    call()
    return out


def moe_decode_layer_prepare(x, topk_ids, topk_w, w, w_dtype, w_scale=None, bias=None, epilogue="none",
                             out=None, c_out=None, stream=None):
    """The decode MoE step in one launch: y[t] = sum_j topk_w[t, j] *
    epilogue(x[t] . W_hat[topk_ids[t, j]]^T + bias), with the bits of
    moe_align -> moe_grouped_gemm -> moe_combine.

    x: bf16 [T, K] token rows (T <= 32); topk_ids int32 and topk_w fp32
    [T, top_k] (contiguous); w, w_scale, bias as for moe_grouped_gemm;
    epilogue "none" or "relu2". c_out (bf16 [T * top_k, N]), when given,
    receives the expert outputs C. Returns (call, y) with y bf16 [T, N];
    call() launches the layer on the stream captured here.
    """
    _need(x, "x", torch.bfloat16, 2)
    _need(topk_ids, "topk_ids", torch.int32, 2)
    _need(topk_w, "topk_w", torch.float32, 2)
    if not (topk_ids.is_contiguous() and topk_w.is_contiguous()):
        raise ValueError("topk_ids and topk_w must be contiguous")
    T, K = x.shape
    k = topk_ids.shape[1]
    if topk_ids.shape[0] != T or tuple(topk_w.shape) != (T, k):
        raise ValueError("topk_ids and topk_w must be [T, top_k] for x's T rows")
    g = MoeGemmArgs()
    E, N, w_t, w_scale = _weight_args(g, w, w_dtype, w_scale, bias, K)
    if out is None:
        out = torch.empty((T, N), dtype=torch.bfloat16, device=x.device)
    _need(out, "out", torch.bfloat16, 2)
    if out.shape[0] < T or out.shape[1] < N:
        raise ValueError(f"out must be at least [{T}, {N}]")
    if c_out is not None:
        _need(c_out, "c_out", torch.bfloat16, 2)
        if c_out.shape[0] < T * k or c_out.shape[1] < N:
            raise ValueError(f"c_out must be at least [{T * k}, {N}]")
        g.c, g.c_ld = c_out.data_ptr(), c_out.stride(0)
    g.num_tokens, g.top_k, g.num_experts = T, k, E
    g.n, g.k = N, K
    g.a_dtype, g.a_row_div, g.a, g.a_ld = MOE_BF16, k, x.data_ptr(), x.stride(0)
    g.epilogue = _EPILOGUES[epilogue]
    st = _stream(stream)
    ref = ctypes.byref(g)
    ids_p, tw_p, y_p, y_ld = _ptr(topk_ids), _ptr(topk_w), _ptr(out), out.stride(0)
    keep = (x, topk_ids, topk_w, w_t, w_scale, bias, out, c_out)  # the call holds its tensors alive

    def call():
        _check(lib.moe_decode_layer(ref, ids_p, tw_p, y_p, y_ld, st))
        return keep[6]
    call.args = g
    return call, out


def moe_quantize_mxfp8(x, out=None, out_scales=None, stream=None):
    """bf16 [R, K] -> (E4M3 codes uint8 [R, K], E8M0 scales uint8 [R, K / 32]):
    the OCP MX conversion, one scale per 32 consecutive K elements."""
    _need(x, "x", torch.bfloat16, 2)
    R, K = x.shape
    if out is None:
        out = torch.empty((R, K), dtype=torch.uint8, device=x.device)
    if out_scales is None:
        out_scales = torch.empty((R, K // 32), dtype=torch.uint8, device=x.device)
    _need(out, "out", torch.uint8, 2)
    _need(out_scales, "out_scales", torch.uint8, 2)
    if out.shape[0] < R or out_scales.shape[0] < R:
        raise ValueError("out / out_scales have fewer rows than x")
    _check(lib.moe_quantize_mxfp8(_ptr(x), x.stride(0), R, K, _ptr(out), out.stride(0), _ptr(out_scales),
                                  out_scales.stride(0), _stream(stream)))
    return out, out_scales


def moe_wgrad(x, grad, routing, num_tokens, top_k, num_experts, out=None, stream=None):
    """dW[e] = sum over slots s routed to e of grad[s]^T x[s // top_k], fp32 [E, N, K]."""
    _need(x, "x", torch.bfloat16, 2)
    _need(grad, "grad", torch.bfloat16, 2)
    N, K = grad.shape[1], x.shape[1]
    if out is None:
        out = torch.empty((num_experts, N, K), dtype=torch.float32, device=x.device)
    _need(out, "out", torch.float32, 3)
    if not out.is_contiguous():
        raise ValueError("out must be contiguous")
    if x.shape[0] < int(num_tokens) or grad.shape[0] < int(num_tokens) * int(top_k):
        raise ValueError("x / grad too small for num_tokens * top_k slots")
    if tuple(out.shape) != (int(num_experts), N, K):
        raise ValueError(f"out must be [E, N, K] = {(int(num_experts), N, K)}")
    sorted_ids, expert_ids, post_pad = routing
    _check(lib.moe_wgrad(_ptr(x), x.stride(0), _ptr(grad), grad.stride(0),
                         _ptr(sorted_ids), _ptr(expert_ids), _ptr(post_pad),
                         int(num_tokens), int(top_k), int(num_experts), N, K,
                         moe_wgrad_block_m(), expert_ids.numel(), _ptr(out), _stream(stream)))
    return out


_warned_padding = False


def moe_w4a16_layer(x, topk_ids, topk_w, w1, s1, w2, s2, b1=None, b2=None, num_tokens=None,
                    pad_token_dim=False, stream=None):
    """The W4A16 MXFP4 expert layer: align -> gate+up GEMM with SwiGLU ->
    down GEMM -> top-k combine. Returns y bf16 [num_tokens, H]. w1 / w2 are
    rows-layout codes with scales s1 / s2, or PackedWeights (s1 / s2 None).

    With pad_token_dim, the token dimension is run at its bucket
    (moe_bucket_round_up): the caller's x / topk_ids / topk_w must hold at
    least that many rows (the rows past num_tokens are the padding; their
    contents cannot change the real rows' results), and only the real rows of
    y are formed. Padding is honoured only where moe_padding_supported() says
    it is exact (bf16 activations x MXFP4 weights); elsewhere it is ignored
    with a warning.
    """
    global _warned_padding
    T = x.shape[0] if num_tokens is None else int(num_tokens)
    Tr = T
    if pad_token_dim:
        if moe_padding_supported(MOE_BF16, MOE_E2M1X2):
            Tr = moe_bucket_round_up(T)
        elif not _warned_padding:
            import warnings
            warnings.warn("pad_token_dim ignored: padding is exact only for W4A16 MXFP4")
            _warned_padding = True
    if x.shape[0] < Tr or topk_ids.shape[0] < Tr:
        raise ValueError(f"pad_token_dim needs {Tr} rows in x and topk_ids (bucket of {T})")
    k = topk_ids.shape[1]
    E = w1.num_experts if isinstance(w1, PackedWeights) else w1.shape[0]
    bm = moe_gemm_block_m("e2m1x2", Tr)
    routing = moe_align(topk_ids, E, bm, num_tokens=Tr, stream=stream)
    h = moe_grouped_gemm(x, w1, "e2m1x2", routing, Tr, k, E, a_row_div=k, w_scale=s1, bias=b1,
                         epilogue="swiglu", stream=stream)
    c2 = moe_grouped_gemm(h, w2, "e2m1x2", routing, Tr, k, E, a_row_div=1, w_scale=s2, bias=b2,
                          stream=stream)
    return moe_combine(c2, topk_w, k, num_tokens=T, stream=stream)


def moe_relu2_layer(x, topk_ids, topk_w, w1, w2, b1=None, b2=None, num_tokens=None, stream=None):
    """The non-gated squared-ReLU expert layer (the Nemotron decode shape):
    align -> up GEMM with h = max(pre, 0)^2 -> down GEMM -> top-k combine, bf16
    weights (rows layout [E, N, H] and [E, H, N], or PackedWeights). Token
    counts up to moe_decode_max_tokens() run the decode GEMM. Returns y bf16
    [num_tokens, H]."""
    T = x.shape[0] if num_tokens is None else int(num_tokens)
    k = topk_ids.shape[1]
    E = w1.num_experts if isinstance(w1, PackedWeights) else w1.shape[0]
    routing = moe_align(topk_ids, E, moe_gemm_block_m("bf16", T), num_tokens=T, stream=stream)
    h = moe_grouped_gemm(x, w1, "bf16", routing, T, k, E, a_row_div=k, bias=b1, epilogue="relu2", stream=stream)
    c2 = moe_grouped_gemm(h, w2, "bf16", routing, T, k, E, a_row_div=1, bias=b2, stream=stream)
    return moe_combine(c2, topk_w, k, num_tokens=T, stream=stream)
