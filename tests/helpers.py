"""Helpers shared by the tests: the parity bar, raw-encoding conversion and
a guard that a device is present."""

import numpy as np
import pytest
import torch

import synth

# Floating-point parity bar: per output tensor, max|gpu - oracle| <= REL * max|oracle|
# over the finite entries, with fp32 accumulation; NaN positions must agree.
# A top-k combine's y is rounded twice, when C is stored in bf16 and when y
# is: it is measured against the size of its terms plus its own
# (combine_scale), each store moving it by up to 2^-8 of the size it rounds.
REL = 5e-3


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def to_dev(d, device="cuda"):
    """Move the tensors of a synth dict to the device."""
    return {k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


class LazyRows:
    """Host view of a large device tensor that copies only the rows the oracle
    indexes (an expert's weights, a set of activation rows)."""

    def __init__(self, t):
        self.t = t
        self.shape = tuple(t.shape)

    def __getitem__(self, i):
        if isinstance(i, np.ndarray):
            i = torch.from_numpy(i.astype(np.int64)).to(self.t.device)
        return synth.bits(self.t[i])


def host(d, lazy_above=1 << 24):
    """Raw encodings (numpy) of the tensors of a synth dict; tensors with more
    than `lazy_above` elements become LazyRows."""
    out = {}
    for k, v in d.items():
        if isinstance(v, torch.Tensor):
            out[k] = LazyRows(v) if v.numel() > lazy_above else synth.bits(v)
        else:
            out[k] = v
    return out


def bf16_to_f64(t):
    return t.detach().float().cpu().double().numpy()


def combine_scale(c, topk_w, top_k):
    """The size a top-k combine's y is measured against: the largest finite
    sum_j |w[t, j]| * |c[t * top_k + j, n]| + |y[t, n]| for c [T * top_k, N]
    (float64) and topk_w [T, top_k]. The GPU stores C in bf16 and then y: the
    first store moves y by up to 2^-8 of sum_j |w| |C|, the second by up to
    2^-8 of |y|."""
    c = np.asarray(c, dtype=np.float64)
    w = np.asarray(topk_w, dtype=np.float64).reshape(-1, top_k)
    T = w.shape[0]
    if T == 0 or c.shape[1] == 0:
        return 0.0
    c3 = c[:T * top_k].reshape(T, top_k, -1)
    terms = np.abs(c3 * w[:, :, None])
    size = terms.sum(axis=1) + np.abs((c3 * w[:, :, None]).sum(axis=1))
    fin = np.isfinite(size)
    return float(size[fin].max()) if fin.any() else 0.0


def assert_parity(gpu, ref, rel=REL, what="", scale=None):
    """max|gpu - ref| <= rel * scale over finite entries (scale defaults to
    max|ref|, never below it); NaN masks equal."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    ng, nr = np.isnan(gpu), np.isnan(ref)
    assert np.array_equal(ng, nr), f"{what}: NaN positions differ ({ng.sum()} vs {nr.sum()})"
    fin = ~nr
    if not fin.any():
        return 0.0
    scale = max(np.abs(ref[fin]).max(), scale or 0.0)
    err = np.abs(gpu[fin] - ref[fin]).max()
    assert err <= rel * scale, f"{what}: max err {err:.3e} > {rel} * {scale:.3e}"
    return err / scale if scale else 0.0
