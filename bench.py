"""Benchmark of the MoE expert-layer hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--phase both|cold|warm]
                    [--workload decode|nemotron|w4a16|mxfp8|mxfp8a|pertoken|wgrad|copy]

Prints one JSON line. The default workload is the bf16 decode MoE
(E=128, N=1856, K=2048, top-6) at the MTP6 verify token counts
M = 1, 7, 14, 21, 28; a step runs, for each M, the decode MoE step (routing,
grouped GEMM, top-k combine) through the fused layer moe_decode_layer (one
launch), and the same step through the three launches moe_align -> decode
grouped GEMM -> moe_combine.

Headline (`value`, `roofline`): the fused decode step with a cold cache.
Every call runs on a routing and activations drawn for it alone, after a
1 GiB device copy that evicts the previous call's weights from the 256 MB
MALL and the L2s, and its inputs (activations, routing) are then written by
small copies as their producers would, so only the weights are cold; HIP
events on the launch stream bracket each call (the copies are outside), and
a GPU spin at the head of each step lets the host queue the whole step
first. `value` = the bytes the timed calls must move (touched experts'
weights, activations, ids and routing weights in, y out) over their summed
event time (GB/s); `roofline` = the same for the layer kernel, the step's
only launch. `cold.per_m` gives median / p10 / p90 per M for both paths;
`cold.three_launch` the three-launch figures and the decode GEMM's own
roofline; `cold_k2688` the fused layer on the same protocol at the page
recipe's hidden size, K = 2688. `warm` holds both paths warm (graph-replayed steps on a cycled set
of routings, and back-to-back launches of the layer kernel and of the
decode GEMM).
`large_m` holds the large-M half of the metric: the W4A16 gate+up GEMM (and
its down GEMM under `large_m.w4a16.down`), the MXFP8 grouped GEMM and the
weight gradient, each kernel's TFLOP/s and fraction of the bf16 MFMA peak
and of HBM bandwidth. The GPU clock (amdsmi, read-only) is sampled in each
timed region.

The other workloads (the Nemotron relu2 decode layer, the W4A16 layer, the
MXFP8 grouped GEMM with bf16 or MXFP8 activations, the per-token-scaled FP8
grouped GEMM over group_sizes, the weight gradient, a 1 GiB copy) are
selected with --workload and measured warm.

Inputs are synthetic (seeded), generated on the device before any timed
region. The CPU baseline is the float64 oracle on a bounded sample of the same
workload, timed on this host.
"""

import argparse
import gc
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP8_TFLOPS = 5000.0
METRIC = "grouped-GEMM TFLOP/s & % MFMA peak (large M); decode µs/call & % HBM BW"
DECODE_LAYER_KERNEL = "moe_decode_layer_kernel"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="decode",
                    choices=["decode", "nemotron", "w4a16", "mxfp8", "mxfp8a", "pertoken", "wgrad", "copy"])
    ap.add_argument("--variants", type=int, default=4, help="routing variants cycled across steps")
    ap.add_argument("--launch-reps", type=int, default=5,
                    help="launches of the dominant kernel per step when timing it (one event pair each, "
                         "back to back)")
    ap.add_argument("--layout", default="auto", choices=["auto", "rows", "kblock"],
                    help="expert weight layout: rows ([E][N][K]) or kblock (packed once by moe_pack_weights "
                         "before timing); auto = kblock for the large-M workloads, rows for decode")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--counters-from", metavar="DIR",
                    help="no GPU run: read rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE csv files (-o fetch, -o write) "
                         "from DIR and record the workload's per-launch HBM traffic in profiles/counters.json")
    ap.add_argument("--counters-key", choices=["decode_layer"],
                    help="with --counters-from: record the fused decode layer kernel's traffic (the cold "
                         "decode headline) instead of the workload's dominant kernel")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU-oracle sample time")
    ap.add_argument("--phase", default="both", choices=["both", "cold", "warm"],
                    help="decode workload: cold-cache calls (the headline), warm graph replays, or both "
                         "(both also runs the large-M block)")
    ap.add_argument("--no-large-m", action="store_true", help="decode workload: skip the large-M block")

    return ap.parse_args()


# sources whose change can change a workload's dominant kernel
KERNEL_SOURCES = {"decode": ["decode.hip"], "decode_layer": ["decode_layer.hip", "decode_layer.h"],
                  "nemotron": ["decode.hip"], "w4a16": ["gemm.hip", "gemm_util.h"],
                  "mxfp8": ["gemm.hip", "gemm_util.h"], "mxfp8a": ["gemm_f8.hip", "gemm_util.h"],
                  "pertoken": ["gemm_f8.hip", "gemm_util.h"],
                  "wgrad": ["wgrad.hip"], "copy": []}


def kernel_source_hash(workload):
    """Hash of the source files the workload's dominant kernel is built from
    (its own file plus the shared headers)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mixture_experts_grouped_moe_amd", "csrc")
    for name in KERNEL_SOURCES[workload] + (["common.h", "params.h"] if KERNEL_SOURCES[workload] else []):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


# HBM byte counters, calibrated on a plain 1 GiB device copy (the copy
# workload): rocprofv3 reads FETCH_SIZE = 524302 KiB for its 1 GiB of reads and
# WRITE_SIZE = 1048576 KiB for its 1 GiB of writes.
FETCH_FACTOR = 2.0
WRITE_FACTOR = 1.0


def record_counters(workload, directory):
    """Average FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the workload's
    dominant kernel over the dispatches in the two rocprofv3 csv files, scale
    them by the copy calibration and store the result in profiles/counters.json
    under the current kernel source hash."""
    import csv
    key = DECODE_LAYER_KERNEL if workload == "decode_layer" else WORKLOADS[workload].dominant
    per = {}
    for counter, stem in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write")):
        path = os.path.join(directory, f"{stem}_counter_collection.csv")
        vals = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter and key in r["Kernel_Name"]:
                    vals[r["Dispatch_Id"]] = vals.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
        if not vals:
            raise SystemExit(f"no {counter} rows for {key} in {path}")
        per[counter] = (sum(vals.values()) / len(vals), len(vals))
    fetch_kib, n_fetch = per["FETCH_SIZE"]
    write_kib, n_write = per["WRITE_SIZE"]
    hbm = (fetch_kib * FETCH_FACTOR + write_kib * WRITE_FACTOR) * 1024
    out = os.path.join(ROOT, "profiles", "counters.json")
    data = {}
    if os.path.exists(out):
        with open(out) as f:
            data = json.load(f)
    data[workload] = {"kernel": key, "source_hash": kernel_source_hash(workload),
                      "fetch_kib_per_dispatch": round(fetch_kib, 1), "write_kib_per_dispatch": round(write_kib, 1),
                      "dispatches": [n_fetch, n_write], "fetch_factor": FETCH_FACTOR, "write_factor": WRITE_FACTOR,
                      "hbm_bytes_per_launch": round(hbm)}
    with open(out, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps({workload: data[workload]}))


def load_traffic(kernel_key, launches_units):
    """HBM traffic per launch from committed rocprofv3 counter summaries, if
    they were taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    ent = data.get(kernel_key)
    if not ent or ent.get("source_hash") != kernel_source_hash(kernel_key):
        return None
    return ent.get("hbm_bytes_per_launch")


# --------------------------------------------------------------------------- workloads

class LazyRows:
    """Host view of a device tensor that copies one leading-index slice (an
    expert's weights) on first use and keeps it, so the CPU oracle's timed
    passes read host memory only."""

    def __init__(self, t):
        self.t, self.shape, self.cache = t, tuple(t.shape), {}

    def __getitem__(self, i):
        import synth
        i = int(i)
        if i not in self.cache:
            self.cache[i] = synth.bits(self.t[i])
        return self.cache[i]


class Workload:
    """A set of pre-generated inputs and the launches of one step."""
    name = ""
    dominant = ""          # kernel name as rocprofv3 reports it (prefix)
    bound = "hbm"

    def step(self, v):            # eager launches of one step on the current stream
        raise NotImplementedError

    def dominant_launches(self, v):  # list of (callable, algorithmic units) for the dominant kernel
        raise NotImplementedError


LAYOUT = {"decode": "rows", "nemotron": "rows", "w4a16": "kblock", "mxfp8": "kblock", "mxfp8a": "kblock",
          "pertoken": "kblock"}  # resolved --layout per workload


def _gemm_weights(moe, name, w, w_dtype, w_scale):
    """The weights the timed GEMMs read: as drawn (rows layout) or packed once
    into the K-block layout (a weight-load-time step, outside the timing)."""
    if LAYOUT.get(name) == "kblock":
        return moe.moe_pack_weights(w, w_dtype, w_scale=w_scale), None
    return w, w_scale


def _routing_buffers(torch, T, k, E, bm, dev):
    import mixture_experts_grouped_moe_amd as moe
    mb = moe.moe_align_max_blocks(T * k, E, bm)
    return (torch.empty(mb * bm, dtype=torch.int32, device=dev),
            torch.empty(mb, dtype=torch.int32, device=dev),
            torch.empty(1, dtype=torch.int32, device=dev))


class Decode(Workload):
    name = "decode"
    dominant = "moe_decode_kernel"
    bound = "hbm"
    MS = (1, 7, 14, 21, 28)

    def __init__(self, torch, dev, variants):
        import numpy as np
        import mixture_experts_grouped_moe_amd as moe
        import synth
        self.torch, self.moe = torch, moe
        self.E, self.N, self.K, self.k = 128, 1856, 2048, 6
        self.w = synth.bf16_normal((self.E, self.N, self.K), 0.02, 1002, "w", dev)
        self.wg, _ = _gemm_weights(moe, self.name, self.w, "bf16", None)
        self.calls = []   # per variant: list of dicts per M
        self.bytes_gemm = []  # per variant: list of algorithmic GEMM bytes per M
        for v in range(variants):
            per_m, per_b = [], []
            for M in self.MS:
                x = synth.bf16_normal((M, self.K), 1.0, 1002, f"x{M}v{v}", dev)
                ids, tw = synth.softmax_topk_routing(M, self.E, self.k, 1002, f"route{M}v{v}", dev)
                bm = moe.moe_gemm_block_m("bf16", M)
                c = dict(M=M, x=x, ids=ids, tw=tw, bm=bm,
                         routing=_routing_buffers(torch, M, self.k, self.E, bm, dev),
                         C=torch.empty((M * self.k, self.N), dtype=torch.bfloat16, device=dev),
                         y=torch.empty((M, self.N), dtype=torch.bfloat16, device=dev))
                touched = len(np.unique(ids.cpu().numpy()))
                c["touched"] = touched
                per_b.append(touched * self.N * self.K * 2 + M * self.K * 2 + M * self.k * self.N * 2)
                per_m.append(c)
            self.calls.append(per_m)
            self.bytes_gemm.append(per_b)

    def _call_bytes(self, v, i):
        c = self.calls[v][i]
        S = c["M"] * self.k
        mb = c["routing"][1].numel()
        align = S * 4 + mb * c["bm"] * 4 + mb * 4 + 4
        combine = S * self.N * 2 + c["M"] * self.N * 2 + S * 4
        return self.bytes_gemm[v][i] + align + combine

    def step_bytes(self, v):
        return sum(self._call_bytes(v, i) for i in range(len(self.MS)))

    def step_flops(self, v):
        return sum(2 * c["M"] * self.k * self.N * self.K for c in self.calls[v])

    def _gemm(self, c):
        if "gemm_call" not in c:
            c["gemm_call"], _ = self.moe.moe_grouped_gemm_prepare(
                c["x"], self.wg, "bf16", c["routing"], c["M"], self.k, self.E, self.k, out=c["C"])
        return c["gemm_call"]()

    def step(self, v):
        moe = self.moe
        for c in self.calls[v]:
            moe.moe_align(c["ids"], self.E, c["bm"], out=c["routing"])
            self._gemm(c)
            moe.moe_combine(c["C"], c["tw"], self.k, out=c["y"])

    def dominant_launches(self, v):
        return [(lambda c=c: self._gemm(c), self.bytes_gemm[v][i]) for i, c in enumerate(self.calls[v])]

    def extra(self, per_call_us):
        return {"us_per_call": {str(M): round(t, 2) for M, t in zip(self.MS, per_call_us)},
                "touched_experts": {str(M): self.calls[0][i]["touched"] for i, M in enumerate(self.MS)}}

    cpu_sample_desc = "align + decode GEMM + combine for M = 1, 7, 14, 21, 28 of routing variant 0"

    def cpu_sample(self):
        """Oracle on variant 0, all five calls (align + GEMM + combine)."""
        import synth
        from oracle import align as oalign, gemm as ogemm
        lw = LazyRows(self.w)
        items = []
        for i, c in enumerate(self.calls[0]):
            items.append((synth.bits(c["x"]), synth.bits(c["ids"]), synth.bits(c["tw"]), c["bm"], i))

        def run(item):
            x, ids, tw, bm, i = item
            oalign.moe_align(ids, self.E, bm)
            C, _ = ogemm.grouped_gemm(x, self.k, lw, "bf16", None, ids, self.E)
            ogemm.combine(C, tw, self.k)
            return self._call_bytes(0, i)
        return items, run, "GB/s"


class DecodeFused(Decode):
    """The decode workload through the fused layer (moe_decode_layer): one
    launch per M does the routing, the GEMM and the combine."""
    name = "decode_layer"
    dominant = DECODE_LAYER_KERNEL

    def _layer(self, c):
        if "layer_call" not in c:
            c["layer_call"], _ = self.moe.moe_decode_layer_prepare(c["x"], c["ids"], c["tw"], self.wg, "bf16",
                                                                   out=c["y"])
        return c["layer_call"]()

    def _layer_bytes(self, v, i):
        c = self.calls[v][i]
        S = c["M"] * self.k
        return c["touched"] * self.N * self.K * 2 + c["M"] * self.K * 2 + S * 8 + c["M"] * self.N * 2

    def step_bytes(self, v):
        return sum(self._layer_bytes(v, i) for i in range(len(self.MS)))

    def step(self, v):
        for c in self.calls[v]:
            self._layer(c)

    def dominant_launches(self, v):
        return [(lambda c=c: self._layer(c), self._layer_bytes(v, i)) for i, c in enumerate(self.calls[v])]


class Nemotron(Workload):
    """The Nemotron-shaped non-gated squared-ReLU decode layer (E=128, top-6,
    hidden 2688, N=1856, bf16) at M = 1, 7, 14, 21, 28: per M one step runs
    moe_align -> up GEMM with relu2 -> down GEMM -> moe_combine, both GEMMs on
    the decode kernel. The line also times the mid-M bucket (M = 64, 120) on
    the large-M kernel (`mid_m`)."""
    name = "nemotron"
    dominant = "moe_decode_kernel"
    bound = "hbm"
    MS = (1, 7, 14, 21, 28)
    cpu_sample_desc = "the whole relu2 layer (align, both GEMMs, combine) for M = 1 and 7 of routing variant 0"

    def __init__(self, torch, dev, variants):
        import numpy as np
        import mixture_experts_grouped_moe_amd as moe
        import synth
        self.torch, self.moe = torch, moe
        self.E, self.H, self.N, self.k = 128, 2688, 1856, 6
        d = synth.nemotron_layer(1, device=dev)
        self.w1, self.w2 = d["w1"], d["w2"]
        self.calls, self.bytes_gemm = [], []
        for v in range(variants):
            per_m, per_b = [], []
            for M in self.MS:
                dm = synth.nemotron_layer(M, seed=1006 + 100 * v, device=dev, weights=False)
                bm = moe.moe_gemm_block_m("bf16", M)
                S = M * self.k
                c = dict(M=M, x=dm["x"], ids=dm["ids"], tw=dm["topk_w"], bm=bm,
                         routing=_routing_buffers(torch, M, self.k, self.E, bm, dev),
                         h=torch.empty((S, self.N), dtype=torch.bfloat16, device=dev),
                         c2=torch.empty((S, self.H), dtype=torch.bfloat16, device=dev),
                         y=torch.empty((M, self.H), dtype=torch.bfloat16, device=dev))
                c["touched"] = len(np.unique(dm["ids"].cpu().numpy()))
                wb = c["touched"] * self.N * self.H * 2
                per_b.append((wb + M * self.H * 2 + S * self.N * 2, wb + S * self.N * 2 + S * self.H * 2))
                per_m.append(c)
            self.calls.append(per_m)
            self.bytes_gemm.append(per_b)

    def _call_bytes(self, v, i):
        c = self.calls[v][i]
        S = c["M"] * self.k
        mb = c["routing"][1].numel()
        align = S * 4 + mb * c["bm"] * 4 + mb * 4 + 4
        combine = S * self.H * 2 + c["M"] * self.H * 2 + S * 4
        return sum(self.bytes_gemm[v][i]) + align + combine

    def step_bytes(self, v):
        return sum(self._call_bytes(v, i) for i in range(len(self.MS)))

    def step_flops(self, v):
        return sum(2 * 2 * c["M"] * self.k * self.N * self.H for c in self.calls[v])

    def _up(self, c):
        if "up" not in c:
            c["up"], _ = self.moe.moe_grouped_gemm_prepare(c["x"], self.w1, "bf16", c["routing"], c["M"], self.k,
                                                           self.E, self.k, epilogue="relu2", out=c["h"])
        return c["up"]()

    def _down(self, c):
        if "down" not in c:
            c["down"], _ = self.moe.moe_grouped_gemm_prepare(c["h"], self.w2, "bf16", c["routing"], c["M"], self.k,
                                                             self.E, 1, out=c["c2"])
        return c["down"]()

    def step(self, v):
        moe = self.moe
        for c in self.calls[v]:
            moe.moe_align(c["ids"], self.E, c["bm"], out=c["routing"])
            self._up(c)
            self._down(c)
            moe.moe_combine(c["c2"], c["tw"], self.k, out=c["y"])

    def dominant_launches(self, v):
        out = []
        for i, c in enumerate(self.calls[v]):
            out.append((lambda c=c: self._up(c), self.bytes_gemm[v][i][0]))
            out.append((lambda c=c: self._down(c), self.bytes_gemm[v][i][1]))
        return out

    def extra(self, per_call_us):
        us = {}
        if per_call_us is not None:
            for i, M in enumerate(self.MS):
                us[str(M)] = {"up": round(per_call_us[2 * i], 2), "down": round(per_call_us[2 * i + 1], 2)}
        out = {"us_per_gemm": us, "touched_experts": {str(M): self.calls[0][i]["touched"] for i, M in enumerate(self.MS)}}
        if per_call_us is not None:
            out["mid_m"] = self._mid_m()
        return out

    MID_MS = (64, 120)

    def _mid_m(self, reps=10):
        """The steady-state mid-M decode bucket (M ~ 115-120 tokens, and 64):
        the same layer's up and down GEMMs run on the large-M kernel (64-row
        routing blocks); each GEMM launched back to back on resident inputs,
        one event pair per launch. GB/s counts the touched experts' weights,
        the activations read and the outputs written."""
        import numpy as np
        import synth
        torch, moe = self.torch, self.moe
        res = {}
        for M in self.MID_MS:
            dm = synth.nemotron_layer(M, device=self.w1.device, weights=False)
            bm = moe.moe_gemm_block_m("bf16", M)
            routing = moe.moe_align(dm["ids"], self.E, bm)
            S = M * self.k
            touched = len(np.unique(dm["ids"].cpu().numpy()))
            h = torch.empty((S, self.N), dtype=torch.bfloat16, device=self.w1.device)
            c2 = torch.empty((S, self.H), dtype=torch.bfloat16, device=self.w1.device)
            up, _ = moe.moe_grouped_gemm_prepare(dm["x"], self.w1, "bf16", routing, M, self.k, self.E, self.k,
                                                 epilogue="relu2", out=h)
            down, _ = moe.moe_grouped_gemm_prepare(h, self.w2, "bf16", routing, M, self.k, self.E, 1, out=c2)
            wb = touched * self.N * self.H * 2
            entry = {"touched_experts": touched}
            for name, fn, nbytes in (("up", up, wb + M * self.H * 2 + S * self.N * 2),
                                     ("down", down, wb + S * self.N * 2 + S * self.H * 2)):
                for _ in range(3):
                    fn()
                ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
                for a, b in ev:
                    a.record()
                    fn()
                    b.record()
                torch.cuda.synchronize()
                t = float(np.median([a.elapsed_time(b) * 1e3 for a, b in ev]))
                entry[name] = {"us": round(t, 1), "GBps": round(nbytes / t / 1e3, 1),
                               "hbm_frac": round(nbytes / t / 1e3 / PEAK_HBM_GBS, 4)}
            res[str(M)] = entry
        return res

    def cpu_sample(self):
        import synth
        from oracle import align as oalign, layer as olayer
        lw1, lw2 = LazyRows(self.w1), LazyRows(self.w2)
        items = []
        for i, c in enumerate(self.calls[0][:2]):
            items.append((synth.bits(c["x"]), synth.bits(c["ids"]), synth.bits(c["tw"]), c["bm"], i))

        def run(item):
            x, ids, tw, bm, i = item
            oalign.moe_align(ids, self.E, bm)
            olayer.relu2_layer(x, ids, tw, self.k, self.E, lw1, None, lw2, None)
            return self._call_bytes(0, i)
        return items, run, "GB/s"


class W4A16(Workload):
    name = "w4a16"
    dominant = "moe_gemm_kernel<4, true"
    bound = "mfma"

    def __init__(self, torch, dev, variants):
        import mixture_experts_grouped_moe_amd as moe
        import synth
        self.torch, self.moe = torch, moe
        self.E, self.H, self.I, self.k = 128, 2880, 2880, 4
        d = synth.config3(8192, device=dev)
        self.d = d
        self.w1, self.s1 = _gemm_weights(moe, self.name, d["w1"], "e2m1x2", d["s1"])
        self.w2, self.s2 = _gemm_weights(moe, self.name, d["w2"], "e2m1x2", d["s2"])
        self.Ts = synth.draw_token_counts(variants, 6554, 8192, seed=1003)
        self.calls = []
        for T in self.Ts:
            Tb = moe.moe_bucket_round_up(T)
            x = d["x"][:Tb].clone()
            x[T:] = 0
            bm = moe.moe_gemm_block_m("e2m1x2", Tb)
            self.calls.append(dict(T=T, Tb=Tb, x=x, ids=d["ids"][:Tb].contiguous(), tw=d["topk_w"][:Tb].contiguous(),
                                   bm=bm, routing=_routing_buffers(torch, Tb, self.k, self.E, bm, dev),
                                   h=torch.empty((Tb * self.k, self.I), dtype=torch.bfloat16, device=dev),
                                   c2=torch.empty((Tb * self.k, self.H), dtype=torch.bfloat16, device=dev),
                                   y=torch.empty((T, self.H), dtype=torch.bfloat16, device=dev)))

    def step_flops(self, v):
        T = self.calls[v]["T"]
        return 2 * T * self.k * (2 * self.I * self.H + self.H * self.I)

    def step_bytes(self, v):
        c = self.calls[v]
        S = c["T"] * self.k
        w = self.E * (2 * self.I * self.H + self.H * self.I) // 2 * (1 + 1 / 16)
        return int(w + c["T"] * self.H * 2 + S * self.I * 2 * 2 + S * self.H * 2 * 2 + c["T"] * self.H * 2)

    def _up(self, c):
        d = self.d
        return self.moe.moe_grouped_gemm(c["x"], self.w1, "e2m1x2", c["routing"], c["Tb"], self.k, self.E, self.k,
                                         w_scale=self.s1, epilogue="swiglu", out=c["h"])

    def step(self, v):
        c, d, moe = self.calls[v], self.d, self.moe
        moe.moe_align(c["ids"], self.E, c["bm"], out=c["routing"])
        self._up(c)
        self._down(c)
        moe.moe_combine(c["c2"], c["tw"], self.k, num_tokens=c["T"], out=c["y"])

    def dominant_launches(self, v):
        c = self.calls[v]
        return [(lambda c=c: self._up(c), 2 * c["T"] * self.k * 2 * self.I * self.H)]

    def dominant_flops_bytes(self, v):
        """Algorithmic flops and HBM bytes of the gate+up GEMM: the 128
        experts' E2M1 codes and E8M0 bytes, the token rows read, h written."""
        T = self.calls[v]["T"]
        w = self.E * 2 * self.I * self.H // 2 * (1 + 1 / 16)
        return 2 * T * self.k * 2 * self.I * self.H, int(w + T * self.H * 2 + T * self.k * self.I * 2)

    def _down(self, c):
        return self.moe.moe_grouped_gemm(c["h"], self.w2, "e2m1x2", c["routing"], c["Tb"], self.k, self.E, 1,
                                         w_scale=self.s2, out=c["c2"])

    def second_launches(self, v):
        """The down GEMM (K = 2880 over h's slot rows, N = 2880), with its
        algorithmic flops and HBM bytes (codes and scales, h read, C written)."""
        c = self.calls[v]
        S = c["T"] * self.k
        w = self.E * self.H * self.I // 2 * (1 + 1 / 16)
        return "down", [(lambda c=c: self._down(c), 2 * S * self.H * self.I,
                         int(w + S * self.I * 2 + S * self.H * 2))]

    def extra(self, per_call_us):
        return {"tokens": [c["T"] for c in self.calls], "buckets": [c["Tb"] for c in self.calls]}

    def dense_shapes(self, v):
        """(M, N, K) of the gate+up and the down products of variant v."""
        S = self.calls[v]["T"] * self.k
        return {"up": (S, 2 * self.I, self.H), "down": (S, self.H, self.I)}

    cpu_sample_desc = "gate+up GEMM with SwiGLU and down GEMM over all slots of experts 0-3"

    def cpu_sample(self):
        """Oracle layer on the slots of 4 experts of variant 0 (up and down GEMM rows)."""
        import numpy as np
        import synth
        from oracle import layer as olayer
        c = self.calls[0]
        ids = synth.bits(c["ids"])[:c["T"]]
        d = self.d
        xs = synth.bits(c["x"])
        w1, s1, w2, s2 = LazyRows(d["w1"]), LazyRows(d["s1"]), LazyRows(d["w2"]), LazyRows(d["s2"])
        flat = ids.reshape(-1)
        items = []
        for e in range(4):
            slots = np.nonzero(flat == e)[0]
            items.append(slots)

        def run(slots):
            olayer.w4a16_layer(xs, ids, None, self.k, self.E, w1, s1, None, w2, s2, None, slots=slots)
            return 2 * len(slots) * (2 * self.I * self.H + self.H * self.I)
        return items, run, "TFLOP/s"


class MXFP8(Workload):
    name = "mxfp8"
    cpu_sample_desc = "grouped GEMM over all slots of the median-load and the top-load expert"
    dominant = "moe_gemm_kernel<3, false"
    bound = "hbm"

    def __init__(self, torch, dev, variants, bias=False):
        import numpy as np
        import mixture_experts_grouped_moe_amd as moe
        import synth
        self.torch, self.moe = torch, moe
        d = synth.config4(device=dev, bias=bias)
        self.d = d
        self.wg, self.sg = _gemm_weights(moe, self.name, d["w"], "e4m3", d["w_scale"])
        self.E, self.N, self.K, self.k, self.T = 256, 4096, 7168, 8, 4096
        bm = moe.moe_gemm_block_m("e4m3", self.T)
        self.bm = bm
        self.routing = _routing_buffers(torch, self.T, self.k, self.E, bm, dev)
        self.C = torch.empty((self.T * self.k, self.N), dtype=torch.bfloat16, device=dev)
        counts = np.bincount(synth.bits(d["ids"]).reshape(-1), minlength=self.E)
        self.touched = int((counts > 0).sum())
        self.empty = int((counts == 0).sum())

    def step_flops(self, v):
        return 2 * self.T * self.k * self.N * self.K

    def gemm_bytes(self):
        w = self.touched * self.N * self.K * (1 + 1 / 32)
        return int(w + self.T * self.K * 2 + self.T * self.k * self.N * 2)

    def step_bytes(self, v):
        return self.gemm_bytes()

    def _gemm(self):
        d = self.d
        return self.moe.moe_grouped_gemm(d["x"], self.wg, "e4m3", self.routing, self.T, self.k, self.E, self.k,
                                         w_scale=self.sg, bias=d["bias"], out=self.C)

    def step(self, v):
        self.moe.moe_align(self.d["ids"], self.E, self.bm, out=self.routing)
        self._gemm()

    def dominant_launches(self, v):
        return [(self._gemm, self.gemm_bytes())]

    def dominant_flops_bytes(self, v):
        return self.step_flops(v), self.gemm_bytes()

    def extra(self, per_call_us):
        return {"touched_experts": self.touched, "empty_experts": self.empty}

    def dense_shapes(self, v):
        return {"gemm": (self.T * self.k, self.N, self.K)}

    def cpu_sample(self):
        import numpy as np
        import synth
        from oracle import gemm as ogemm
        d = self.d
        ids = synth.bits(d["ids"])
        flat = ids.reshape(-1)
        x, w, ws = synth.bits(d["x"]), LazyRows(d["w"]), LazyRows(d["w_scale"])
        counts = np.bincount(flat, minlength=self.E)
        order = np.argsort(counts)
        experts = [int(order[len(order) // 2]), int(order[-1])]
        items = [np.nonzero(flat == e)[0] for e in experts]

        def run(slots):
            ogemm.grouped_gemm(x, self.k, w, "e4m3", ws, ids, self.E, slots=slots)
            return 2 * len(slots) * self.N * self.K
        return items, run, "TFLOP/s"


class MXFP8A(MXFP8):
    """The MXFP8 workload with MXFP8 activations: each step converts the bf16
    activations (E4M3 codes + E8M0 per 32 along K) and runs the both-operands
    MXFP8 grouped GEMM on the scaled fp8 MFMA."""
    name = "mxfp8a"
    cpu_sample_desc = ("MXFP8 conversion of the activation rows and grouped GEMM over all slots of the "
                       "median-load and the top-load expert")
    dominant = "moe_gemm_f8_kernel"
    bound = "hbm"

    def __init__(self, torch, dev, variants, bias=False):
        super().__init__(torch, dev, variants, bias)
        moe = self.moe
        self.bm = moe.moe_gemm_block_m("e4m3", self.T, moe.MOE_E4M3)
        self.routing = _routing_buffers(torch, self.T, self.k, self.E, self.bm, dev)
        self.q = torch.empty((self.T, self.K), dtype=torch.uint8, device=dev)
        self.qs = torch.empty((self.T, self.K // 32), dtype=torch.uint8, device=dev)
        moe.moe_align(self.d["ids"], self.E, self.bm, out=self.routing)
        moe.moe_quantize_mxfp8(self.d["x"], out=self.q, out_scales=self.qs)

    def gemm_bytes(self):
        w = self.touched * self.N * self.K * (1 + 1 / 32)
        return int(w + self.T * self.K * (1 + 1 / 32) + self.T * self.k * self.N * 2)

    def step_bytes(self, v):
        return self.gemm_bytes() + self.T * self.K * 2  # + the conversion's bf16 reads

    def _gemm(self):
        return self.moe.moe_grouped_gemm(self.q, self.wg, "e4m3", self.routing, self.T, self.k, self.E, self.k,
                                         w_scale=self.sg, bias=self.d["bias"], out=self.C, a_scale=self.qs)

    def step(self, v):
        self.moe.moe_align(self.d["ids"], self.E, self.bm, out=self.routing)
        self.moe.moe_quantize_mxfp8(self.d["x"], out=self.q, out_scales=self.qs)
        self._gemm()

    def cpu_sample(self):
        import numpy as np
        import synth
        from oracle import gemm as ogemm
        from oracle import quant as oquant
        d = self.d
        ids = synth.bits(d["ids"])
        flat = ids.reshape(-1)
        x = d["x"]
        w, ws = LazyRows(d["w"]), LazyRows(d["w_scale"])
        counts = np.bincount(flat, minlength=self.E)
        order = np.argsort(counts)
        experts = [int(order[len(order) // 2]), int(order[-1])]
        items = []
        for e in experts:
            slots = np.nonzero(flat == e)[0]
            rows = np.unique(slots // self.k)
            items.append((slots, rows, x[torch_index(rows)].float().cpu().double().numpy()))

        def run(item):
            slots, rows, xr = item
            q = np.zeros((self.T, self.K), dtype=np.uint8)
            s = np.zeros((self.T, self.K // 32), dtype=np.uint8)
            q[rows], s[rows] = oquant.mx_quantize_e4m3(xr)
            ogemm.grouped_gemm(q, self.k, w, "e4m3", ws, ids, self.E, a_dtype="e4m3", a_scale=s, slots=slots)
            return 2 * len(slots) * self.N * self.K
        return items, run, "TFLOP/s"


class PerToken(Workload):
    """Per-token-scaled FP8 grouped GEMM over the group_sizes interface at the
    MXFP8 workload's shape: each step builds the block mapping from the group
    sizes on the device and runs the GEMM (E4M3 x E4M3, per-row and
    per-expert fp32 scales after the fp8 dot product)."""
    name = "pertoken"
    cpu_sample_desc = "per-token GEMM over all rows of the median-load and the top-load expert"
    dominant = "moe_gemm_f8_kernel"
    bound = "hbm"

    def __init__(self, torch, dev, variants, bias=False):
        import mixture_experts_grouped_moe_amd as moe
        import synth
        self.torch, self.moe = torch, moe
        d = synth.config_per_token(device=dev, bias=bias)
        self.d = d
        self.E, self.N, self.K, self.R = d["E"], d["N"], d["K"], d["R"]
        self.wg = moe.moe_pack_weights(d["w"], "e4m3") if LAYOUT[self.name] == "kblock" else d["w"]
        self.mapping = moe.moe_block_mapping(d["group_sizes"], self.R)
        self.C = torch.empty((self.R, self.N), dtype=torch.bfloat16, device=dev)
        gs = synth.bits(d["group_sizes"])
        self.gs = gs
        self.touched = int((gs > 0).sum())
        self.empty = int((gs == 0).sum())

    def step_flops(self, v):
        return 2 * self.R * self.N * self.K

    def gemm_bytes(self):
        w = self.touched * self.N * self.K + self.E * 4
        return int(w + self.R * (self.K + 4) + self.R * self.N * 2)

    def step_bytes(self, v):
        return self.gemm_bytes()

    def _gemm(self):
        d = self.d
        return self.moe.moe_grouped_gemm_per_token(d["a"], d["a_scale"], self.wg, d["w_scale"], self.mapping,
                                                   bias=d["bias"], out=self.C)

    def step(self, v):
        self.moe.moe_block_mapping(self.d["group_sizes"], self.R, out=self.mapping)
        self._gemm()

    def dominant_launches(self, v):
        return [(self._gemm, self.gemm_bytes())]

    def dominant_flops_bytes(self, v):
        return self.step_flops(v), self.gemm_bytes()

    def extra(self, per_call_us):
        return {"touched_experts": self.touched, "empty_experts": self.empty}

    def cpu_sample(self):
        import numpy as np
        import synth
        from oracle import gemm as ogemm
        d = self.d
        gs = self.gs.astype(np.int64)
        offs = np.concatenate([[0], np.cumsum(gs)])
        order = np.argsort(gs)
        experts = [int(order[len(order) // 2]), int(order[-1])]
        w = LazyRows(d["w"])
        w_s = synth.bits(d["w_scale"])
        items = []
        for e in experts:
            rows = torch_index(np.arange(offs[e], offs[e + 1]))
            sub = np.zeros_like(gs)
            sub[e] = gs[e]
            items.append((synth.bits(d["a"][rows.to(d["a"].device)]),
                          synth.bits(d["a_scale"][rows.to(d["a"].device)]), sub))

        def run(item):
            a, a_s, sub = item
            ogemm.grouped_gemm_per_token(a, a_s, w, w_s, sub)
            return 2 * a.shape[0] * self.N * self.K
        return items, run, "TFLOP/s"


def torch_index(rows):
    import torch
    return torch.from_numpy(rows.astype("int64"))


class Wgrad(Workload):
    name = "wgrad"
    cpu_sample_desc = "dW of experts 0, 128 and 255"
    dominant = "wgrad_kernel"
    bound = "hbm"

    def __init__(self, torch, dev, variants):
        import mixture_experts_grouped_moe_amd as moe
        import synth
        self.torch, self.moe = torch, moe
        d = synth.config5(device=dev)
        self.d = d
        self.E, self.N, self.K, self.k, self.T = 256, 2048, 7168, 8, 16384
        self.routing = _routing_buffers(torch, self.T, self.k, self.E, moe.moe_wgrad_block_m(), dev)
        self.dw = torch.empty((self.E, self.N, self.K), dtype=torch.float32, device=dev)

    def step_flops(self, v):
        return 2 * self.T * self.k * self.N * self.K

    def wgrad_bytes(self):
        return self.E * self.N * self.K * 4 + self.T * self.K * 2 + self.T * self.k * self.N * 2

    def step_bytes(self, v):
        return self.wgrad_bytes()

    def _wgrad(self):
        d = self.d
        return self.moe.moe_wgrad(d["x"], d["grad"], self.routing, self.T, self.k, self.E, out=self.dw)

    def step(self, v):
        self.moe.moe_align(self.d["ids"], self.E, self.moe.moe_wgrad_block_m(), out=self.routing)
        self._wgrad()

    def dominant_launches(self, v):
        return [(self._wgrad, self.wgrad_bytes())]

    def dominant_flops_bytes(self, v):
        return self.step_flops(v), self.wgrad_bytes()

    def extra(self, per_call_us):
        return {}

    def cpu_sample(self):
        import numpy as np
        import synth
        from oracle import wgrad as owgrad
        d = self.d
        ids = synth.bits(d["ids"])
        x, g = synth.bits(d["x"]), synth.bits(d["grad"])
        items = [0, 128, 255]

        def run(e):
            owgrad.wgrad_expert(x, g, ids, self.k, e)
            slots = int((ids.reshape(-1) == e).sum())
            return 2 * slots * self.N * self.K
        return items, run, "TFLOP/s"


class Copy(Workload):
    """A plain device-to-device copy of a known size (1 GiB): the reference
    kernel against which the HBM byte counters are calibrated."""
    name = "copy"
    dominant = "__amd_rocclr_copyBuffer"
    bound = "hbm"
    cpu_sample_desc = "numpy copy of 64 MiB"

    def __init__(self, torch, dev, variants):
        self.torch = torch
        self.n = 1 << 30
        self.src = torch.ones(self.n, dtype=torch.uint8, device=dev)
        self.dst = torch.empty(self.n, dtype=torch.uint8, device=dev)

    def step_flops(self, v):
        return 0

    def step_bytes(self, v):
        return 2 * self.n

    def _copy(self):
        self.dst.copy_(self.src)

    def step(self, v):
        self._copy()

    def dominant_launches(self, v):
        return [(self._copy, 2 * self.n)]

    def extra(self, per_call_us):
        return {"bytes_copied": self.n}

    def cpu_sample(self):
        import numpy as np
        a = np.ones(1 << 26, dtype=np.uint8)
        b = np.empty_like(a)

        def run(_):
            np.copyto(b, a)
            return 2 * a.size
        return [0], run, "GB/s"


WORKLOADS = {"decode": Decode, "nemotron": Nemotron, "w4a16": W4A16, "mxfp8": MXFP8, "mxfp8a": MXFP8A,
             "pertoken": PerToken, "wgrad": Wgrad, "copy": Copy}
CONFIG_NAMES = {
    "decode": "decode bf16 MoE, E=128 N=1856 K=2048 top-6, M in {1,7,14,21,28}",
    "nemotron": "Nemotron-shaped relu2 decode MoE layer, E=128 top-6 hidden=2688 N=1856, bf16, M in {1,7,14,21,28}",
    "w4a16": "W4A16 MXFP4 MoE layer (gpt-oss-shaped), E=128 top-4 H=2880, gate+up 5760 -> SwiGLU -> down 2880, T~U[6554,8192] bucketed",
    "mxfp8": "MXFP8 grouped GEMM, E=256 top-8 K=7168 N=4096 T=4096, Zipf(1.1) routing with 16 empty experts",
    "mxfp8a": "MXFP8 grouped GEMM with MXFP8 activations (bf16 converted each step), E=256 top-8 K=7168 N=4096 "
              "T=4096, Zipf(1.1) routing with 16 empty experts",
    "pertoken": "per-token-scaled FP8 grouped GEMM over group_sizes, E=256 K=7168 N=4096, 32768 rows "
                "(4096 tokens x top-8) grouped by Zipf(1.1) top-8 counts with 16 empty experts",
    "wgrad": "moe_wgrad, E=256 top-8 T=16384, x [T,7168], grad [8T,2048], fp32 dW [256,2048,7168]",
    "copy": "device-to-device copy of 1 GiB (counter calibration)",
}


def cpu_baseline(wl, target_s):
    """Time the float64 oracle on a bounded sample of the workload."""
    import numpy as np
    items, run, unit = wl.cpu_sample()
    cores = len(os.sched_getaffinity(0))
    for it in items:  # untimed pass: moves the sample's device data to host memory
        run(it)
    done_units, n, t0 = 0, 0, time.perf_counter()
    while True:  # cycle over the sample until the time target (at least one pass)
        done_units += run(items[n % len(items)])
        n += 1
        if n >= len(items) and time.perf_counter() - t0 > target_s:
            break
    dt = time.perf_counter() - t0
    scale = 1e9 if unit == "GB/s" else 1e12
    blas = "unknown"
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        threads = max((i.get("num_threads", 1) for i in info), default=1)
        libs = [i for i in info if i.get("user_api") == "blas"]
        if libs:
            blas = f"{libs[0].get('internal_api', '?')} {libs[0].get('version', '')}".strip()
    except Exception:
        threads = cores
    _ = np
    return {"value": done_units / dt / scale, "unit": unit, "cores": int(threads), "kind": "oracle",
            "blas": blas, "affinity_cpus": cores,
            "sample": f"{n} runs over a {len(items)}-item sample of the {wl.name} workload "
                      f"({wl.cpu_sample_desc}), {dt:.1f} s"}


def stats(xs):
    """median, p10, p90 and mean of a list of numbers (linear interpolation)."""
    import numpy as np
    a = np.asarray(xs, dtype=np.float64)
    return {"median": round(float(np.median(a)), 3), "p10": round(float(np.percentile(a, 10)), 3),
            "p90": round(float(np.percentile(a, 90)), 3), "mean": round(float(a.mean()), 3), "n": int(a.size)}


class ClockSampler:
    """Reads the GPU's current graphics clock through amdsmi (read-only
    queries) in a background thread while a named region runs; regions
    report the median, min and max of their samples in MHz."""

    def __init__(self, torch):
        import threading
        self.samples, self.region, self.err, self.h = {}, None, None, None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self.amdsmi = amdsmi
            handles = amdsmi.amdsmi_get_processor_handles()
            want = getattr(torch.cuda.get_device_properties(0), "pci_bus_id", None)
            self.h = handles[0]
            for h in handles:
                bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)  # "dddd:bb:dd.f"
                if want is not None and int(bdf.split(":")[1], 16) == int(want):
                    self.h = h
            self.read()
        except Exception as ex:  # no clock readings: reported as such
            self.err, self.h = f"{type(ex).__name__}: {ex}", None
        self.stop = False
        if self.h is not None:
            self.thread = threading.Thread(target=self._run, daemon=True)
            self.thread.start()

    def read(self):
        m = self.amdsmi.amdsmi_get_gpu_metrics_info(self.h)
        vals = m.get("current_gfxclks")
        if isinstance(vals, (list, tuple)):
            vals = [v for v in vals if isinstance(v, (int, float)) and 0 < v < 10000]
            if vals:
                return sum(vals) / len(vals)
        for key in ("current_gfxclk", "average_gfxclk_frequency"):
            v = m.get(key)
            if isinstance(v, (int, float)) and 0 < v < 10000:
                return float(v)
        return None

    def _run(self):
        import time as _t
        while not self.stop:
            r = self.region
            if r is not None:
                try:
                    v = self.read()
                    if v is not None:
                        self.samples.setdefault(r, []).append(v)
                except Exception as ex:
                    self.err = f"{type(ex).__name__}: {ex}"
            _t.sleep(0.01)

    def summary(self, region):
        xs = self.samples.get(region, [])
        if not xs:
            return {"mhz": None, "note": self.err or "no sample taken in this region"}
        xs = sorted(xs)
        return {"median_mhz": round(xs[len(xs) // 2]), "min_mhz": round(xs[0]), "max_mhz": round(xs[-1]),
                "samples": len(xs)}

    def close(self):
        self.stop = True


DECODE_MS = (1, 7, 14, 21, 28)
SPIN_MS = 20.0  # GPU spin ahead of each cold decode step


def spin_cycles(torch, stream, ms):
    """torch.cuda._sleep cycles that spin the GPU for about `ms` (measured)."""
    n = 1_000_000
    with torch.cuda.stream(stream):
        torch.cuda._sleep(n)  # first launch outside the measurement
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        torch.cuda._sleep(n)
        b.record(stream)
    b.synchronize()
    per_ms = n / max(a.elapsed_time(b), 1e-3)
    return int(per_ms * ms)


def decode_cold(torch, moe, dev, stream, args, clock):
    """The decode workload with a cold cache, through both of the library's
    paths for the step: the fused layer (moe_decode_layer, one launch) and
    the three launches moe_align -> decode grouped GEMM -> moe_combine. Every
    call runs on a routing and activations drawn for it alone, after a 1 GiB
    device copy (512 MiB read, 512 MiB written) that evicts the previous
    call's weights from the 256 MB MALL and the L2s; the call's activations,
    ids and routing weights are then written by small copies, as the kernels
    that produce them would, so only the expert weights are cold. The copies
    run outside the timed span: HIP events on the launch stream bracket each
    call and, inside the three-launch call, each launch. W warmup steps, then
    K timed steps; a step is, for each M in 1, 7, 14, 21, 28, one call of
    each path (each on its own draw, each after its own eviction)."""
    import numpy as np
    import synth
    E, N, K, k = 128, 1856, 2048, 6
    w = synth.bf16_normal((E, N, K), 0.02, 1002, "w", dev)
    n_steps = args.warmup + args.steps
    calls = {}
    for M in DECODE_MS:
        bm = moe.moe_gemm_block_m("bf16", M)
        lst = []
        for r in range(n_steps):
            pair = []
            for path in ("fused", "three"):
                x_src = synth.bf16_normal((M, K), 1.0, 1002, f"cold-x{M}c{r}{path}", dev)
                ids_src, tw_src = synth.softmax_topk_routing(M, E, k, 1002, f"cold-route{M}c{r}{path}", dev)
                x, ids, tw = torch.empty_like(x_src), torch.empty_like(ids_src), torch.empty_like(tw_src)
                y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
                touched = len(np.unique(ids_src.cpu().numpy()))
                S = M * k
                # what the step has to move: the touched experts' weights, the
                # activations, ids and routing weights in, y out
                step_bytes = touched * N * K * 2 + M * K * 2 + S * 4 * 2 + M * N * 2
                c = dict(path=path, srcs=((x, x_src), (ids, ids_src), (tw, tw_src)), touched=touched,
                         step_bytes=step_bytes, y=y)
                if path == "fused":
                    c["layer"], _ = moe.moe_decode_layer_prepare(x, ids, tw, w, "bf16", out=y, stream=stream)
                else:
                    routing = _routing_buffers(torch, M, k, E, bm, dev)
                    C = torch.empty((S, N), dtype=torch.bfloat16, device=dev)
                    gemm, _ = moe.moe_grouped_gemm_prepare(x, w, "bf16", routing, M, k, E, k, out=C,
                                                           stream=stream)
                    mb = routing[1].numel()
                    gemm_bytes = touched * N * K * 2 + M * K * 2 + S * N * 2
                    call_bytes = gemm_bytes + (S * 4 + mb * bm * 4 + mb * 4 + 4) + (S * N * 2 + M * N * 2 + S * 4)
                    c.update(ids=ids, tw=tw, bm=bm, routing=routing, C=C, gemm=gemm, gemm_bytes=gemm_bytes,
                             call_bytes=call_bytes)
                pair.append(c)
            lst.append(pair)
        calls[M] = lst
    flush_src = torch.ones(1 << 29, dtype=torch.uint8, device=dev)
    flush_dst = torch.empty_like(flush_src)
    spin = spin_cycles(torch, stream, SPIN_MS)
    # per step, per M: events of the fused call (2) and of the three-launch call (4)
    events = [[([torch.cuda.Event(enable_timing=True) for _ in range(2)],
                [torch.cuda.Event(enable_timing=True) for _ in range(4)]) for _ in DECODE_MS]
              for _ in range(n_steps)]
    torch.cuda.synchronize()
    timed = []  # (M, fused events, fused call, three-launch events, three-launch call)
    clock.region = "decode_cold"
    gc.collect()
    gc.disable()  # no collector pause inside a step (the spin below covers the host's queueing of it)
    with torch.cuda.stream(stream):
        for step in range(n_steps):
            # a spin at the head of each step, so that the host has queued all
            # of the step's launches before the first one runs: no host-side
            # gap falls inside an event pair
            torch.cuda._sleep(spin)
            for i, M in enumerate(DECODE_MS):
                cf, c3 = calls[M][step]
                evf, ev3 = events[step][i]
                flush_dst.copy_(flush_src)
                for dst, src in cf["srcs"]:  # the call's inputs, written just before it as their producer would
                    dst.copy_(src)
                evf[0].record(stream)
                cf["layer"]()
                evf[1].record(stream)
                flush_dst.copy_(flush_src)
                for dst, src in c3["srcs"]:
                    dst.copy_(src)
                ev3[0].record(stream)
                moe.moe_align(c3["ids"], E, c3["bm"], out=c3["routing"], stream=stream)
                ev3[1].record(stream)
                c3["gemm"]()
                ev3[2].record(stream)
                moe.moe_combine(c3["C"], c3["tw"], k, out=c3["y"], stream=stream)
                ev3[3].record(stream)
                if step >= args.warmup:
                    timed.append((M, evf, cf, ev3, c3))
            stream.synchronize()
    gc.enable()
    torch.cuda.synchronize()
    clock.region = None
    keys = ("layer", "call", "gemm", "align", "combine", "touched", "layer_frac", "gemm_frac")
    per_m = {M: {key: [] for key in keys} for M in DECODE_MS}
    tot = {"layer_bytes": 0.0, "layer_us": 0.0, "call_bytes": 0.0, "call_step_bytes": 0.0, "call_us": 0.0,
           "gemm_bytes": 0.0, "gemm_us": 0.0}
    for M, evf, cf, ev3, c3 in timed:
        layer = evf[0].elapsed_time(evf[1]) * 1e3
        call = ev3[0].elapsed_time(ev3[3]) * 1e3
        g = ev3[1].elapsed_time(ev3[2]) * 1e3
        d = per_m[M]
        d["layer"].append(layer)
        d["call"].append(call)
        d["gemm"].append(g)
        d["align"].append(ev3[0].elapsed_time(ev3[1]) * 1e3)
        d["combine"].append(ev3[2].elapsed_time(ev3[3]) * 1e3)
        d["touched"].append(cf["touched"])
        d["layer_frac"].append(cf["step_bytes"] / layer / 1e3 / PEAK_HBM_GBS)
        d["gemm_frac"].append(c3["gemm_bytes"] / g / 1e3 / PEAK_HBM_GBS)
        tot["layer_bytes"] += cf["step_bytes"]
        tot["layer_us"] += layer
        tot["call_bytes"] += c3["call_bytes"]
        tot["call_step_bytes"] += c3["step_bytes"]
        tot["call_us"] += call
        tot["gemm_bytes"] += c3["gemm_bytes"]
        tot["gemm_us"] += g
    out = {}
    for M in DECODE_MS:
        d = per_m[M]
        out[str(M)] = {"layer_us": stats(d["layer"]),
                       "layer_hbm_frac_median": round(float(np.median(d["layer_frac"])), 4),
                       "three_launch": {"call_us": stats(d["call"]), "gemm_us": stats(d["gemm"]),
                                        "align_us": stats(d["align"]), "combine_us": stats(d["combine"]),
                                        "gemm_hbm_frac_median": round(float(np.median(d["gemm_frac"])), 4)},
                       "touched_experts_mean": round(float(np.mean(d["touched"])), 1)}
    del calls, flush_src, flush_dst, w
    torch.cuda.empty_cache()
    n = len(timed)
    return {"value": tot["layer_bytes"] / (tot["layer_us"] * 1e-6) / 1e9,
            "ms_per_step": tot["layer_us"] / args.steps / 1e3, "layer_avg_us": tot["layer_us"] / n,
            "three_launch": {"GBps": round(tot["call_step_bytes"] / (tot["call_us"] * 1e-6) / 1e9, 3),
                             "GBps_with_intermediates": round(tot["call_bytes"] / (tot["call_us"] * 1e-6) / 1e9, 3),
                             "ms_per_step": round(tot["call_us"] / args.steps / 1e3, 4),
                             "gemm_GBps": round(tot["gemm_bytes"] / (tot["gemm_us"] * 1e-6) / 1e9, 3),
                             "gemm_avg_us": round(tot["gemm_us"] / n, 3)},
            "per_m": out, "calls": n}


def decode_cold_k2688(torch, moe, dev, stream, args, clock):
    """The extra decode row at the page recipe's hidden size (K = 2688, the
    Nemotron shape; E=128, N=1856, top-6, bf16), through the fused layer
    alone, with the cold-cache protocol of decode_cold: per M, median / p10 /
    p90 of the call and its fraction of 8 TB/s. 28 tokens of 2688 are the
    most whose activations the layer holds on chip at once."""
    import numpy as np
    import synth
    E, N, K, k = 128, 1856, 2688, 6
    w = synth.bf16_normal((E, N, K), 0.02, 1006, "w1", dev)
    n_steps = args.warmup + args.steps
    calls = {}
    for M in DECODE_MS:
        lst = []
        for r in range(n_steps):
            x_src = synth.bf16_normal((M, K), 1.0, 1006, f"cold-x{M}c{r}", dev)
            ids_src, tw_src = synth.softmax_topk_routing(M, E, k, 1006, f"cold-route{M}c{r}", dev)
            x, ids, tw = torch.empty_like(x_src), torch.empty_like(ids_src), torch.empty_like(tw_src)
            y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            touched = len(np.unique(ids_src.cpu().numpy()))
            layer, _ = moe.moe_decode_layer_prepare(x, ids, tw, w, "bf16", out=y, stream=stream)
            lst.append(dict(srcs=((x, x_src), (ids, ids_src), (tw, tw_src)), layer=layer, touched=touched,
                            step_bytes=touched * N * K * 2 + M * K * 2 + M * k * 8 + M * N * 2))
        calls[M] = lst
    flush_src = torch.ones(1 << 29, dtype=torch.uint8, device=dev)
    flush_dst = torch.empty_like(flush_src)
    spin = spin_cycles(torch, stream, SPIN_MS)
    events = [[[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in DECODE_MS] for _ in range(n_steps)]
    torch.cuda.synchronize()
    timed = []
    clock.region = "decode_cold_k2688"
    gc.collect()
    gc.disable()
    with torch.cuda.stream(stream):
        for step in range(n_steps):
            torch.cuda._sleep(spin)
            for i, M in enumerate(DECODE_MS):
                c = calls[M][step]
                flush_dst.copy_(flush_src)
                for dst, src in c["srcs"]:
                    dst.copy_(src)
                ev = events[step][i]
                ev[0].record(stream)
                c["layer"]()
                ev[1].record(stream)
                if step >= args.warmup:
                    timed.append((M, ev, c))
            stream.synchronize()
    gc.enable()
    torch.cuda.synchronize()
    clock.region = None
    per_m = {M: ([], []) for M in DECODE_MS}
    tot_b = tot_us = 0.0
    for M, ev, c in timed:
        us = ev[0].elapsed_time(ev[1]) * 1e3
        per_m[M][0].append(us)
        per_m[M][1].append(c["step_bytes"] / us / 1e3 / PEAK_HBM_GBS)
        tot_b += c["step_bytes"]
        tot_us += us
    del calls, flush_src, flush_dst, w
    torch.cuda.empty_cache()
    return {"workload": "decode bf16 MoE at the recipe's hidden size, E=128 N=1856 K=2688 top-6, fused layer",
            "GBps": round(tot_b / (tot_us * 1e-6) / 1e9, 3),
            "hbm_frac": round(tot_b / (tot_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            "per_m": {str(M): {"layer_us": stats(per_m[M][0]),
                               "layer_hbm_frac_median": round(float(np.median(per_m[M][1])), 4)}
                      for M in DECODE_MS}}


def measure(wl, torch, stream, args, nv, clock, region):
    """Warm measurement of a workload: K graph-replayed steps (W warmup), then
    the dominant kernel's launch durations from HIP events on its stream, one
    event pair per launch, launched back to back on resident inputs."""
    graphs = []
    with torch.cuda.stream(stream):
        for v in range(nv):
            wl.step(v)  # eager run first (warms caches of the library and allocator)
        torch.cuda.synchronize()
        for v in range(nv):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                wl.step(v)
            graphs.append(g)
    torch.cuda.synchronize()
    for i in range(args.warmup):
        graphs[i % nv].replay()
    torch.cuda.synchronize()
    clock.region = region
    t0 = time.perf_counter()
    for i in range(args.steps):
        graphs[i % nv].replay()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    step_bytes = sum(wl.step_bytes(i % nv) for i in range(args.steps))
    step_flops = sum(wl.step_flops(i % nv) for i in range(args.steps))
    per_call, durs, units_all = {}, [], []
    with torch.cuda.stream(stream):
        for i in range(args.steps):
            v = i % nv
            launches = wl.dominant_launches(v)
            for j, (fn, units) in enumerate(launches):
                fn()  # queue ahead so the timed launches run back to back
                for _ in range(args.launch_reps):
                    a = torch.cuda.Event(enable_timing=True)
                    b = torch.cuda.Event(enable_timing=True)
                    a.record(stream)
                    fn()
                    b.record(stream)
                    durs.append((a, b, units, j, v))
    torch.cuda.synchronize()
    clock.region = None
    dom_ms, dom_units = 0.0, 0.0
    us = []
    variants = []
    for a, b, units, j, v in durs:
        variants.append(v)
        t = a.elapsed_time(b)
        dom_ms += t
        dom_units += units
        us.append(t * 1e3)
        per_call.setdefault(j, []).append(t * 1e3)
    del graphs
    return dict(dt=dt, step_bytes=step_bytes, step_flops=step_flops, dom_ms=dom_ms, dom_units=dom_units,
                launch_us=us, per_call=per_call, n=len(us), launch_variant=variants)


def roofline_of(wl, m):
    if wl.bound == "hbm":
        achieved = m["dom_units"] / (m["dom_ms"] * 1e-3) / 1e9
        peak, unit = PEAK_HBM_GBS, "GB/s"
    else:
        achieved = m["dom_units"] / (m["dom_ms"] * 1e-3) / 1e12
        peak, unit = PEAK_BF16_TFLOPS, "TFLOP/s"
    return {"bound": wl.bound, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": load_traffic(wl.name, None),
            "kernel": wl.dominant, "avg_launch_us": round(m["dom_ms"] / m["n"] * 1e3, 3),
            "launch_us": stats(m["launch_us"])}


LARGE_M = ("w4a16", "mxfp8", "wgrad")


def time_second_kernel(wl, torch, stream, args, nv):
    """A workload's second GEMM timed like its dominant one: its launches
    back to back on resident inputs, one event pair each, after the step's
    earlier launches produced its input."""
    durs = []
    key = None
    with torch.cuda.stream(stream):
        for i in range(args.steps):
            v = i % nv
            wl.step(v)  # the second GEMM's input (h) for this variant
            key, launches = wl.second_launches(v)
            for fn, flops, nbytes in launches:
                fn()
                for _ in range(args.launch_reps):
                    a = torch.cuda.Event(enable_timing=True)
                    b = torch.cuda.Event(enable_timing=True)
                    a.record(stream)
                    fn()
                    b.record(stream)
                    durs.append((a, b, flops, nbytes))
    torch.cuda.synchronize()
    us = [a.elapsed_time(b) * 1e3 for a, b, _, _ in durs]
    secs = sum(us) * 1e-6
    flops = sum(f for _, _, f, _ in durs)
    nbytes = sum(n for _, _, _, n in durs)
    return {key: {"launch_us": stats(us), "tflops": round(flops / secs / 1e12, 1),
                  "bf16_peak_frac": round(flops / secs / 1e12 / PEAK_BF16_TFLOPS, 4),
                  "hbm_GBps": round(nbytes / secs / 1e9, 1),
                  **attainable(flops, nbytes, flops / secs / 1e12)}}


def library_dense(torch, dev, stream, shapes, reps=10):
    """A reference, not part of the path: the library's dense bf16 GEMM
    (torch.matmul, i.e. hipBLASLt) on dense operands of the same product
    sizes (C[M, N] = A[M, K] B[N, K]^T), timed with one event pair per launch
    after warmup: the MFMA rate this machine sustains on a plain GEMM of that
    size. Returns its TFLOP/s over all shapes and the median launch time of
    each distinct shape."""
    flops, secs, per_shape = 0, 0.0, {}
    with torch.cuda.stream(stream):
        for (M, N, K) in shapes:
            key = f"{M}x{N}x{K}"
            if key not in per_shape:
                a = torch.randn(M, K, device=dev, dtype=torch.bfloat16)
                b = torch.randn(N, K, device=dev, dtype=torch.bfloat16)
                for _ in range(3):
                    torch.matmul(a, b.t())
                ev = []
                for _ in range(reps):
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    torch.matmul(a, b.t())
                    e1.record(stream)
                    ev.append((e0, e1))
                torch.cuda.synchronize()
                ts = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
                per_shape[key] = ts[len(ts) // 2]
                del a, b
            flops += 2 * M * N * K
            secs += per_shape[key] * 1e-3
    torch.cuda.empty_cache()
    return {"tflops": round(flops / secs / 1e12, 1), "median_ms": {k: round(v, 4) for k, v in per_shape.items()}}


def attainable(flops, nbytes, tflops, peak_tflops=PEAK_BF16_TFLOPS):
    """Arithmetic intensity (flop/B of the algorithmic work) and the fraction
    of the attainable roofline min(MFMA peak of the dtype, AI x HBM peak)
    reached."""
    ai = flops / nbytes
    roof = min(peak_tflops, ai * PEAK_HBM_GBS / 1e3)
    return {"arith_intensity": round(ai, 1), "attainable_tflops": round(roof, 1),
            "attainable_frac": round(tflops / roof, 4)}


def large_m_block(torch, dev, stream, args, clock):
    """The large-M half of the metric: per workload, the dominant kernel's
    TFLOP/s and fractions of the bf16 MFMA peak and of HBM bandwidth (sums
    of algorithmic flops and bytes over sums of launch times; the launch
    times' median, p10 and p90 beside them) and the whole step's TFLOP/s."""
    out = {}
    for name in LARGE_M:
        wl = WORKLOADS[name](torch, dev, args.variants)
        nv = len(wl.calls) if name == "w4a16" else 1
        m = measure(wl, torch, stream, args, nv, clock, f"large_m_{name}")
        roof = roofline_of(wl, m)
        flops = sum(wl.dominant_flops_bytes(v)[0] for v in m["launch_variant"])
        nbytes = sum(wl.dominant_flops_bytes(v)[1] for v in m["launch_variant"])
        secs = m["dom_ms"] * 1e-3
        out[name] = {
            "workload": CONFIG_NAMES[name], "kernel": wl.dominant, "launch_us": roof["launch_us"],
            "tflops": round(flops / secs / 1e12, 1),
            "bf16_peak_frac": round(flops / secs / 1e12 / PEAK_BF16_TFLOPS, 4),
            "hbm_GBps": round(nbytes / secs / 1e9, 1),
            "hbm_frac": round(nbytes / secs / 1e9 / PEAK_HBM_GBS, 4),
            **attainable(flops, nbytes, flops / secs / 1e12),
            "roofline": {k: roof[k] for k in ("bound", "achieved", "peak", "unit", "frac", "traffic")},
            "step_tflops": round(m["step_flops"] / m["dt"] / 1e12, 1),
            "ms_per_step": round(m["dt"] / args.steps * 1e3, 4),
            "clock": clock.summary(f"large_m_{name}"),
        }
        out[name].update(wl.extra(None))
        if hasattr(wl, "second_launches"):
            out[name].update(time_second_kernel(wl, torch, stream, args, nv))
        if hasattr(wl, "dense_shapes"):
            # the same products as one dense bf16 library GEMM each (variants
            # weighted as the timed launches cycle through them)
            ref = {}
            for part in wl.dense_shapes(0):
                lib = library_dense(torch, dev, stream, [wl.dense_shapes(v)[part] for v in range(nv)])
                ours = out[name]["tflops"] if part in ("up", "gemm") else out[name][part]["tflops"]
                ref[part] = dict(lib, kernel_frac=round(ours / lib["tflops"], 3))
            out[name]["library_dense_bf16"] = dict(ref, note=(
                "reference only: torch.matmul (hipBLASLt) on dense bf16 operands of the same product "
                "sizes; kernel_frac = this kernel's TFLOP/s over the library's"))
        del wl, m
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.counters_from:
        record_counters(args.counters_key or args.workload, args.counters_from)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: the library has no multi-GPU path "
                                   "(--gpus must be 1)"}))
        sys.exit(2)
    import torch
    import mixture_experts_grouped_moe_amd as moe  # noqa: F401  (fails loudly if libmoe.so is missing)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.layout != "auto":
        for name in LAYOUT:
            LAYOUT[name] = args.layout
    clock = ClockSampler(torch)
    stream = torch.cuda.Stream()
    if args.workload == "decode":
        line = decode_main(torch, moe, dev, stream, args, clock)
    else:
        line = workload_main(torch, dev, stream, args, clock)
    clock.close()
    print(json.dumps(line), flush=True)


def decode_main(torch, moe, dev, stream, args, clock):
    """The headline: the decode workload with a cold cache (value, roofline),
    its warm figures under "warm", and the large-M block."""
    cold = decode_cold(torch, moe, dev, stream, args, clock) if args.phase in ("cold", "both") else None
    warm = None
    wl = None
    if args.phase in ("warm", "both") or cold is None:
        wl = Decode(torch, dev, args.variants)
        nv = len(wl.calls)
        m = measure(wl, torch, stream, args, nv, clock, "decode_warm")
        roof = roofline_of(wl, m)
        per_call = [sum(v) / len(v) for _, v in sorted(m["per_call"].items())]
        warm = {"value": round(m["step_bytes"] / m["dt"] / 1e9, 3), "unit": "GB/s",
                "ms_per_step": round(m["dt"] / args.steps * 1e3, 4), "routing_variants": nv,
                "roofline": roof, "launch_reps": args.launch_reps, "clock": clock.summary("decode_warm")}
        warm.update(wl.extra(per_call))
        wf = DecodeFused(torch, dev, args.variants)
        m = measure(wf, torch, stream, args, nv, clock, "decode_warm_fused")
        per_call = [sum(v) / len(v) for _, v in sorted(m["per_call"].items())]
        warm_fused = {"value": round(m["step_bytes"] / m["dt"] / 1e9, 3), "unit": "GB/s",
                      "ms_per_step": round(m["dt"] / args.steps * 1e3, 4), "roofline": roofline_of(wf, m),
                      "clock": clock.summary("decode_warm_fused")}
        warm_fused.update(wf.extra(per_call))
        warm = {"fused_layer": warm_fused, "three_launch": warm}
        del wf, m
        torch.cuda.empty_cache()
    if cold is not None:
        # the fused layer is the step's one launch: its roofline is the step's
        roof_cold = {"bound": "hbm", "achieved": round(cold["value"], 3), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(cold["value"] / PEAK_HBM_GBS, 4), "traffic": load_traffic("decode_layer", None),
                     "kernel": DECODE_LAYER_KERNEL, "avg_launch_us": round(cold["layer_avg_us"], 3),
                     "cache": "cold (1 GiB copy between calls)"}
        value, ms = cold["value"], cold["ms_per_step"]
        roofline = roof_cold
    else:
        wfl = warm["fused_layer"]
        value, ms, roofline = wfl["value"], wfl["ms_per_step"], wfl["roofline"]
    cpu = None
    if not args.no_cpu_baseline:
        if wl is None:
            wl = Decode(torch, dev, 1)
        cpu = cpu_baseline(wl, args.cpu_seconds)
    line = {"metric": METRIC, "value": round(value, 3), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": CONFIG_NAMES["decode"],
                       "path": "moe_decode_layer: routing, grouped GEMM and top-k combine in one launch",
                       "cache": "cold: every call on its own routing, after a 1 GiB copy that evicts the MALL",
                       "weight_layout": LAYOUT["decode"], "parallelism": "single GPU"},
            "roofline": roofline, "cpu_baseline": cpu}
    if cold is not None:
        line["hbm_frac_step"] = round(value / PEAK_HBM_GBS, 4)
        three = dict(cold["three_launch"])
        three["gemm_roofline"] = {"bound": "hbm", "achieved": three["gemm_GBps"], "peak": PEAK_HBM_GBS,
                                  "unit": "GB/s", "frac": round(three["gemm_GBps"] / PEAK_HBM_GBS, 4),
                                  "traffic": load_traffic("decode", None), "kernel": "moe_decode_kernel"}
        if args.phase == "both":  # (the profiled --phase cold runs time the headline's launches only)
            line["cold_k2688"] = decode_cold_k2688(torch, moe, dev, stream, args, clock)
        line["cold"] = {"per_m": cold["per_m"], "calls_per_path": cold["calls"],
                        "three_launch": three,
                        "clock": dict(clock.summary("decode_cold"), note=(
                            "sampled every 10 ms over the whole cold region, most of whose time is the "
                            "20 ms one-wave spin heading each step, so it describes the region, not the "
                            "calls (it has read 190 to 2020 MHz on different runs); the calls run right "
                            "after 1 GiB copies, and 8 more copies ahead of each step's first call moved "
                            "no per-M median by more than 1.5%")),
                        "ms_per_step_note": "device time of the step's launches (events); the copies that "
                                            "evict the cache between calls are outside it",
                        "bytes_note": "value counts the bytes the step must move (touched experts' weights, "
                                      "activations, ids and routing weights in, y out); the three-launch "
                                      "path also moves C and the routing buffers "
                                      "(GBps_with_intermediates counts them)"}
    if warm is not None:
        line["warm"] = warm
    if not args.no_large_m and args.phase == "both":
        del wl
        torch.cuda.empty_cache()
        line["large_m"] = large_m_block(torch, dev, stream, args, clock)
    return line


def workload_main(torch, dev, stream, args, clock):
    """One workload chosen with --workload (warm, graph-replayed steps)."""
    wl = WORKLOADS[args.workload](torch, dev, args.variants)
    nv = len(getattr(wl, "calls", [None])) if args.workload in ("nemotron", "w4a16") else 1
    m = measure(wl, torch, stream, args, nv, clock, "workload")
    roofline = roofline_of(wl, m)
    dt = m["dt"]
    if args.workload in ("nemotron", "copy"):
        value = m["step_bytes"] / dt / 1e9
        unit_v = "GB/s"
        extra = wl.extra([sum(v) / len(v) for _, v in sorted(m["per_call"].items())])
        extra["hbm_frac_step"] = round(value / PEAK_HBM_GBS, 4)
        dtype = "u8" if args.workload == "copy" else "bf16"
    else:
        value = m["step_flops"] / dt / 1e12
        unit_v = "TFLOP/s"
        extra = wl.extra(None)
        extra["mfma_frac_step_bf16"] = round(value / PEAK_BF16_TFLOPS, 4)
        if args.workload in ("mxfp8a", "pertoken"):
            extra["mfma_frac_step_fp8"] = round(value / (2 * PEAK_BF16_TFLOPS), 4)
        extra["hbm_GBps_step"] = round(m["step_bytes"] / dt / 1e9, 1)
        if hasattr(wl, "dominant_flops_bytes"):
            # the dominant kernel against min(its dtype's MFMA peak, AI x HBM peak)
            fl = sum(wl.dominant_flops_bytes(v)[0] for v in m["launch_variant"])
            nb = sum(wl.dominant_flops_bytes(v)[1] for v in m["launch_variant"])
            peak = 2 * PEAK_BF16_TFLOPS if args.workload in ("mxfp8a", "pertoken") else PEAK_BF16_TFLOPS
            extra["kernel_roofline"] = attainable(fl, nb, fl / (m["dom_ms"] * 1e-3) / 1e12, peak)
        dtype = {"w4a16": "bf16 x e2m1 (bf16 MFMA)", "mxfp8": "bf16 x e4m3 (bf16 MFMA)",
                 "mxfp8a": "e4m3 x e4m3, E8M0 per 32 (scaled fp8 MFMA)",
                 "pertoken": "e4m3 x e4m3, fp32 per-row and per-expert scales (fp8 MFMA)",
                 "wgrad": "bf16 (bf16 MFMA, fp32 out)"}[args.workload]
    cpu = None if args.no_cpu_baseline else cpu_baseline(wl, args.cpu_seconds)
    line = {"metric": METRIC, "value": round(value, 3), "unit": unit_v, "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(dt / args.steps * 1e3, 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": dtype, "data": "synthetic",
            "config": {"workload": CONFIG_NAMES[args.workload], "routing_variants": nv,
                       "weight_layout": LAYOUT.get(args.workload, "n/a"), "parallelism": "single GPU"},
            "roofline": roofline, "cpu_baseline": cpu, "clock": clock.summary("workload")}
    line.update(extra)
    return line


if __name__ == "__main__":
    main()
