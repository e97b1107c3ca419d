"""Float64 CPU oracle for the routed, block-scaled MoE expert-layer path.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
link this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the HIP
library and imports nothing from it; it imports numpy and the standard
library only.

Every function is the plain definition of what the method computes, written
in float64 (the pages fix no precision for a reference), with no blocking,
fusion or reordering beyond the definition. Each function's docstring names
the passage of the pages it follows and the test that pins it to something
other than itself:

    formats.e8m0_to_f64     pinned  (all 256 codes vs a library decoder; printed edge values)
    formats.e4m3_to_f64     pinned  (all 256 codes vs a library decoder)
    formats.e2m1_to_f64     pinned  (the 16-entry table of the OCP MX format)
    formats.bf16_to_f64     pinned  (all 65536 codes vs a library decoder)
    bucket.bucket_round_up  pinned  (exhaustive properties on [1, 65536]; printed bucket count)
    bucket.bucket_enumerate pinned  (closure, sortedness, printed count)
    align.moe_align         pinned  (brute force on tiny inputs, invariants, hand-worked example)
    gemm.dequant_expert     pinned  (constant-input closed form, Fraction brute force)
    gemm.grouped_gemm       pinned  (constant input, bias, linearity, Fraction brute force)
    gemm.dequant_act        pinned  (MXFP8 activations, a_scale by token row: constant input
                                     with per-row and per-block scales, Fraction brute
                                     force at a_row_div 1 and top_k, one scale row per token)
    gemm.silu / swiglu      pinned  (closed forms and the odd-part identity)
    gemm.relu2              pinned  (closed forms; constant-input GEMM epilogue)
    gemm.build_block_mapping pinned (hand-worked example; every row in exactly one block)
    gemm.grouped_gemm_per_token pinned (constant input with bias, scalar loop, empty groups)
    gemm.combine            pinned  (identity at k = 1, hand-worked example, linearity)
    wgrad.wgrad             pinned  (constant input, linearity, zero/PAD slots, Fraction brute force)
    layer.w4a16_layer       pinned  (composition of pinned functions; padded == unpadded)
    layer.relu2_layer       pinned  (composition of pinned functions; constant-input closed form)
    layout.pack_kblock      pinned  (per-element loop over the layout's index formula)
    quant.mx_quantize_e4m3  pinned  (every code round-trips at a known shared exponent;
                                     scale rule, ties, saturation, zero and clamped
                                     blocks; torch's float8_e4m3fn cast in range)
"""

from . import formats, bucket, align, gemm, wgrad, layer, layout, quant  # noqa: F401

__all__ = ["formats", "bucket", "align", "gemm", "wgrad", "layer", "layout", "quant"]
