"""The LDS-DMA helpers set m0 (the LDS destination of `buffer_load ... lds`)
inside inline asm. The compiler reserves m0 and does not honour it as an asm
clobber, so this is safe only while no compiler-generated instruction uses
m0: compile every kernel source for gfx950 and check that each m0 in the
assembly is a helper's `s_mov_b32 m0, sN` directly followed by its LDS DMA."""

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mixture_experts_grouped_moe_amd", "csrc")
HIPCC = next((c for c in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")) if c and os.path.exists(c)), None)


def _asm(src, tmp):
    out = os.path.join(tmp, src + ".s")
    cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", "-x", "hip",
           "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", out]
    subprocess.run(cmd, check=True, capture_output=True)
    return [l.split(";")[0].strip() for l in open(out)]


@pytest.mark.skipif(HIPCC is None, reason="hipcc not available")
def test_m0_is_only_written_by_the_lds_dma_helpers(tmp_path):
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    with ThreadPoolExecutor(max_workers=4) as ex:
        listings = dict(zip(srcs, ex.map(lambda s: _asm(s, str(tmp_path)), srcs)))
    dma_seen = 0
    for src, lines in listings.items():
        for i, l in enumerate(lines):
            if "m0" not in l.replace(",", " ").split() and not l.startswith("s_mov_b32 m0,"):
                continue
            nxt = lines[i + 1] if i + 1 < len(lines) else ""
            assert l.startswith("s_mov_b32 m0, s") and nxt.startswith("buffer_load") and nxt.endswith(" lds"), \
                f"{src}: m0 used outside an LDS-DMA helper: {l!r} then {nxt!r}"
            dma_seen += 1
    assert dma_seen > 0
