"""The device code compiles for gfx950 without inline-asm warnings.

The LDS copy asm takes its LDS address as an M0 input operand; an asm block
that wrote M0 itself and listed it as clobbered would be silently ignored by
the compiler (M0 is reserved) and warn.  Compiling the kernels here with the
product's flags and no GPU keeps that from coming back, and checks that the
bf16 kernel still fits three work-groups per CU and the fp32 kernel two,
without scratch.
"""

import os
import re
import shutil
import subprocess

import pytest

from ring_blockwise_softmax_amd import build as B


def _hipcc():
    try:
        return B.hipcc()
    except RuntimeError:
        return None


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
def test_kernels_compile_without_inline_asm_warnings(tmp_path):
    src = os.path.join(B.CSRC, "ra_kernels.hip")
    out = tmp_path / "ra_kernels.s"
    cmd = [_hipcc(), *B.COMMON, *B.DEVICE, "--cuda-device-only", "-S", src, "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    bad = [l for l in res.stderr.splitlines() if "inline-asm" in l or "inline asm" in l or "m0" in l.lower()]
    assert not bad, "\n".join(bad[:10])
    asm = out.read_text()

    def resources(name):
        start = asm.index(name + ":")
        meta = asm[asm.index(".Lfunc_end", start):][:4000]
        return tuple(int(re.search(r"; %s: (\d+)" % key, meta).group(1))
                     for key in ("NumVgprs", "NumAgprs", "ScratchSize", "Occupancy"))

    vgprs, _, scratch, occ = resources("_ZN2ra13attn_fwd_bf16ILi128ELb0ELb0EEEvNS_8AttnArgsE")
    assert scratch == 0 and occ >= 3 and vgprs <= 168, (vgprs, scratch, occ)
    # the fp32 exact path: two waves per SIMD (two work-groups per CU)
    for d in (128, 64):
        vgprs, agprs, scratch, occ = resources("_ZN2ra12attn_fwd_f32ILi%dEEEvNS_8AttnArgsE" % d)
        assert scratch == 0 and occ >= 2 and vgprs + agprs <= 256, (d, vgprs, agprs, scratch, occ)
