"""Properties of the generated gfx950 device code (CPU only: hipcc cross-compiles).

- M0: the direct global -> LDS copies are inline assembly that sets M0 (the LDS destination of
  the copy) and declares it clobbered.  The compiler treats M0 as reserved and does not promise to
  keep its own values in M0 across such a statement, so the copies are only correct while the
  compiler places nothing of its own in M0.  Every M0 reference in the device code must therefore
  be the copies' own write, inside their asm block and followed there by the copy that reads it.
- Packed float32 arithmetic is disabled for all device code by the build flags; no packed float32
  add, multiply or FMA may appear in the generated code.
"""
import concurrent.futures as cf
import glob
import os
import re
import subprocess

import pytest

from long_context_exact_attn_amd import build as B

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "long_context_exact_attn_amd", "csrc")


def _have_hipcc():
    try:
        B.hipcc()
    except RuntimeError:
        return False
    return True


pytestmark = pytest.mark.skipif(not _have_hipcc(), reason="hipcc is required")


@pytest.fixture(scope="module")
def device_asm(tmp_path_factory):
    out = tmp_path_factory.mktemp("asm")
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))

    def one(src):
        dst = os.path.join(out, os.path.basename(src) + ".s")
        cmd = [B.hipcc(), *B.common_flags(), "--cuda-device-only", "-S", src, "-o", dst]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return os.path.basename(src), open(dst).read().splitlines()

    with cf.ThreadPoolExecutor(min(8, len(sources))) as ex:
        return dict(ex.map(one, sources))


M0 = re.compile(r"\bm0\b")


def test_m0_written_only_by_the_copies(device_asm):
    copies = 0
    for name, lines in device_asm.items():
        in_asm = False
        block = []
        for ln in lines:
            s = ln.split(";")[0].strip()
            if ln.strip().startswith(";;#ASMSTART"):
                in_asm, block = True, []
                continue
            if ln.strip().startswith(";;#ASMEND"):
                writes = [i for i, x in enumerate(block) if M0.search(x)]
                for i in writes:
                    # the "s" operand may be any scalar register, vcc_lo / vcc_hi included
                    assert re.fullmatch(r"s_mov_b32 m0, (s\d+|vcc_lo|vcc_hi)", block[i]), (name, block)
                    assert any(x.startswith("global_load_lds_dwordx4") for x in block[i + 1:]), (name, block)
                    copies += 1
                in_asm = False
                continue
            if not s:
                continue
            if in_asm:
                block.append(s)
            else:
                assert not M0.search(s), f"{name}: compiler-generated M0 use: {s}"
    assert copies > 0, "no direct copies found: the test no longer looks at the right code"


def test_no_packed_fp32_arithmetic(device_asm):
    pat = re.compile(r"\bv_pk_(add|mul|fma)_f32\b")
    for name, lines in device_asm.items():
        bad = [ln.strip() for ln in lines if pat.search(ln.split(";")[0])]
        assert not bad, f"{name}: {bad[:3]}"
