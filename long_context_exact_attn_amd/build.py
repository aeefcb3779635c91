"""Build libra_attn.so (gfx950) in-tree with hipcc.

Every HIP source under csrc/ is compiled to an object in _build/ and the
objects are linked into long_context_exact_attn_amd/libra_attn.so.  The
issue-rate microbenchmark (microbench/rates.hip) is built as a standalone
program next to its source.  Packed fp32 VALU instructions are disabled for
all device code.
"""
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libra_attn.so")
ARCH = "gfx950"


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found (ROCm is required to build libra_attn)")
    return exe


def common_flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
            "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-Wno-unused-command-line-argument"]


def _compile(src, verbose):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *common_flags(), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the device-only feature flag; keep other output
    noise = [ln for ln in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n" + "\n".join(noise))
    if verbose and noise:
        print("\n".join(noise), file=sys.stderr)
    return obj


MICROBENCH = os.path.join(PKG, "microbench", "rates.hip")


def build_microbench():
    """Compile the issue-rate microbenchmark into microbench/rates; returns its path."""
    exe = os.path.splitext(MICROBENCH)[0]
    cmd = [hipcc(), *[f for f in common_flags() if f != "-fPIC"], MICROBENCH, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"microbenchmark build failed: {' '.join(cmd)}\n{r.stdout}{r.stderr}")
    return exe


def build(verbose=False, jobs=None):
    """Compile every csrc/*.hip and link libra_attn.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not sources:
        raise RuntimeError("no HIP sources found")
    jobs = jobs or min(len(sources), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), sources))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
