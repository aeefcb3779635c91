"""Build libra_attn.so (gfx950) in-tree with hipcc.

Every HIP source under csrc/ is compiled to an object in _build/ and the
objects are linked into long_context_exact_attn_amd/libra_attn.so.  The
issue-rate microbenchmark (microbench/rates.hip) is built as a standalone
program next to its source.  The library links the roctx marker library of
ROCm's profiler SDK (one named range per entry-point call).  Packed fp32
VALU instructions are disabled for all device code.
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


def rocm_lib():
    return os.path.normpath(os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "lib"))


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
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-L", rocm_lib(), "-lrocprofiler-sdk-roctx",
           "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


# ---------------------------------------------------------------- host-sanitized build
# The C-ABI layer (argument validation, workspace sizing, the static-scratch lookup) with its host code
# under AddressSanitizer and UndefinedBehaviorSanitizer, linked with the ordinary kernel objects into a
# second library.  Device code is never instrumented: every sanitizer flag is scoped to the host pass.
SAN_BUILD = os.path.join(PKG, "_build_san")
SAN_LIB = os.path.join(PKG, "libra_attn_san.so")
SANITIZED = ("ra_api.hip", "noalloc.hip")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def _clang():
    exe = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm", "bin", "clang++")
    exe = os.path.normpath(exe)
    return exe if os.path.exists(exe) else "/opt/rocm/llvm/bin/clang++"


def asan_runtime():
    """Path of the shared AddressSanitizer runtime a host program must preload to load SAN_LIB."""
    r = subprocess.run([_clang(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("AddressSanitizer runtime not found next to the ROCm clang")
    return path


def build_sanitized(verbose=False):
    """Link libra_attn_san.so: SANITIZED compiled with host sanitizers, every other source as in build()
    (built first when its objects are missing or older than their sources).  Returns the library path."""
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    headers = glob.glob(os.path.join(CSRC, "*.cuh")) + [os.path.join(ROOT, "include", "ra_attn.h")]
    newest_header = max(os.path.getmtime(h) for h in headers)
    plain = [s for s in sources if os.path.basename(s) not in SANITIZED]

    def stale(obj, src):
        return not os.path.exists(obj) or os.path.getmtime(obj) < max(os.path.getmtime(src), newest_header)

    objs = [os.path.join(BUILD, os.path.basename(s) + ".o") for s in plain]
    if any(stale(o, s) for o, s in zip(objs, plain)):
        build(verbose)
    os.makedirs(SAN_BUILD, exist_ok=True)
    for name in SANITIZED:
        src = os.path.join(CSRC, name)
        obj = os.path.join(SAN_BUILD, name + ".o")
        cmd = [hipcc(), *common_flags(), *SAN_FLAGS, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"sanitized compile failed: {' '.join(cmd)}\n{r.stdout}{r.stderr}")
        objs.append(obj)
    tmp = SAN_LIB + ".tmp"
    cmd = [_clang(), "-shared", "-fPIC", "-fsanitize=address,undefined", "-shared-libasan", *objs,
           "-L", rocm_lib(), "-lamdhip64", "-lrocprofiler-sdk-roctx", "-Wl,-rpath," + rocm_lib(), "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized link failed: {' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


if __name__ == "__main__":
    if "--sanitized" in sys.argv:
        print(build_sanitized(verbose=True))
    else:
        print(build(verbose=True))
