"""Build libspecverify.so (HIP for gfx950) in-tree.

Every .hip file under csrc/ is compiled with hipcc for gfx950 into
_build/, then linked into target_verification_amd/libspecverify.so.  Packed
FP32 instructions are disabled for all device code.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libspecverify.so")
BUILD = os.path.join(os.path.dirname(HERE), "_build")
ARCH = os.environ.get("SV_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-result", "-Wno-unused-function"]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src, build_dir=BUILD, defines=()):
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *[f"-D{d}" for d in defines], "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{errs}")
    return obj, errs


def build(verbose: bool = False, jobs: int = 8, defines=(), out: str = OUT,
          build_dir: str = BUILD) -> str:
    """Compile and link the library; `defines` (e.g. ("SV_TIMELINE",)) make
    a measurement build, linked to `out` from objects in `build_dir`."""
    os.makedirs(build_dir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(lambda src: _compile(src, build_dir, defines), sources()))
    if verbose:
        for obj, errs in results:
            if errs:
                print(f"[{os.path.basename(obj)}]\n{errs}", file=sys.stderr)
    objs = [o for o, _ in results]
    tmp = out + ".tmp"
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-Wl,--no-undefined", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
