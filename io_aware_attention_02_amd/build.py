"""Build libfa.so (the C-ABI attention library) for gfx950 with hipcc, in-tree.

    python -m io_aware_attention_02_amd.build

Each source is compiled to an object under ``_build/`` (in parallel), then linked into
``io_aware_attention_02_amd/libfa.so``.  The library is always rebuilt from source.
"""

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
OUT = os.path.join(HERE, "libfa.so")
ARCH = "gfx950"

# Packed fp32 VALU ops are disabled for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Wall", "-Wno-unused-function"]
# Per-source extras.  The backward kernels run one wave per SIMD with more than 256 live
# registers; keeping every MFMA accumulator in architectural VGPRs (the extra registers then
# serve as cheap spill space) avoids copying score tiles out of accumulation registers.
PER_FILE = {"fa_bwd_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def _compile(src, hipcc, verbose):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    extra = PER_FILE.get(os.path.basename(src), [])
    cmd = [hipcc, *COMMON, *DEVICE_FLAGS, *extra, *lang, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines()
            if "not a recognized feature for this target" not in ln]
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), file=sys.stderr)
    return obj


def build_library(verbose=False):
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    if os.path.exists(OUT):  # a failed build must not leave an older library behind
        os.remove(OUT)
    srcs = sources()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, hipcc, verbose), srcs))
    tmp = OUT + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build_library(verbose=True))
