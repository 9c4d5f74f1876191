"""Build libmsa_nvfp4.so (HIP, gfx950) in-tree with hipcc.

    python -m nvfp4_kv_cache_amd.build              # the library
    python -m nvfp4_kv_cache_amd.build --sanitize   # host-sanitized copy for the host tests

Every HIP source under csrc/ is compiled for gfx950 with packed-FP32
instructions disabled, then linked into one shared library next to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmsa_nvfp4.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


# per-source extra flags: the scan's ReLU and maxima and the insertion's
# clamps and maxima need no IEEE NaN quieting (the inputs are finite by
# contract), which saves one VALU op each
_NO_NAN = ["-mno-amdgpu-ieee", "-fno-honor-nans"]
EXTRA = {"indexer.hip": _NO_NAN, "insert.hip": _NO_NAN}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str, out_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(out_dir, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(os.path.basename(src), []), *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


# Host-side AddressSanitizer and UndefinedBehaviorSanitizer for the C shim
# (argument checks, group derivation, launch set-up); the device code is
# built as usual. Each -fsanitize= applies to the host compilation only.
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]
SAN_BUILD = os.path.join(PKG, "_build_sanitize")
SAN_LIB = os.path.join(SAN_BUILD, "libmsa_nvfp4_sanitize.so")


def build(verbose: bool = True, sanitize: bool = False) -> str:
    out_dir = SAN_BUILD if sanitize else BUILD
    out_lib = SAN_LIB if sanitize else LIB
    os.makedirs(out_dir, exist_ok=True)
    srcs = sources()
    extra = SANITIZE if sanitize else []

    def comp(src):
        return _compile(src, out_dir, extra)
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(comp, srcs))
    tmp = out_lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out_lib)
    if verbose:
        print(f"built {out_lib} from {len(srcs)} sources for {ARCH}")
    return out_lib


if __name__ == "__main__":
    build(sanitize="--sanitize" in sys.argv)
    sys.exit(0)
