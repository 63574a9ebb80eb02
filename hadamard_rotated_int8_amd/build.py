"""Ahead-of-time build of libsdnq_hip.so for gfx950 (hipcc, in-tree).

Every translation unit is compiled with:
  * --offload-arch=gfx950 only (CDNA4; no other target, no host fallback);
  * -ffp-contract=off: the rotation and quantization must be evaluated exactly
    as written (no fused multiply-add contraction), so their int8 codes and fp32
    scales are reproducible bit for bit;
  * -Xclang -target-feature -Xclang -packed-fp32-ops: no packed fp32 VALU
    instructions are generated.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libsdnq_hip.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

DEVICE_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


# Per-file device flags.  attn.hip: keep MFMA accumulators in ordinary VGPRs.  Its
# online softmax rescales the output accumulators with VALU multiplies, which
# cost an accumulator-register read and write around each multiply otherwise.
FILE_FLAGS = {"attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _compile(src: str, extra: list[str]) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *DEVICE_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 target feature and says so.
    noise = ("packed-fp32-ops", "unknown target feature", "warning generated", "warnings generated")
    lines = [ln for ln in (r.stdout + r.stderr).splitlines() if ln.strip() and not any(n in ln for n in noise)]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(lines))
    if lines:
        sys.stderr.write("\n".join(lines) + "\n")
    return obj


def build(extra: list[str] | None = None, verbose: bool = False) -> str:
    """Compile every csrc/*.hip for gfx950 and link the shared library in place."""
    extra = list(extra or [])
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), srcs))
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build(sys.argv[1:], verbose=True)
