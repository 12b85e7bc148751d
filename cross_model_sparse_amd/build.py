"""Builds libmapflow.so in-tree with hipcc for gfx950.

    python -m cross_model_sparse_amd.build          # or: build() from Python
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
INCLUDE = ROOT / "include"
LIB = PKG / "libmapflow.so"
OBJ_DIR = PKG / "_build"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# No fast-math: fp16 subnormals and IEEE rounding matter for parity.  Packed
# fp32 instructions are disabled for all device code.
DEVICE_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


# Per-source additions.  The Q/K score kernels consume MFMA results with
# vector ALU code right away: results in ordinary VGPRs save a copy out of the
# accumulation registers for every score tile.
EXTRA_FLAGS = {
    "k_qk.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _compile(src: Path) -> Path:
    obj = OBJ_DIR / (src.stem + ".o")
    cmd = [HIPCC, *DEVICE_FLAGS, *EXTRA_FLAGS.get(src.name, []), "-c", str(src), "-o", str(obj)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src.name}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> Path:
    """Compiles every HIP source under csrc/ and links libmapflow.so."""
    if not Path(HIPCC).exists():
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    OBJ_DIR.mkdir(exist_ok=True)
    srcs = sorted(CSRC.glob("*.hip"))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB.with_suffix(".so.tmp")
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *map(str, objs),
           "-o", str(tmp)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def clean() -> None:
    shutil.rmtree(OBJ_DIR, ignore_errors=True)
    LIB.unlink(missing_ok=True)


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
