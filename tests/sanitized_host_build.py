"""A libmapflow whose host code is built with AddressSanitizer and
UndefinedBehaviorSanitizer (test infrastructure, CPU only).

The host-side logic of the library -- the argument checks of every entry
point, the workspace arithmetic, the per-device scratch bookkeeping
(mapflow_api.hip) and the Block Manager's hash table, LRU list and page pool
(block_manager.hip) -- is compiled at -O1 with both sanitizers on the host
pass only; device code is never instrumented.  The kernel translation units
are linked in as the ordinary build made them, so the library exports the
same symbols as libmapflow.so and every host test can run against it by
pointing MAPFLOW_LIB at it and preloading the ASan runtime.

    python tests/sanitized_host_build.py OUT_DIR
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from pathlib import Path

ROOT = Path(__file__).resolve().parents[1]
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))

from cross_model_sparse_amd import build as B  # noqa: E402

HOST_SOURCES = ("mapflow_api.hip", "block_manager.hip")
# Each sanitizer option applies to the host compilation pass only.
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime() -> str:
    """Path of the shared ASan runtime of the ROCm clang (LD_PRELOAD target:
    python itself is not instrumented, so the runtime must load first)."""
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("no libclang_rt.asan-x86_64.so under /opt/rocm/lib/llvm")
    return hits[-1]


def _kernel_objects() -> list[Path]:
    srcs = [s for s in sorted(B.CSRC.glob("*.hip")) if s.name not in HOST_SOURCES]
    objs = [B.OBJ_DIR / (s.stem + ".o") for s in srcs]
    stale = [s for s, o in zip(srcs, objs)
             if not o.exists() or o.stat().st_mtime < max(
                 s.stat().st_mtime, *(h.stat().st_mtime for h in B.CSRC.glob("*.h")),
                 (B.INCLUDE / "mapflow.h").stat().st_mtime)]
    if stale:
        B.OBJ_DIR.mkdir(exist_ok=True)
        for s in stale:
            B._compile(s)
    return objs


def build(out_dir: Path) -> Path:
    """Builds OUT_DIR/libmapflow.so with sanitized host code; returns its path."""
    out_dir = Path(out_dir)
    out_dir.mkdir(parents=True, exist_ok=True)
    flags = [f for f in B.DEVICE_FLAGS if f != "-O3"] + ["-O1", "-g"]
    host_objs = []
    for name in HOST_SOURCES:
        obj = out_dir / (Path(name).stem + ".san.o")
        cmd = [B.HIPCC, *flags, *SAN, "-c", str(B.CSRC / name), "-o", str(obj)]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"sanitized compile of {name} failed:\n{r.stderr}")
        host_objs.append(obj)
    lib = out_dir / "libmapflow.so"
    cmd = [B.HIPCC, f"--offload-arch={B.ARCH}", "-shared", "-fPIC",
           *map(str, _kernel_objects()), *map(str, host_objs),
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-shared-libsan",
           # lets a C program that links this library find the runtime too
           f"-Wl,-rpath,{Path(asan_runtime()).parent}", "-o", str(lib)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized link failed:\n{r.stderr}")
    return lib


def env_for(lib: Path) -> dict:
    """Environment that runs python against the sanitized library: any ASan
    report or UBSan finding ends the process with a nonzero status."""
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": asan_runtime(),
        "MAPFLOW_LIB": str(lib),
        # CPython's own allocations are not freed at exit; leaks are not checked
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0:exitcode=86",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1:exitcode=87",
    })
    return env


if __name__ == "__main__":
    print(build(Path(sys.argv[1]) if len(sys.argv) > 1 else ROOT / "_build_san"))
