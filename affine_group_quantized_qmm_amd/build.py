"""Build the gfx950 HIP library ``libqmm.so`` in this package directory.

Every ``csrc/*.hip`` file is compiled with hipcc for gfx950 only and linked
into one shared library exporting the C ABI of ``include/qmm.h``.

The build also compiles each file's device code to assembly and fails if any
kernel spills registers to scratch memory: the kernels are designed to fit
their registers, and spilled variants of the matrix-core kernels have produced
wrong results with this toolchain.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
BUILD_DIR = PKG / "_build"
LIBRARY = PKG / "libqmm.so"
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # no packed fp32 instructions (compiler-generated v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    f"-I{ROOT / 'include'}", f"-I{CSRC}",
]


def _run(cmd, src: Path):
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src.name}:\n{err}")
    return err


def _check_no_scratch(asm: Path, src: Path):
    """Fail if a kernel in the device assembly uses scratch (register spills)."""
    text = asm.read_text()
    bad = []
    for block in text.split("  - .agpr_count:")[1:]:
        name = re.search(r"\.name:\s+(\S+)", block)
        priv = re.search(r"\.private_segment_fixed_size:\s+(\d+)", block)
        spill = re.search(r"\.vgpr_spill_count:\s+(\d+)", block)
        if name and ((priv and int(priv.group(1))) or (spill and int(spill.group(1)))):
            bad.append(name.group(1))
    if bad:
        raise RuntimeError(f"{src.name}: kernels spill to scratch memory: {bad[:4]}")


def _compile(src: Path) -> Path:
    obj = BUILD_DIR / (src.stem + ".o")
    asm = BUILD_DIR / (src.stem + ".s")
    err = _run([HIPCC, *FLAGS, "-c", str(src), "-o", str(obj)], src)
    _run([HIPCC, *FLAGS, "--cuda-device-only", "-S", str(src), "-o", str(asm)], src)
    _check_no_scratch(asm, src)
    if err.strip():
        print(err, file=sys.stderr)
    return obj


def build(jobs: int | None = None) -> Path:
    """Compile all sources (always) and link ``libqmm.so``; returns its path."""
    BUILD_DIR.mkdir(exist_ok=True)
    sources = sorted(CSRC.glob("*.hip"))
    with cf.ThreadPoolExecutor(max_workers=jobs or min(8, len(sources))) as ex:
        objs = list(ex.map(_compile, sources))
    tmp = LIBRARY.with_suffix(".so.tmp")
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", str(tmp), *map(str, objs)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build())
