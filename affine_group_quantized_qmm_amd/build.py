"""Build the gfx950 HIP library ``libqmm.so`` in this package directory.

Every ``csrc/*.hip`` file is compiled with hipcc for gfx950 only and linked
into one shared library exporting the C ABI of ``include/qmm.h``.

The build also reads the compiler's kernel-resource-usage remarks and fails if
any kernel spills registers to scratch memory: the kernels are designed to fit
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
    # LDS regions are written and read through different types (staged words,
    # group sums, (scale, bias) words): no type-based alias assumptions
    "-fno-strict-aliasing",
    "-Wall", "-Wno-unused-command-line-argument",
    f"-I{ROOT / 'include'}", f"-I{CSRC}",
]


def _run(cmd, src: Path):
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    text = res.stdout + res.stderr
    if res.returncode != 0:
        err = "\n".join(l for l in text.splitlines() if noise not in l and "remark:" not in l)
        raise RuntimeError(f"hipcc failed for {src.name}:\n{err}")
    return text


def _check_no_scratch(text: str, src: Path):
    """Fail if a kernel uses scratch (register spills), from the compiler's
    kernel-resource-usage remarks."""
    bad, name = [], None
    for line in text.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"remark:\s+(ScratchSize \[bytes/lane\]|VGPRs Spill): (\d+)", line)
        if m and int(m.group(2)) and name not in bad:
            bad.append(name)
    if bad:
        raise RuntimeError(f"{src.name}: kernels spill to scratch memory: {bad[:4]}")


def _compile(src: Path) -> Path:
    obj = BUILD_DIR / (src.stem + ".o")
    text = _run([HIPCC, *FLAGS, "-Rpass-analysis=kernel-resource-usage", "-c", str(src), "-o", str(obj)], src)
    _check_no_scratch(text, src)
    lines, skip = [], 0
    for l in text.splitlines():  # warnings only: drop the remarks and the feature notice
        if "remark:" in l:
            skip = 2  # the source line and caret that follow a remark
            continue
        if skip:
            skip -= 1
            continue
        if "is not a recognized feature for this target" not in l:
            lines.append(l)
    if "\n".join(lines).strip():
        print("\n".join(lines), file=sys.stderr)
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
