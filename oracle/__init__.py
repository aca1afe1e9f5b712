"""CPU fp64 oracle for the affine group-quantized matrix product.

TEST INFRASTRUCTURE ONLY: only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package. The GPU library never calls it and
shares no code with it.

The arithmetic lives in ``qmm_oracle.c`` (plain C, fp64). This module builds
it with gcc and marshals numpy arrays through ctypes; it adds no arithmetic
of its own.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
SOURCE = _HERE / "qmm_oracle.c"
BUILD_DIR = _HERE / "_build"
LIBRARY = BUILD_DIR / "libqmm_oracle.so"

GCC_FLAGS = ["-O2", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
             "-pthread", "-Wall", "-Wextra"]


def build(source: Path = SOURCE, output: Path = LIBRARY, defines: tuple[str, ...] = ()) -> Path:
    """Compile the oracle (or a variant of its source) into a shared library."""
    output.parent.mkdir(parents=True, exist_ok=True)
    cmd = ["gcc", *GCC_FLAGS, *[f"-D{d}" for d in defines], "-o", str(output), str(source), "-lm"]
    subprocess.run(cmd, check=True)
    return output


_i64 = ctypes.c_int64
_p = ctypes.c_void_p


DTYPES = {"f16": 0, "bf16": 1}  # operand types of x, scales and biases


class Oracle:
    """ctypes view of one compiled oracle library."""

    def __init__(self, path: Path):
        lib = ctypes.CDLL(str(path))
        lib.qo_half_to_double.argtypes = [ctypes.c_uint16]
        lib.qo_half_to_double.restype = ctypes.c_double
        lib.qo_half_array_to_double.argtypes = [_p, _p, _i64]
        lib.qo_half_array_to_double.restype = None
        lib.qo_bf16_to_double.argtypes = [ctypes.c_uint16]
        lib.qo_bf16_to_double.restype = ctypes.c_double
        lib.qo_pack.argtypes = [_p, _p, _i64, _i64, ctypes.c_int]
        lib.qo_pack.restype = ctypes.c_int
        lib.qo_unpack.argtypes = [_p, _p, _i64, _i64, ctypes.c_int]
        lib.qo_unpack.restype = ctypes.c_int
        lib.qo_forward.argtypes = [_p, _p, _p, _p, _p, _p, _i64, _i64, _i64,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_int]
        lib.qo_forward.restype = ctypes.c_int
        lib.qo_forward_rows.argtypes = [_p, _p, _p, _p, _p, _p, _i64, _i64, _i64,
                                        ctypes.c_int, ctypes.c_int, _p, _i64, ctypes.c_int]
        lib.qo_forward_rows.restype = ctypes.c_int
        lib.qo_forward_ex.argtypes = [_p, _p, _p, _p, _p, _p, _i64, _i64, _i64,
                                      ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int]
        lib.qo_forward_ex.restype = ctypes.c_int
        lib.qo_forward_rows_ex.argtypes = [_p, _p, _p, _p, _p, _p, _i64, _i64, _i64,
                                           ctypes.c_int, ctypes.c_int, _p, _i64, ctypes.c_int,
                                           ctypes.c_int]
        lib.qo_forward_rows_ex.restype = ctypes.c_int
        lib.qo_forward_factored.argtypes = [_p, _p, _p, _p, _p, _i64, _i64, _i64,
                                            ctypes.c_int, ctypes.c_int, ctypes.c_int]
        lib.qo_forward_factored.restype = ctypes.c_int
        lib.qo_repack_tiled.argtypes = [_p, _p, _p, _p, _p, _i64, _i64, ctypes.c_int, ctypes.c_int]
        lib.qo_repack_tiled.restype = ctypes.c_int
        self.lib = lib
        self.path = path

    # -- conversions -------------------------------------------------------
    def half_to_double(self, h: np.ndarray) -> np.ndarray:
        h = np.ascontiguousarray(h).view(np.uint16)
        out = np.empty(h.shape, dtype=np.float64)
        self.lib.qo_half_array_to_double(h.ctypes.data, out.ctypes.data, h.size)
        return out

    # -- packing -----------------------------------------------------------
    def pack(self, codes: np.ndarray, bits: int) -> np.ndarray:
        codes = np.ascontiguousarray(codes, dtype=np.uint8)
        N, K = codes.shape
        if (K * bits) % 32:
            raise ValueError("K*bits must be a multiple of 32")
        words = np.empty((N, K * bits // 32), dtype=np.uint32)
        rc = self.lib.qo_pack(codes.ctypes.data, words.ctypes.data, N, K, bits)
        if rc:
            raise ValueError(f"qo_pack failed ({rc})")
        return words

    def unpack(self, words: np.ndarray, K: int, bits: int) -> np.ndarray:
        words = np.ascontiguousarray(words, dtype=np.uint32)
        N = words.shape[0]
        if words.shape[1] * 32 != K * bits:
            raise ValueError("word count does not match K*bits/32")
        codes = np.empty((N, K), dtype=np.uint8)
        rc = self.lib.qo_unpack(words.ctypes.data, codes.ctypes.data, N, K, bits)
        if rc:
            raise ValueError(f"qo_unpack failed ({rc})")
        return codes

    def repack_tiled(self, words, scales, biases, K: int, bits: int, G: int):
        """The tiled layout of packed weights: (codes as uint8 [Np*K*bits/8],
        (s | b << 16) words as uint32 [Np*K/G]), Np = N rounded up to 16."""
        words = np.ascontiguousarray(words, dtype=np.uint32)
        s = np.ascontiguousarray(scales, dtype=np.float16).view(np.uint16)
        b = np.ascontiguousarray(biases, dtype=np.float16).view(np.uint16)
        N = words.shape[0]
        Np = (N + 15) // 16 * 16
        tw = np.empty(Np * K * bits // 8, dtype=np.uint8)
        tsb = np.empty(Np * (K // G), dtype=np.uint32)
        rc = self.lib.qo_repack_tiled(words.ctypes.data, s.ctypes.data, b.ctypes.data,
                                      tw.ctypes.data, tsb.ctypes.data, N, K, bits, G)
        if rc:
            raise ValueError(f"qo_repack_tiled failed ({rc})")
        return tw, tsb

    # -- products ----------------------------------------------------------
    @staticmethod
    def _operands(x, words, scales, biases, dtype="f16"):
        """fp16 operands as float16 arrays; bf16 operands as uint16 bit patterns."""
        if dtype not in DTYPES:
            raise ValueError(f"dtype must be one of {tuple(DTYPES)}")
        t = np.float16 if dtype == "f16" else np.uint16
        x = np.ascontiguousarray(x, dtype=t)
        words = np.ascontiguousarray(words, dtype=np.uint32)
        scales = np.ascontiguousarray(scales, dtype=t)
        biases = np.ascontiguousarray(biases, dtype=t)
        return x, words, scales, biases

    def bf16_to_double(self, h: np.ndarray) -> np.ndarray:
        """bfloat16 bit patterns (uint16) -> float64, elementwise."""
        h = np.ascontiguousarray(h, dtype=np.uint16)
        out = np.empty(h.shape, dtype=np.float64)
        flat, o = h.ravel(), out.ravel()
        for i in range(flat.size):
            o[i] = self.lib.qo_bf16_to_double(int(flat[i]))
        return out

    def forward(self, x, words, scales, biases, bits: int, G: int, nthreads: int | None = None,
                dtype: str = "f16"):
        """Dequantize-then-dot. Returns (y, A) as float64 [M, N]; A = sum_k |w x|.
        dtype "bf16": x, scales and biases are bfloat16 bit patterns (uint16)."""
        x, words, scales, biases = self._operands(x, words, scales, biases, dtype)
        M, K = x.shape
        N = words.shape[0]
        y = np.empty((M, N), dtype=np.float64)
        a = np.empty((M, N), dtype=np.float64)
        rc = self.lib.qo_forward_ex(x.ctypes.data, words.ctypes.data, scales.ctypes.data,
                                    biases.ctypes.data, y.ctypes.data, a.ctypes.data,
                                    M, K, N, bits, G, DTYPES[dtype], nthreads or default_threads())
        if rc:
            raise ValueError(f"qo_forward failed ({rc})")
        return y, a

    def forward_rows(self, x, words, scales, biases, bits: int, G: int, rows,
                     nthreads: int | None = None, dtype: str = "f16"):
        """Like ``forward`` for the listed output rows only: (y, A) are [M, len(rows)]."""
        x, words, scales, biases = self._operands(x, words, scales, biases, dtype)
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        M, K = x.shape
        N = words.shape[0]
        y = np.empty((M, rows.size), dtype=np.float64)
        a = np.empty((M, rows.size), dtype=np.float64)
        rc = self.lib.qo_forward_rows_ex(x.ctypes.data, words.ctypes.data, scales.ctypes.data,
                                         biases.ctypes.data, y.ctypes.data, a.ctypes.data,
                                         M, K, N, bits, G, rows.ctypes.data, rows.size,
                                         DTYPES[dtype], nthreads or default_threads())
        if rc:
            raise ValueError(f"qo_forward_rows failed ({rc})")
        return y, a

    def forward_factored(self, x, words, scales, biases, bits: int, G: int,
                         nthreads: int | None = None):
        """The factored form sum_g (s*P + b*XS), fp64. Returns y [M, N]."""
        x, words, scales, biases = self._operands(x, words, scales, biases)
        M, K = x.shape
        N = words.shape[0]
        y = np.empty((M, N), dtype=np.float64)
        rc = self.lib.qo_forward_factored(x.ctypes.data, words.ctypes.data,
                                          scales.ctypes.data, biases.ctypes.data,
                                          y.ctypes.data, M, K, N, bits, G,
                                          nthreads or default_threads())
        if rc:
            raise ValueError(f"qo_forward_factored failed ({rc})")
        return y


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


_DEFAULT: Oracle | None = None


def get() -> Oracle:
    """The oracle built from ``qmm_oracle.c`` (compiled on first use if needed)."""
    global _DEFAULT
    if _DEFAULT is None:
        if not LIBRARY.exists() or LIBRARY.stat().st_mtime < SOURCE.stat().st_mtime:
            build()
        _DEFAULT = Oracle(LIBRARY)
    return _DEFAULT


def parity_bound(absum: np.ndarray) -> np.ndarray:
    """Per-element tolerance of the GPU fp32 result: 1e-5 * sum_k |w x| + 1e-6."""
    return 1e-5 * absum + 1e-6
