"""Python binding of the gfx950 affine group-quantized matrix product library.

Thin argument marshalling over the C ABI of ``include/qmm.h`` (``libqmm.so``
built in this directory): the functions below carry the C names, check
tensor dtypes/devices/shapes, pass device pointers and torch's current HIP
stream, and turn negative return codes into exceptions. Every step of the
product runs in the library's HIP kernels; there is no fallback path.

Tensors (all on one ROCm device, contiguous):
  x       float16 [M, K]
  wq      int32 or uint32 [N, K*bits/32]   (bit patterns of the packed words)
  scales  float16 [N, K/G]
  biases  float16 [N, K/G]
  y       float32 [M, N]
"""
from __future__ import annotations

import ctypes
from pathlib import Path

import torch

LIBRARY_PATH = Path(__file__).resolve().parent / "libqmm.so"

if not LIBRARY_PATH.exists():
    raise ImportError(
        f"{LIBRARY_PATH} is missing: build the HIP library first "
        "(python -c 'import __graft_entry__ as g; g.build()' at the repository root)")

_lib = ctypes.CDLL(str(LIBRARY_PATH))

_p, _i, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
_lib.qmm_pack.argtypes = [_p, _p, _i, _i, _i, _p]
_lib.qmm_forward.argtypes = [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _p]
_lib.qmm_forward_rowexact.argtypes = [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _p]
_lib.qmm_forward_bf16.argtypes = [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _p]
_lib.qmm_forward_splitk.argtypes = [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _p, _sz, _p]
_lib.qmm_forward_splitk_noalloc.argtypes = [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _p]
_lib.qmm_forward_kernel.argtypes = [ctypes.c_char_p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _p]
_lib.qmm_forward_fused.argtypes = [_p, _i, _p, _p, _p, _p, _p, _i, _i, _i, _i, _p]
_lib.qmm_tiled_bytes.argtypes = [_i, _i, _i, _i, ctypes.POINTER(_sz)]
_lib.qmm_tiled_bytes.restype = _sz
_lib.qmm_repack_tiled.argtypes = [_p, _p, _p, _p, _p, _i, _i, _i, _i, _p]
_lib.qmm_forward_tiled.argtypes = [_p, _p, _p, _p, _i, _i, _i, _i, _i, _p]
_lib.qmm_stream_read.argtypes = [_p, _sz, _p, _p]
_lib.qmm_admit_workspace_bytes.argtypes = [_i, _i]
_lib.qmm_admit_workspace_bytes.restype = _sz
_lib.qmm_admit.argtypes = [ctypes.c_char_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _p, _sz, _p,
                           ctypes.POINTER(_i)]
_lib.qmm_admission.argtypes = [ctypes.c_char_p, _i, _i, _i, _i, _i]
_lib.qmm_admission_clear.argtypes = []
_lib.qmm_admission_clear.restype = None
_lib.qmm_stream_read_sink_words.argtypes = [_sz]
_lib.qmm_stream_read_sink_words.restype = _sz
_lib.qmm_splitk_workspace_bytes.argtypes = [_i, _i, _i]
_lib.qmm_splitk_workspace_bytes.restype = _sz
_lib.qmm_validate.argtypes = [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _p, _sz]
_lib.qmm_strerror.argtypes = [_i]
_lib.qmm_strerror.restype = ctypes.c_char_p
_lib.qmm_kernel_name.argtypes = [_i, _i, _i, _i, _i]
_lib.qmm_kernel_name.restype = ctypes.c_char_p
for _f in (_lib.qmm_pack, _lib.qmm_forward, _lib.qmm_forward_rowexact, _lib.qmm_forward_bf16,
           _lib.qmm_forward_splitk, _lib.qmm_forward_splitk_noalloc,
           _lib.qmm_forward_kernel, _lib.qmm_forward_fused, _lib.qmm_repack_tiled,
           _lib.qmm_forward_tiled, _lib.qmm_validate, _lib.qmm_stream_read, _lib.qmm_admit,
           _lib.qmm_admission):
    _f.restype = _i

EXPORTED = ("qmm_pack", "qmm_forward", "qmm_forward_rowexact", "qmm_forward_bf16", "qmm_forward_splitk",
            "qmm_forward_splitk_noalloc",
            "qmm_splitk_workspace_bytes", "qmm_validate", "qmm_strerror", "qmm_kernel_name",
            "qmm_forward_kernel", "qmm_forward_fused", "qmm_tiled_bytes", "qmm_repack_tiled",
            "qmm_forward_tiled", "qmm_stream_read", "qmm_stream_read_sink_words",
            "qmm_admit_workspace_bytes", "qmm_admit", "qmm_admission", "qmm_admission_clear")

QMM_MAX_FUSED = 4  # projections per qmm_forward_fused call


QMM_ERR_UNSUPPORTED = -9  # qmm_forward_kernel: the named kernel cannot run this shape
QMM_ERR_SCRATCH = -10     # qmm_forward_splitk_noalloc: partials exceed the static scratch
QMM_NOALLOC_SCRATCH_BYTES = 16 << 20
QMM_ADMISSION_UNKNOWN = 2  # qmm_admission: the shape was never examined


class QmmError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {qmm_strerror(code)} (code {code})")
        self.code = code


def qmm_strerror(code: int) -> str:
    return _lib.qmm_strerror(code).decode()


def qmm_splitk_workspace_bytes(M: int, N: int, split_k: int) -> int:
    return int(_lib.qmm_splitk_workspace_bytes(M, N, split_k))


def qmm_kernel_name(M: int, K: int, N: int, bits: int, G: int) -> str | None:
    name = _lib.qmm_kernel_name(M, K, N, bits, G)
    return name.decode() if name else None


def qmm_validate(x_ptr: int, wq_ptr: int, s_ptr: int, b_ptr: int, y_ptr: int, M: int, K: int,
                 N: int, bits: int, G: int, split_k: int = 0, ws_ptr: int = 0,
                 ws_bytes: int = 0) -> int:
    """Host-only argument validation on raw addresses (no GPU needed)."""
    return int(_lib.qmm_validate(x_ptr or None, wq_ptr or None, s_ptr or None, b_ptr or None,
                                 y_ptr or None, M, K, N, bits, G, split_k, ws_ptr or None,
                                 ws_bytes))


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _check(t: torch.Tensor, name: str, dtypes, shape, device) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} must have dtype in {dtypes}, got {t.dtype}")
    if t.device.type != "cuda" or (device is not None and t.device != device):
        raise ValueError(f"{name} must be on the GPU device {device}, got {t.device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


_WORD_DTYPES = (torch.int32, torch.uint32)


def _operands(x, wq, scales, biases, bits, G, dtype=torch.float16):
    if x.dim() != 2 or wq.dim() != 2:
        raise ValueError("x and wq must be 2-D")
    M, K = x.shape
    N = wq.shape[0]
    if K % G or (K * bits) % 32:
        raise ValueError("K must be a multiple of G (and K*bits of 32)")
    dev = x.device
    _check(x, "x", (dtype,), (M, K), None)
    _check(wq, "wq", _WORD_DTYPES, (N, K * bits // 32), dev)
    _check(scales, "scales", (dtype,), (N, K // G), dev)
    _check(biases, "biases", (dtype,), (N, K // G), dev)
    return M, K, N, dev


def qmm_pack(codes: torch.Tensor, bits: int, out: torch.Tensor | None = None) -> torch.Tensor:
    """Pack uint8 codes [N, K] into int32 words [N, K*bits/32] on the GPU."""
    if codes.dim() != 2:
        raise ValueError("codes must be 2-D")
    N, K = codes.shape
    _check(codes, "codes", (torch.uint8,), (N, K), None)
    if (K * bits) % 32:
        raise ValueError("K*bits must be a multiple of 32")
    if out is None:
        out = torch.empty((N, K * bits // 32), dtype=torch.int32, device=codes.device)
    _check(out, "out", _WORD_DTYPES, (N, K * bits // 32), codes.device)
    rc = _lib.qmm_pack(codes.data_ptr(), out.data_ptr(), N, K, bits, _stream(codes))
    if rc:
        raise QmmError(rc, "qmm_pack")
    return out


def qmm_forward(x, wq, scales, biases, bits: int, G: int, out=None) -> torch.Tensor:
    """y = x . W^T (fp32 [M, N]) for packed affine weights."""
    M, K, N, dev = _operands(x, wq, scales, biases, bits, G)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=dev)
    _check(out, "out", (torch.float32,), (M, N), dev)
    rc = _lib.qmm_forward(x.data_ptr(), wq.data_ptr(), scales.data_ptr(), biases.data_ptr(),
                          out.data_ptr(), M, K, N, bits, G, _stream(x))
    if rc:
        raise QmmError(rc, "qmm_forward")
    return out


def qmm_forward_rowexact(x, wq, scales, biases, bits: int, G: int, out=None) -> torch.Tensor:
    """qmm_forward whose every row is bitwise equal to the one-row call on that row."""
    M, K, N, dev = _operands(x, wq, scales, biases, bits, G)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=dev)
    _check(out, "out", (torch.float32,), (M, N), dev)
    rc = _lib.qmm_forward_rowexact(x.data_ptr(), wq.data_ptr(), scales.data_ptr(),
                                   biases.data_ptr(), out.data_ptr(), M, K, N, bits, G, _stream(x))
    if rc:
        raise QmmError(rc, "qmm_forward_rowexact")
    return out


def qmm_forward_bf16(x, wq, scales, biases, bits: int, G: int, out=None) -> torch.Tensor:
    """The product with bfloat16 x, scales and biases (fp32 y)."""
    M, K, N, dev = _operands(x, wq, scales, biases, bits, G, dtype=torch.bfloat16)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=dev)
    _check(out, "out", (torch.float32,), (M, N), dev)
    rc = _lib.qmm_forward_bf16(x.data_ptr(), wq.data_ptr(), scales.data_ptr(),
                               biases.data_ptr(), out.data_ptr(), M, K, N, bits, G, _stream(x))
    if rc:
        raise QmmError(rc, "qmm_forward_bf16")
    return out


def _ptr_array(ptrs):
    return (ctypes.c_void_p * len(ptrs))(*ptrs)


def qmm_forward_fused(x, projections, bits: int, G: int, outs=None) -> list[torch.Tensor]:
    """Several projections of the same x in one launch.

    `projections` is a sequence of (wq, scales, biases) triples with a common K;
    returns one fp32 [M, N_p] tensor per projection (or fills `outs`)."""
    count = len(projections)
    if count < 1:
        raise ValueError("at least one projection")
    dims = [_operands(x, wq, s, b, bits, G) for wq, s, b in projections]
    M, K, _, dev = dims[0]
    Ns = [d[2] for d in dims]
    if outs is None:
        outs = [torch.empty((M, n), dtype=torch.float32, device=dev) for n in Ns]
    if len(outs) != count:
        raise ValueError("one output per projection")
    for o, n in zip(outs, Ns):
        _check(o, "out", (torch.float32,), (M, n), dev)
    rc = _lib.qmm_forward_fused(
        x.data_ptr(), count,
        _ptr_array([p[0].data_ptr() for p in projections]),
        _ptr_array([p[1].data_ptr() for p in projections]),
        _ptr_array([p[2].data_ptr() for p in projections]),
        _ptr_array([o.data_ptr() for o in outs]),
        (ctypes.c_int * count)(*Ns), M, K, bits, G, _stream(x))
    if rc:
        raise QmmError(rc, "qmm_forward_fused")
    return outs


def qmm_tiled_bytes(N: int, K: int, bits: int, G: int) -> tuple[int, int]:
    """(code bytes, (s, b) word bytes) of the tiled layout; (0, 0) if it does not exist."""
    sb = _sz(0)
    w = _lib.qmm_tiled_bytes(N, K, bits, G, ctypes.byref(sb))
    return int(w), int(sb.value)


def qmm_repack_tiled(wq, scales, biases, bits: int, G: int):
    """The tiled (matrix-core) layout of packed weights: (uint8 codes, int32 (s, b) words)."""
    N = wq.shape[0]
    K = scales.shape[1] * G
    _operands(torch.empty((1, K), dtype=torch.float16, device=wq.device), wq, scales, biases, bits, G)
    wb, sbb = qmm_tiled_bytes(N, K, bits, G)
    if not wb:
        raise QmmError(QMM_ERR_UNSUPPORTED, "qmm_repack_tiled")
    tw = torch.empty(wb, dtype=torch.uint8, device=wq.device)
    tsb = torch.empty(sbb // 4, dtype=torch.int32, device=wq.device)
    rc = _lib.qmm_repack_tiled(wq.data_ptr(), scales.data_ptr(), biases.data_ptr(), tw.data_ptr(),
                               tsb.data_ptr(), N, K, bits, G, _stream(wq))
    if rc:
        raise QmmError(rc, "qmm_repack_tiled")
    return tw, tsb


def qmm_forward_tiled(x, tw, tsb, N: int, bits: int, G: int, out=None) -> torch.Tensor:
    """y = x . W^T from the tiled layout (qmm_repack_tiled's output)."""
    if x.dim() != 2:
        raise ValueError("x must be 2-D")
    M, K = x.shape
    _check(x, "x", (torch.float16,), (M, K), None)
    wb, sbb = qmm_tiled_bytes(N, K, bits, G)
    if not wb:
        raise QmmError(QMM_ERR_UNSUPPORTED, "qmm_forward_tiled")
    _check(tw, "tiled_w", (torch.uint8,), (wb,), x.device)
    _check(tsb, "tiled_sb", (torch.int32, torch.uint32), (sbb // 4,), x.device)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=x.device)
    _check(out, "out", (torch.float32,), (M, N), x.device)
    rc = _lib.qmm_forward_tiled(x.data_ptr(), tw.data_ptr(), tsb.data_ptr(), out.data_ptr(), M, K, N,
                                bits, G, _stream(x))
    if rc:
        raise QmmError(rc, "qmm_forward_tiled")
    return out


def qmm_forward_kernel(kernel: str, x, wq, scales, biases, bits: int, G: int,
                       out=None) -> torch.Tensor:
    """qmm_forward with an explicitly named kernel ("qmv", "mfma" or "mfma_lds")."""
    M, K, N, dev = _operands(x, wq, scales, biases, bits, G)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=dev)
    _check(out, "out", (torch.float32,), (M, N), dev)
    rc = _lib.qmm_forward_kernel(kernel.encode(), x.data_ptr(), wq.data_ptr(),
                                 scales.data_ptr(), biases.data_ptr(), out.data_ptr(), M, K, N,
                                 bits, G, _stream(x))
    if rc:
        raise QmmError(rc, "qmm_forward_kernel")
    return out


def qmm_admit_workspace_bytes(M: int, N: int) -> int:
    return int(_lib.qmm_admit_workspace_bytes(M, N))


def qmm_admit(kind: str, x, wq, scales, biases, bits: int, G: int, workspace=None) -> bool:
    """Bitwise admission of `kind` ("rowexact" or "forward") against one-row
    launches on these inputs; records and returns the verdict (waits for the
    current stream)."""
    M, K, N, dev = _operands(x, wq, scales, biases, bits, G)
    need = qmm_admit_workspace_bytes(M, N)
    if workspace is None:
        workspace = torch.empty(-(-need // 4), dtype=torch.float32, device=dev)
    nbytes = workspace.numel() * workspace.element_size()
    out = ctypes.c_int(-1)
    rc = _lib.qmm_admit(kind.encode(), x.data_ptr(), wq.data_ptr(), scales.data_ptr(), biases.data_ptr(),
                        M, K, N, bits, G, workspace.data_ptr(), nbytes, _stream(x), ctypes.byref(out))
    if rc:
        raise QmmError(rc, "qmm_admit")
    return bool(out.value)


def qmm_admission(kind: str, M: int, K: int, N: int, bits: int, G: int) -> int:
    """1 admitted, 0 rejected, QMM_ADMISSION_UNKNOWN never examined (host-only)."""
    rc = _lib.qmm_admission(kind.encode(), M, K, N, bits, G)
    if rc < 0:
        raise QmmError(rc, "qmm_admission")
    return rc


def qmm_admission_clear() -> None:
    _lib.qmm_admission_clear()


def qmm_stream_read_sink_words(nbytes: int) -> int:
    return int(_lib.qmm_stream_read_sink_words(nbytes))


def qmm_stream_read(src: torch.Tensor, sink: torch.Tensor | None = None) -> torch.Tensor:
    """Streaming-read ceiling: reads every byte of the contiguous GPU tensor
    `src` once; returns the int32 sink (one XOR word per 8 KiB span)."""
    if not isinstance(src, torch.Tensor) or src.device.type != "cuda" or not src.is_contiguous():
        raise ValueError("src must be a contiguous GPU tensor")
    nbytes = src.numel() * src.element_size()
    words = qmm_stream_read_sink_words(nbytes)
    if sink is None:
        sink = torch.empty(max(words, 1), dtype=torch.int32, device=src.device)
    _check(sink, "sink", _WORD_DTYPES, (max(words, 1),), src.device)
    rc = _lib.qmm_stream_read(src.data_ptr(), nbytes, sink.data_ptr(), _stream(src))
    if rc:
        raise QmmError(rc, "qmm_stream_read")
    return sink


def qmm_forward_splitk(x, wq, scales, biases, bits: int, G: int, split_k: int,
                       workspace=None, out=None) -> torch.Tensor:
    """The product with K split into split_k slices and an in-order fp32 reduction."""
    M, K, N, dev = _operands(x, wq, scales, biases, bits, G)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=dev)
    _check(out, "out", (torch.float32,), (M, N), dev)
    need = qmm_splitk_workspace_bytes(M, N, split_k)
    if workspace is None and need:
        workspace = torch.empty(need // 4, dtype=torch.float32, device=dev)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = _lib.qmm_forward_splitk(x.data_ptr(), wq.data_ptr(), scales.data_ptr(),
                                 biases.data_ptr(), out.data_ptr(), M, K, N, bits, G, split_k,
                                 ws_ptr, ws_bytes, _stream(x))
    if rc:
        raise QmmError(rc, "qmm_forward_splitk")
    return out


def qmm_forward_splitk_noalloc(x, wq, scales, biases, bits: int, G: int, split_k: int,
                               out=None) -> torch.Tensor:
    """qmm_forward_splitk with its partials in the library's static scratch
    (the library allocates nothing; `out` may be preallocated by the caller)."""
    M, K, N, dev = _operands(x, wq, scales, biases, bits, G)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=dev)
    _check(out, "out", (torch.float32,), (M, N), dev)
    rc = _lib.qmm_forward_splitk_noalloc(x.data_ptr(), wq.data_ptr(), scales.data_ptr(),
                                         biases.data_ptr(), out.data_ptr(), M, K, N, bits, G,
                                         split_k, _stream(x))
    if rc:
        raise QmmError(rc, "qmm_forward_splitk_noalloc")
    return out
