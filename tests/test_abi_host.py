"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/qmm.h declares, and rejects bad arguments with the
documented codes before touching the GPU."""
import ctypes
import re
from pathlib import Path

import pytest

# A missing libqmm.so is a failure here (ImportError at collection), not a skip:
# these checks are what shows that the boundary exists at all.
import affine_group_quantized_qmm_amd as qmm

ROOT = Path(__file__).resolve().parents[1]
HEADER = ROOT / "include" / "qmm.h"


def declared_functions():
    text = re.sub(r"/\*.*?\*/", "", HEADER.read_text(), flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(qmm_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("qmm_pack", "qmm_forward", "qmm_forward_splitk"):
        assert required in names


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(str(qmm.LIBRARY_PATH))
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, f"declared but not exported: {missing}"
    assert set(declared_functions()) == set(qmm.EXPORTED)


def test_error_codes_and_messages():
    for code in range(0, -11, -1):
        assert qmm.qmm_strerror(code) and "unknown" not in qmm.qmm_strerror(code)
    assert "unknown" in qmm.qmm_strerror(-99)


A = 0x10000  # a fake, 16-byte aligned address: validation never dereferences it


def v(**kw):
    args = dict(x=A, wq=A, s=A, b=A, y=A, M=4, K=512, N=256, bits=4, G=32, split=0, ws=0, wsb=0)
    args.update(kw)
    return qmm.qmm_validate(args["x"], args["wq"], args["s"], args["b"], args["y"], args["M"],
                            args["K"], args["N"], args["bits"], args["G"], args["split"],
                            args["ws"], args["wsb"])


def test_validation_accepts_good_arguments():
    assert v() == 0
    for bits in (2, 3, 4, 5, 6, 8):
        for G in (32, 64, 128):
            assert v(bits=bits, G=G, K=G * 3) == 0
    need = qmm.qmm_splitk_workspace_bytes(4, 256, 3)
    assert need == 3 * 4 * 256 * 4
    assert v(split=3, ws=A, wsb=need) == 0
    assert v(split=1) == 0  # no workspace needed for one slice
    assert qmm.qmm_splitk_workspace_bytes(4, 256, 1) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(x=0), -1), (dict(wq=0), -1), (dict(s=0), -1), (dict(b=0), -1), (dict(y=0), -1),
    (dict(split=2, ws=0, wsb=1 << 20), -1),
    (dict(M=0), -2), (dict(K=0), -2), (dict(N=0), -2), (dict(K=100), -2), (dict(K=48, G=32), -2),
    (dict(N=-5), -2), (dict(K=1 << 29), -2),
    (dict(bits=1), -3), (dict(bits=7), -3), (dict(bits=16), -3),
    (dict(G=16), -4), (dict(G=96), -4),
    (dict(split=-1, ws=A, wsb=1 << 30), -5), (dict(split=17, ws=A, wsb=1 << 30), -5),
    (dict(split=2, ws=A, wsb=100), -6),
    (dict(x=A + 2), -7), (dict(wq=A + 4), -7), (dict(y=A + 8), -7), (dict(s=A + 2), -7),
    (dict(split=2, ws=A + 4, wsb=1 << 20), -7),
])
def test_validation_rejects(kw, code):
    assert v(**kw) == code


def test_kernel_choice():
    assert qmm.qmm_kernel_name(1, 5120, 17408, 4, 32) == "qmv"
    assert qmm.qmm_kernel_name(2, 5120, 17408, 4, 32) == "qmv"
    assert qmm.qmm_kernel_name(3, 5120, 17408, 4, 32) == "mfma"
    assert qmm.qmm_kernel_name(16, 5120, 17408, 4, 32) == "mfma"
    assert qmm.qmm_kernel_name(16, 5120, 17408, 7, 32) is None
    # K past 8 parts of 768 activations: each wave walks several parts (768
    # activations for 2-4-bit codes, 640 otherwise; at most 8 passes), past
    # that the LDS-streaming kernel
    assert qmm.qmm_kernel_name(16, 17408, 5120, 4, 32) == "mfma"
    assert qmm.qmm_kernel_name(4, 6144, 1024, 4, 32) == "mfma"
    assert qmm.qmm_kernel_name(4, 6176, 1024, 4, 32) == "mfma"
    assert qmm.qmm_kernel_name(4, 49152, 64, 4, 32) == "mfma"      # 8 passes of 8 parts of 768
    assert qmm.qmm_kernel_name(4, 49152 + 64, 64, 4, 32) == "mfma_lds"
    assert qmm.qmm_kernel_name(4, 40960, 64, 8, 32) == "mfma"      # 8 passes of 8 parts of 640
    assert qmm.qmm_kernel_name(4, 40960 + 64, 64, 8, 32) == "mfma_lds"
    assert qmm.qmm_kernel_name(4, 65536, 64, 4, 32) == "mfma_lds"
    # 5-bit rows of 13 groups are not whole 16-byte units
    assert qmm.qmm_kernel_name(4, 13 * 32, 200, 5, 32) == "mfma_lds"
    assert qmm.qmm_kernel_name(4, 5120, 5120, 8, 64) == "mfma"      # 8-bit: parts of 640 activations
    assert qmm.qmm_kernel_name(4, 17408, 5120, 8, 64) == "mfma"
    assert qmm.qmm_kernel_name(4, 5120, 5120, 6, 64) == "mfma"
    # 2- and 3-bit codes
    assert qmm.qmm_kernel_name(2, 5120, 1000, 2, 32) == "qmv"
    assert qmm.qmm_kernel_name(8, 5120, 1000, 2, 32) == "mfma"
    assert qmm.qmm_kernel_name(8, 5120, 1000, 3, 32) == "mfma"
    assert qmm.qmm_kernel_name(8, 17408, 1000, 2, 32) == "mfma"
    assert qmm.qmm_kernel_name(8, 17408, 1000, 3, 64) == "mfma"
    assert qmm.qmm_kernel_name(8, 17408, 1000, 3, 32) == "mfma"
    # past the register-resident kernel: LDS kernel, except 3-bit G=32 (VALU kernel)
    assert qmm.qmm_kernel_name(8, 65536, 1000, 2, 32) == "mfma_lds"
    assert qmm.qmm_kernel_name(8, 65536, 1000, 3, 32) == "qmv"


def test_fused_rejects_before_launch():
    """qmm_forward_fused checks its arrays and every projection on the host."""
    lib = qmm._lib
    good = (ctypes.c_void_p * 2)(4096, 8192)
    ns = (ctypes.c_int * 2)(16, 8)
    assert lib.qmm_forward_fused(4096, 2, None, good, good, good, ns, 1, 64, 4, 32, None) == -1
    assert lib.qmm_forward_fused(None, 2, good, good, good, good, ns, 1, 64, 4, 32, None) == -1
    assert lib.qmm_forward_fused(4096, 0, good, good, good, good, ns, 1, 64, 4, 32, None) == -2
    assert lib.qmm_forward_fused(4096, qmm.QMM_MAX_FUSED + 1, good, good, good, good, ns, 1, 64,
                                 4, 32, None) == -2
    assert lib.qmm_forward_fused(4096, 2, good, good, good, good, ns, 1, 64, 7, 32, None) == -3
    assert lib.qmm_forward_fused(4096, 2, good, good, good, good, ns, 1, 64, 4, 48, None) == -4
    bad_n = (ctypes.c_int * 2)(16, 0)
    assert lib.qmm_forward_fused(4096, 2, good, good, good, good, bad_n, 1, 64, 4, 32, None) == -2
    odd = (ctypes.c_void_p * 2)(4096, 8200)  # second projection's pointer misaligned
    assert lib.qmm_forward_fused(4096, 2, odd, good, good, good, ns, 1, 64, 4, 32, None) == -7
    null_p = (ctypes.c_void_p * 2)(4096, None)
    assert lib.qmm_forward_fused(4096, 2, good, good, null_p, good, ns, 1, 64, 4, 32, None) == -1


def test_tiled_sizes_and_rejections():
    """Sizes of the tiled layout, and shapes it does not exist for, on the host."""
    assert qmm.qmm_tiled_bytes(17408, 5120, 4, 32) == (17408 * 5120 // 2, 17408 * 160 * 4)
    assert qmm.qmm_tiled_bytes(20, 512, 8, 32) == (32 * 512, 32 * 16 * 4)  # rows padded to 32
    for args in ((100, 5120, 5, 32), (100, 5120, 6, 64), (16, 416, 4, 32), (16, 192, 8, 64)):
        assert qmm.qmm_tiled_bytes(*args) == (0, 0), args
    lib = qmm._lib
    assert lib.qmm_repack_tiled(None, 16, 16, 16, 16, 16, 512, 4, 32, None) == -1
    assert lib.qmm_repack_tiled(16, 16, 16, 16, 16, 16, 512, 5, 32, None) == -9
    assert lib.qmm_repack_tiled(16, 16, 16, 16, 24, 16, 512, 4, 32, None) == -7
    assert lib.qmm_forward_tiled(16, 16, 16, 16, 1, 512, 16, 3, 32, None) == -9
    assert lib.qmm_forward_tiled(16, 16, 16, 16, 1, 416, 16, 4, 32, None) == -9
    assert lib.qmm_forward_tiled(16, 16, None, 16, 1, 512, 16, 4, 32, None) == -1


def test_stream_read_rejects_before_launch():
    lib = qmm._lib
    assert qmm.qmm_stream_read_sink_words(0) == 0
    assert qmm.qmm_stream_read_sink_words(40) == 0
    assert qmm.qmm_stream_read_sink_words(16) == 1
    assert qmm.qmm_stream_read_sink_words(8192) == 1
    assert qmm.qmm_stream_read_sink_words(8192 + 16) == 2
    assert lib.qmm_stream_read(None, 64, A, None) == -1
    assert lib.qmm_stream_read(A, 64, None, None) == -1
    assert lib.qmm_stream_read(A, 0, A, None) == -2
    assert lib.qmm_stream_read(A, 40, A, None) == -2
    assert lib.qmm_stream_read(A + 4, 64, A, None) == -7
    assert lib.qmm_stream_read(A, 64, A + 2, None) == -7


def test_admission_table_and_rejections_before_launch():
    lib = qmm._lib
    qmm.qmm_admission_clear()
    assert qmm.qmm_admission("rowexact", 4, 512, 256, 4, 32) == qmm.QMM_ADMISSION_UNKNOWN
    assert lib.qmm_admission(None, 4, 512, 256, 4, 32) == -1
    assert lib.qmm_admission(b"nonsense", 4, 512, 256, 4, 32) == -2
    assert qmm.qmm_admit_workspace_bytes(4, 256) == 2 * 4 * 256 * 4 + 16
    assert qmm.qmm_admit_workspace_bytes(0, 256) == 0
    out = ctypes.c_int(-1)
    need = qmm.qmm_admit_workspace_bytes(4, 256)

    def admit(kind=b"rowexact", ws=A, wsb=need, ptr=ctypes.byref(out), M=4, bits=4):
        return lib.qmm_admit(kind, A, A, A, A, M, 512, 256, bits, 32, ws, wsb, None, ptr)
    assert admit(kind=None) == -1
    assert admit(ptr=None) == -1
    assert admit(ws=None) == -1
    assert admit(kind=b"nonsense") == -2
    assert admit(M=0) == -2
    assert admit(bits=7) == -3
    assert admit(wsb=need - 1) == -6
    assert admit(ws=A + 4) == -7
    assert out.value == -1  # nothing was recorded or written
    assert qmm.qmm_admission("rowexact", 4, 512, 256, 4, 32) == qmm.QMM_ADMISSION_UNKNOWN
