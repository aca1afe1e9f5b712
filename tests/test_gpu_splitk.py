"""qmm_forward_splitk: every split factor (including uneven splits) meets the
bound against the oracle, and reruns are bitwise identical."""
import pytest
import torch

import qmm_inputs
from tests import _gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("S", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("M", [1, 5, 16])
@pytest.mark.parametrize("bits,G", [(4, 32), (6, 64), (8, 32)])
def test_splitk_parity(S, M, bits, G):
    K, N = 43 * G, 150  # 43 groups: uneven for every S > 1
    dp = _gpu.DeviceProblem(qmm_inputs.make_problem(seed=S + M, M=M, K=K, N=N, bits=bits, G=G))
    qmm = _gpu.lib()
    y = qmm.qmm_forward_splitk(dp.x, dp.wq, dp.s, dp.b, bits, G, S)
    y2 = qmm.qmm_forward_splitk(dp.x, dp.wq, dp.s, dp.b, bits, G, S)
    torch.cuda.synchronize()
    ref, absum = dp.oracle()
    _gpu.assert_parity(y, ref, absum, f"split-K S={S} M={M} bits={bits} G={G}")
    assert torch.equal(y, y2), "split-K rerun is not bitwise identical"


def test_split_equals_groups():
    """split_k = K/G: every slice holds exactly one group."""
    bits, G, K, N, M = 4, 32, 8 * 32, 70, 3
    dp = _gpu.DeviceProblem(qmm_inputs.make_problem(seed=2, M=M, K=K, N=N, bits=bits, G=G))
    y = _gpu.lib().qmm_forward_splitk(dp.x, dp.wq, dp.s, dp.b, bits, G, K // G)
    torch.cuda.synchronize()
    ref, absum = dp.oracle()
    _gpu.assert_parity(y, ref, absum, "split = K/G")


def test_splitk_rejects_small_workspace():
    qmm = _gpu.lib()
    bits, G, K, N, M = 4, 32, 512, 64, 2
    dp = _gpu.DeviceProblem(qmm_inputs.make_problem(seed=4, M=M, K=K, N=N, bits=bits, G=G))
    ws = torch.empty(10, dtype=torch.float32, device=dp.x.device)
    with pytest.raises(qmm.QmmError) as e:
        qmm.qmm_forward_splitk(dp.x, dp.wq, dp.s, dp.b, bits, G, 4, workspace=ws)
    assert e.value.code == -6
