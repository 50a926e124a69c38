"""The matrix-core rate probe (a measurement helper, not part of the method): every
work-group writes the same values, and each lane's value is the sum of its entries of
4 * iters accumulated 32x32x16 products.  The expected values are built on the CPU from
the documented operand layout of v_mfma_f32_32x32x16_bf16 (lane l holds row l%32 of A
and column l%32 of B at k = 8 (l/32) .. +7, and output rows 8 (v/4) + 4 (l/32) + v%4 of
column l%32), so the test also pins the layout every matrix-core kernel here relies on.
"""
import numpy as np
import pytest
import torch

import draft_kv_attention_amd as M

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    M.lib()


def _expected(iters):
    A = np.zeros((32, 16))
    B = np.zeros((16, 32))
    for l in range(64):
        for i in range(8):
            A[l % 32, 8 * (l // 32) + i] = 0.0078125 * ((l + i) & 7)
            B[8 * (l // 32) + i, l % 32] = 0.0078125 * ((3 * l + i) & 7)
    D = iters * (A @ B)
    out = np.zeros(64)
    for l in range(64):
        out[l] = 4 * sum(D[8 * (v // 4) + 4 * (l // 32) + v % 4, l % 32] for v in range(16))
    return out


@pytest.mark.parametrize("wgs,iters", [(1, 1), (4, 8), (300, 3)])
def test_mfma_rate_values_and_clocks(wgs, iters):
    out = torch.full((wgs * 256,), float("nan"), dtype=torch.float32, device="cuda")
    clocks = torch.zeros(2, dtype=torch.int64, device="cuda")
    M.mfma_rate(wgs, iters, out, clocks)
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(wgs * 4, 64)
    np.testing.assert_allclose(got, np.broadcast_to(_expected(iters), got.shape), rtol=1e-6, atol=0)
    c = clocks.cpu().tolist()
    assert c[0] > 0 and c[1] >= 0
