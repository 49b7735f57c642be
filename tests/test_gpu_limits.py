"""The plan's size limits on the GPU: the GEMM at the largest k it accepts
(k = 2^20, where its 32-bit buffer offsets are largest), the GEMV beyond it
(k is unbounded there: thousands of k splits summed across workgroups), and a
GEMV over hundreds of thousands of columns.  Bars as everywhere:
max|C - ref| / max|ref| <= 2e-3 and the per-element fp32 summation bound."""
import numpy as np
import pytest

import oracle
import workloads as WL
from conftest import REL_TOL, rel_err, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
sk = pytest.importorskip("row_gemv_decode_amd")


def _check(m, n, k, seed, max_m, w_std=0.02):
    A = WL.gen_matrix((m, k), "f16", ("normal", 1.0), seed)
    W = WL.gen_matrix((n, k), "f16", ("normal", w_std), seed + 1)
    plan = sk.Plan(n, k, max_m, sk.F16, sk.F16, sk.F32)
    print(f"m={m} n={n} k={k}: {plan.info(m)}", flush=True)
    C = torch.empty((m, n), dtype=torch.float32, device="cuda")
    plan.run(m, to_dev(A, "f16"), to_dev(W, "f16"), C)
    torch.cuda.synchronize()
    got = C.cpu().numpy()
    ref = oracle.mm(A, "f16", W, "f16")
    absum = oracle.mm(A, "f16", W, "f16", absolute=True)
    assert np.all(np.abs(got - ref) <= (k + 2) * 2.0 ** -24 * absum + 1e-30)
    assert rel_err(got, ref) <= REL_TOL
    return plan


@pytest.mark.parametrize("m", [17, 40])
def test_gemm_at_the_largest_k(m):
    plan = _check(m, 70, 1 << 20, 1101 + m, max_m=64)
    assert "path=gemm" in plan.info(m)


@pytest.mark.parametrize("m", [1, 16])
def test_gemv_beyond_the_gemm_k_limit(m):
    # k = 2^21 + 64: 4097 k splits of 512 (the last one 64 long), summed across
    # workgroups by the last wave to arrive
    plan = _check(m, 5, (1 << 21) + 64, 1201 + m, max_m=16)
    assert "split_reduce=global" in plan.info(m)


def test_gemv_many_columns():
    # 300000 columns of k = 16: 37500 waves in 9375 workgroups
    plan = _check(3, 300000, 16, 1301, max_m=16, w_std=0.1)
    assert "path=gemv" in plan.info(3)
