"""A deterministic spread of shapes through both paths, every weight kind and
output kind, against the CPU oracle: ragged n and k (k a multiple of 8, of 32
for Q8_0), every m of the GEMV regime and GEMM rows just past each tile size,
GEMV k splits inside and across workgroups, GEMM plans with and without k
chunks.  Bars as everywhere: max|C - ref| / max|ref| <= 2e-3 and, per element,
the fp32 summation bound (plus the output's own rounding for 16-bit C)."""
import numpy as np
import pytest

import oracle
import workloads as WL
from conftest import REL_TOL, rel_err, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
sk = pytest.importorskip("row_gemv_decode_amd")

OUT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
OUT_ULP = {"f32": 0.0, "f16": 2.0 ** -11, "bf16": 2.0 ** -8}

# (m, n, k, weight kind, output kind)
CASES = [
    (1, 1, 8, "f16", "f32"), (1, 7, 24, "bf16", "f32"), (2, 65, 136, "f16", "f16"),
    (3, 129, 1000, "bf16", "bf16"), (5, 300, 2056, "f16", "f32"), (7, 64, 4104, "bf16", "f32"),
    (9, 1001, 520, "f16", "f16"), (11, 33, 8200, "bf16", "f32"), (13, 96, 12288, "f16", "f32"),
    (16, 257, 3000, "bf16", "f16"), (16, 5000, 64, "f16", "f32"), (4, 8, 32, "q8_0", "f16"),
    (6, 100, 1056, "q8_0", "f32"), (16, 513, 2080, "q8_0", "f16"), (1, 2, 9216, "q8_0", "f32"),
    (17, 96, 264, "f16", "f16"), (31, 130, 1000, "bf16", "f32"), (33, 200, 2048, "f16", "f16"),
    (63, 64, 72, "f16", "f32"), (65, 1000, 520, "bf16", "bf16"), (95, 96, 2560, "f16", "f16"),
    (97, 4000, 136, "f16", "f32"), (127, 257, 1032, "bf16", "f32"), (129, 513, 256, "f16", "f16"),
    (191, 96, 3000, "f16", "f32"), (255, 300, 512, "bf16", "f16"), (257, 2050, 520, "f16", "f32"),
    (300, 7680, 200, "f16", "f16"), (33, 512, 2560, "q8_0", "f16"), (200, 96, 1024, "q8_0", "f32"),
    (130, 2000, 544, "q8_0", "bf16"),
    (4, 8, 32, "q4_0", "f16"), (6, 100, 1056, "q4_0", "f32"), (16, 513, 2080, "q4_0", "f16"),
    (1, 2, 9216, "q4_0", "f32"), (33, 512, 2560, "q4_0", "f16"), (200, 96, 1024, "q4_0", "f32"),
    (130, 2000, 544, "q4_0", "bf16"), (257, 70, 96, "q4_0", "f16"),
]


def _case(m, n, k, wk, ck, seed):
    a_kind = "bf16" if wk == "bf16" else "f16"
    A = WL.gen_matrix((m, k), a_kind, ("normal", 1.0), seed)
    if wk in ("q8_0", "q4_0"):
        qs, d = (WL.gen_q8_0 if wk == "q8_0" else WL.gen_q4_0)(n, k, seed + 1, seed + 2)
        dW = (to_dev(qs, "i8" if wk == "q8_0" else "u8"), to_dev(d, "f16"))
        ref = oracle.mm(A, "f16", qs, wk, w_scales=d)
        absum = oracle.mm(A, "f16", qs, wk, w_scales=d, absolute=True)
    else:
        W = WL.gen_matrix((n, k), wk, ("normal", 0.05), seed + 1)
        dW = to_dev(W, wk)
        ref = oracle.mm(A, a_kind, W, wk)
        absum = oracle.mm(A, a_kind, W, wk, absolute=True)
    C = sk.mm(to_dev(A, a_kind), dW, out_dtype=OUT[ck])
    torch.cuda.synchronize()
    return C.float().cpu().numpy(), ref, absum


@pytest.mark.parametrize("m,n,k,wk,ck", CASES)
def test_shape_parity(m, n, k, wk, ck):
    plan = sk.get_plan(n, k, m, sk.BF16 if wk == "bf16" else sk.F16,
                       {"f16": sk.F16, "bf16": sk.BF16, "q8_0": sk.Q8_0, "q4_0": sk.Q4_0}[wk], {"f32": sk.F32, "f16": sk.F16,
                                                                              "bf16": sk.BF16}[ck])
    print(f"m={m} n={n} k={k} {wk}->{ck}: {plan.info(m)}", flush=True)
    got, ref, absum = _case(m, n, k, wk, ck, 1000 + 7 * m + n)
    bound = (k + 2) * 2.0 ** -24 * absum * (1 + OUT_ULP[ck]) + OUT_ULP[ck] * np.abs(ref) + 1e-30
    assert np.all(np.abs(got - ref) <= bound)
    if ck != "bf16":
        assert rel_err(got, ref) <= REL_TOL
