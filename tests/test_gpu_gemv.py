"""GPU parity of the multi-row GEMV path (m <= 16) against the CPU oracle.

Bars: max|C_gpu - C_ref| / max|C_ref| <= 2e-3 for floating outputs, and the
fp32-accumulation error bound k * 2^-24 * sum|a*w| per element (f32 out);
row invariance (row r at any m equals the m = 1 call) bit for bit.
"""
import numpy as np
import pytest

import oracle
import workloads as WL
from conftest import REL_TOL, bits_of, rel_err, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
sk = pytest.importorskip("row_gemv_decode_amd")


def _f32_bound(A, a_kind, W, w_kind, scales=None):
    k = A.shape[1]
    absum = oracle.mm(A, a_kind, W, w_kind, w_scales=scales, absolute=True)
    return (k + 2) * 2.0 ** -24 * absum + 1e-30


def _run(wl, m, out_dtype=torch.float32, flags=0):
    W = WL.gen_w(wl)
    A = WL.gen_a(wl, 16)[:m]
    dA = to_dev(A, wl.a_kind)
    if wl.w_kind == "q8_0":
        qs, d = W
        dW = (to_dev(qs, "i8"), to_dev(d, "f16"))
    else:
        dW = to_dev(W, wl.w_kind)
    C = sk.mm(dA, dW, out_dtype=out_dtype, flags=flags, max_m=16)
    torch.cuda.synchronize()
    return A, W, C


@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 8, 13, 16])
def test_gemv_k896_parity(m):
    wl = WL.WORKLOADS["gemv_k896"]
    print(f"gemv_k896 m={m}", flush=True)
    A, W, C = _run(wl, m)
    ref = oracle.mm(A, "f16", W, "f16")
    got = C.cpu().numpy().astype(np.float64)
    assert rel_err(got, ref) <= REL_TOL
    assert np.all(np.abs(got - ref) <= _f32_bound(A, "f16", W, "f16"))


def test_gemv_k896_row_invariance():
    wl = WL.WORKLOADS["gemv_k896"]
    W = to_dev(WL.gen_w(wl), "f16")
    A = to_dev(WL.gen_a(wl, 16), "f16")
    plan = sk.Plan(wl.n, wl.k, 16, sk.F16, sk.F16, sk.F32)
    singles = []
    for r in range(16):
        c1 = torch.empty((1, wl.n), dtype=torch.float32, device="cuda")
        plan.run(1, A[r:r + 1], W, c1)
        singles.append(c1)
    single = torch.cat(singles).cpu().numpy().view(np.uint32)
    for m in (2, 3, 4, 8, 16):
        cm = torch.empty((m, wl.n), dtype=torch.float32, device="cuda")
        plan.run(m, A[:m], W, cm)
        torch.cuda.synchronize()
        assert np.array_equal(cm.cpu().numpy().view(np.uint32), single[:m]), m


@pytest.mark.parametrize("m", [1, 2, 4, 8, 16])
def test_router_topk_parity(m):
    wl = WL.WORKLOADS["router_topk"]
    print(f"router_topk m={m}", flush=True)
    W = WL.gen_w(wl)
    A = WL.gen_a(wl, 16)[:m]
    logits, idx, val = sk.gemv_topk(to_dev(A, "bf16"), to_dev(W, "bf16"), topk=10, max_m=16)
    torch.cuda.synchronize()
    lg = logits.cpu().numpy()
    ref = oracle.mm(A, "bf16", W, "bf16")
    assert rel_err(lg, ref) <= REL_TOL
    assert np.all(np.abs(lg - ref) <= _f32_bound(A, "bf16", W, "bf16"))
    # exact: the GPU's top-k equals the oracle's top-k of the GPU's own logits
    oi, ov = oracle.topk(lg.astype(np.float64), 10)
    assert np.array_equal(idx.cpu().numpy(), oi)
    assert np.array_equal(val.cpu().numpy().view(np.uint32), ov.astype(np.float32).view(np.uint32))


def test_dequant_exhaustive_bitwise():
    """Every finite f16 scale x every int8 code, GPU against the oracle."""
    d_all = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    d_all = d_all[((d_all >> 10) & 0x1F) != 0x1F]
    codes = np.arange(-128, 128, dtype=np.int16).astype(np.int8)
    n = d_all.size
    qs = np.broadcast_to(codes, (n, 256)).copy()
    d = np.repeat(d_all[:, None], 8, axis=1).copy()
    out = sk.dequant_q8_0(to_dev(qs, "i8"), to_dev(d, "f16"))
    torch.cuda.synchronize()
    ref = oracle.dequant_q8_0(qs, d)
    got = bits_of(out)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, [(hex(d[i, 0]), int(qs[i, j]), hex(got[i, j]), hex(ref[i, j])) for i, j in bad[:5]]


@pytest.mark.parametrize("m", [1, 4, 16])
def test_q8_gemv_parity_and_fused_equals_unfused(m):
    wl = WL.WORKLOADS["q8_0_n512"]
    print(f"q8_0_n512 gemv m={m}", flush=True)
    A, (qs, d), C = _run(wl, m, out_dtype=torch.float16)
    ref = oracle.mm(A, "f16", qs, "q8_0", w_scales=d)
    got = C.float().cpu().numpy()
    assert rel_err(got, ref) <= REL_TOL
    w16 = sk.dequant_q8_0(to_dev(qs, "i8"), to_dev(d, "f16"))
    C2 = sk.mm(to_dev(A, "f16"), w16, out_dtype=torch.float16, max_m=16)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(C), bits_of(C2))
