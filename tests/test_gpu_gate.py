"""GPU parity of the window-row cast and the scalar gate (Strata PR #109,
"What": the bf16 cast of the window's fp32 rows in one call; the shared
expert's scalar gate, a multi-row GEMV followed by a sigmoid, here applied as
the GEMV stores) against the CPU oracle, and of the cast fused into the GEMV's
A load (one launch) against the cast launch followed by the bf16 GEMV.

Bars: the cast is bitwise equal to the oracle's round-to-nearest-even; the
gate meets max|g - g_ref| / max|g_ref| <= 2e-3 and an element-wise bound (the
sigmoid's slope is at most 1/4, so the logit's fp32 bound shrinks by 4, plus
the fp32 evaluation of the sigmoid); the sigmoid epilogue agrees with the
fp64 sigmoid of the same call's own fp32 logits to a few units in the last
place; row invariance holds bit for bit.
"""
import numpy as np
import pytest

import oracle
import workloads as WL
from conftest import REL_TOL, bits_of, rel_err, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
sk = pytest.importorskip("row_gemv_decode_amd")

EVAL = 2.0 ** -21  # fp32 evaluation of 1 / (1 + e^-x): a few ulp of a value <= 1


def _f32_values():
    rng = np.random.default_rng(901)
    specials = np.array([
        0.0, -0.0, 1.0, 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -20, -(1 + 2.0 ** -8),
        2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -134, 2.0 ** -126 - 2.0 ** -134, 1e-45,
        (2 - 2.0 ** -7) * 2.0 ** 127, (2 - 2.0 ** -8) * 2.0 ** 127, 3.0e38, -3.0e38,
    ], dtype=np.float64).astype(np.float32)
    normal = rng.normal(0, 1, 4000).astype(np.float32)
    wide = (np.ldexp(rng.random(4000) + 0.5, rng.integers(-140, 128, 4000)) *
            rng.choice([-1, 1], 4000)).astype(np.float32)
    raw = rng.integers(0, 2 ** 32, 4000, dtype=np.uint64).astype(np.uint32)
    raw = raw[((raw >> 23) & 0xFF) != 0xFF].view(np.float32)  # finite bit patterns
    return np.concatenate([specials, normal, wide, raw])


@pytest.mark.parametrize("count", [1, 7, 8, 9, 1000, 16 * 5120, 16 * 5120 + 3])
def test_cast_bitwise_equals_oracle(count):
    print(f"cast count={count}", flush=True)
    vals = _f32_values()
    x = np.resize(vals, count).astype(np.float32)
    dx = torch.from_numpy(x).cuda()
    out = sk.cast_f32_bf16(dx)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(out), oracle.cast_bf16(x))


def _gate_case(m, n, k, seed, max_m=16):
    A = WL.gen_matrix((m, k), "f32", ("normal", 1.0), seed)
    W = WL.gen_matrix((n, k), "bf16", ("normal", 0.02), seed + 1)
    g = sk.gate(torch.from_numpy(A).cuda(), to_dev(W, "bf16"), max_m=max_m)
    torch.cuda.synchronize()
    return A, W, g.cpu().numpy()


def _check_gate(A, W, got):
    ref = oracle.gate(A, W)
    assert rel_err(got, ref) <= REL_TOL
    A16 = oracle.cast_bf16(A)
    k = A.shape[1]
    bound = (k + 2) * 2.0 ** -24 * oracle.mm(A16, "bf16", W, "bf16", absolute=True) / 4 + EVAL
    assert np.all(np.abs(got - ref) <= bound)


@pytest.mark.parametrize("m", [1, 2, 5, 8, 16])
def test_scalar_gate_parity(m):
    # the gate workload: n = 1, the router's k = 5120 (k split in-block)
    wl = WL.WORKLOADS["scalar_gate"]
    print(f"scalar gate m={m}", flush=True)
    A = WL.gen_a(wl, 16)[:m]
    W = WL.gen_w(wl)
    g = sk.gate(torch.from_numpy(np.ascontiguousarray(A)).cuda(), to_dev(W, "bf16"), max_m=16)
    torch.cuda.synchronize()
    _check_gate(A, W, g.cpu().numpy())


@pytest.mark.parametrize("n,k", [(1, 512), (7, 2048), (3, 16384)])
def test_gate_every_reduction_shape(n, k):
    # k = 512: one k range, the wave stores; k = 2048: splits summed in the
    # workgroup; k = 16384: splits summed by the last wave to arrive
    print(f"gate n={n} k={k}", flush=True)
    A, W, got = _gate_case(16, n, k, 911 + k)
    _check_gate(A, W, got)


def test_sigmoid_epilogue_matches_fp64_sigmoid_of_the_same_logits():
    # the same bf16 rows through the plain plan give the fp32 logits the gate
    # plan sums (same split, same order); its stores must be their sigmoid
    n, k, m = 5, 5120, 16
    A = WL.gen_matrix((m, k), "f32", ("normal", 3.0), 921)
    W = WL.gen_matrix((n, k), "bf16", ("normal", 0.05), 922)
    dA16 = sk.cast_f32_bf16(torch.from_numpy(A).cuda())
    dW = to_dev(W, "bf16")
    plain = sk.Plan(n, k, 16, sk.BF16, sk.BF16, sk.F32)
    gated = sk.Plan(n, k, 16, sk.BF16, sk.BF16, sk.F32, flags=sk.EPILOGUE_SIGMOID)
    logits = torch.empty((m, n), dtype=torch.float32, device="cuda")
    g = torch.empty((m, n), dtype=torch.float32, device="cuda")
    plain.run(m, dA16, dW, logits)
    gated.run(m, dA16, dW, g)
    torch.cuda.synchronize()
    lg = logits.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(lg)) > 4.0  # the sigmoid's curved part and its tails are exercised
    assert np.all(np.abs(g.cpu().numpy() - oracle.sigmoid(lg)) <= EVAL)


def test_gate_row_invariance():
    n, k = 1, 5120
    A = WL.gen_matrix((16, k), "f32", ("normal", 1.0), 931)
    W = to_dev(WL.gen_matrix((n, k), "bf16", ("normal", 0.02), 932), "bf16")
    dA = torch.from_numpy(A).cuda()
    full = sk.gate(dA, W, max_m=16).cpu().numpy().view(np.uint32)
    for m in (1, 3, 8, 15):
        part = sk.gate(dA[:m].contiguous(), W, max_m=16).cpu().numpy().view(np.uint32)
        assert np.array_equal(part, full[:m]), m


def test_gate_f16_output():
    n, k, m = 2, 5120, 4
    A = WL.gen_matrix((m, k), "f32", ("normal", 1.0), 941)
    W = WL.gen_matrix((n, k), "bf16", ("normal", 0.02), 942)
    dW = to_dev(W, "bf16")
    out16 = torch.empty((m, n), dtype=torch.float16, device="cuda")
    out32 = torch.empty((m, n), dtype=torch.float32, device="cuda")
    sk.gate(torch.from_numpy(A).cuda(), dW, out=out16)
    sk.gate(torch.from_numpy(A).cuda(), dW, out=out32)
    torch.cuda.synchronize()
    # the f16 gate is the f32 gate rounded to nearest even
    assert np.array_equal(bits_of(out16), bits_of(out32.to(torch.float16)))


# --- the cast fused into the GEMV's A load (plans with fp32 A) --------------
# Every reduction shape: k = 512 unsplit (A in registers for m < 4, staged in
# LDS for m >= 4), k = 2048 / 5120 split inside the workgroup, k = 16384 split
# across workgroups.  The fused launch must give the bits of the cast launch
# followed by the bf16 plan.

@pytest.mark.parametrize("n,k,m", [(1, 512, 3), (1, 512, 16), (7, 2048, 5), (1, 5120, 1), (1, 5120, 16),
                                   (3, 16384, 16)])
def test_fused_gate_equals_cast_then_gate(n, k, m):
    print(f"fused gate n={n} k={k} m={m}", flush=True)
    A = WL.gen_matrix((m, k), "f32", ("normal", 1.0), 951 + k + m)
    W = WL.gen_matrix((n, k), "bf16", ("normal", 0.02), 952 + k)
    dA, dW = torch.from_numpy(A).cuda(), to_dev(W, "bf16")
    fused = sk.gate(dA, dW, max_m=16)
    two = torch.empty_like(fused)
    plan = sk.Plan(n, k, 16, sk.BF16, sk.BF16, sk.F32, flags=sk.EPILOGUE_SIGMOID)
    plan.run(m, sk.cast_f32_bf16(dA), dW, two)
    torch.cuda.synchronize()
    assert "a=f32(" in sk.get_plan(n, k, 16, sk.F32, sk.BF16, sk.F32, sk.EPILOGUE_SIGMOID).info(m)
    assert np.array_equal(bits_of(fused), bits_of(two))
    _check_gate(A, W, fused.cpu().numpy())


@pytest.mark.parametrize("n,k", [(4864, 896), (256, 5120), (64, 16384)])
@pytest.mark.parametrize("out", ["f32", "f16", "bf16"])
def test_fp32_rows_gemv_equals_cast_then_gemv(n, k, out):
    odt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[out]
    code = {"f32": sk.F32, "f16": sk.F16, "bf16": sk.BF16}[out]
    A = WL.gen_matrix((16, k), "f32", ("normal", 1.0), 961 + k)
    W = WL.gen_matrix((n, k), "bf16", ("normal", 0.02), 962 + k)
    dA, dW = torch.from_numpy(A).cuda(), to_dev(W, "bf16")
    dA16 = sk.cast_f32_bf16(dA)
    fused_plan = sk.Plan(n, k, 16, sk.F32, sk.BF16, code)
    plain_plan = sk.Plan(n, k, 16, sk.BF16, sk.BF16, code)
    for m in (1, 4, 10, 11, 16):  # fused up to m = 10, cast launch above when k is split
        print(f"fp32 rows n={n} k={k} m={m} -> {out}: {fused_plan.info(m)}", flush=True)
        a = torch.empty((m, n), dtype=odt, device="cuda")
        b = torch.empty((m, n), dtype=odt, device="cuda")
        fused_plan.run(m, dA[:m], dW, a)
        plain_plan.run(m, dA16[:m], dW, b)
        torch.cuda.synchronize()
        assert np.array_equal(bits_of(a), bits_of(b)), m
    ref = oracle.mm(oracle.cast_bf16(A), "bf16", W, "bf16")
    if out != "bf16":
        assert rel_err(a.float().cpu().numpy(), ref) <= REL_TOL


def test_router_topk_from_fp32_rows():
    wl = WL.WORKLOADS["router_topk"]
    W = to_dev(WL.gen_w(wl), "bf16")
    A = WL.gen_matrix((16, wl.k), "f32", ("normal", 1.0), 971)
    dA = torch.from_numpy(A).cuda()
    for m in (1, 5, 16):
        print(f"router top-k from fp32 rows m={m}", flush=True)
        lg, idx, val = sk.gemv_topk(dA[:m], W, topk=10, max_m=16)
        lg2, idx2, val2 = sk.gemv_topk(sk.cast_f32_bf16(dA[:m]), W, topk=10, max_m=16)
        torch.cuda.synchronize()
        for x, y in ((lg, lg2), (idx, idx2), (val, val2)):
            assert np.array_equal(bits_of(x), bits_of(y)), m


def test_fp32_rows_strided():
    # lda > k: the fused load and the cast launch read rows at the stride
    n, k, lda = 256, 5120, 5128
    A = WL.gen_matrix((16, lda), "f32", ("normal", 1.0), 981)
    W = to_dev(WL.gen_matrix((n, k), "bf16", ("normal", 0.02), 982), "bf16")
    dA = torch.from_numpy(A).cuda()
    dA16 = sk.cast_f32_bf16(dA[:, :k].contiguous())
    fused_plan = sk.Plan(n, k, 16, sk.F32, sk.BF16, sk.F32, lda=lda)
    plain_plan = sk.Plan(n, k, 16, sk.BF16, sk.BF16, sk.F32)
    for m in (4, 16):
        print(f"fp32 rows lda={lda} m={m}: {fused_plan.info(m)}", flush=True)
        a = torch.empty((m, n), dtype=torch.float32, device="cuda")
        b = torch.empty((m, n), dtype=torch.float32, device="cuda")
        fused_plan.run(m, dA, W, a)
        plain_plan.run(m, dA16[:m], W, b)
        torch.cuda.synchronize()
        assert np.array_equal(bits_of(a), bits_of(b)), m


def _random_gate_cases(count=24, seed=2030):
    import random

    rng = random.Random(seed)
    return [(i, rng.randrange(1, 17), (rng.randrange(1, 4), rng.randrange(4, 300))[i % 2],
             rng.randrange(8, 12289, 8)) for i in range(count)]


@pytest.mark.parametrize("i,m,n,k", _random_gate_cases())
def test_gate_random_shapes(i, m, n, k):
    # seeded random rows, columns and k (fused cast, cast launch, row groups,
    # splits inside and across workgroups), each against the oracle; and row
    # 0 equal to the one-row call
    print(f"gate random {i}: m={m} n={n} k={k}", flush=True)
    A, W, got = _gate_case(m, n, k, 6600 + 2 * i)
    _check_gate(A, W, got)
    one = sk.gate(torch.from_numpy(A[:1]).cuda(), to_dev(W, "bf16"), max_m=16)
    torch.cuda.synchronize()
    assert np.array_equal(got[:1].view(np.uint32), one.cpu().numpy().view(np.uint32))
