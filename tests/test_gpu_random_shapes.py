"""GPU parity on seeded random shapes across every weight kind and both
paths (the multi-row GEMV for m <= 16, the MFMA GEMM above), against the
CPU oracle: ragged n (1 .. 700), k anywhere the formats allow (a multiple of
8, or of 32 for the block formats), f32 and f16 outputs.  Bars: 2e-3
max-normalised, the fp32-accumulation bound per element (plus the output's
own rounding), and in the GEMV regime row 0 equal to the m = 1 call, bit for
bit; strided A and C rows; the router step's top-k at random n, topk and m
with equal logits, bit for bit against the oracle's ranking."""
import random

import numpy as np
import pytest

import oracle
import workloads as WL
from conftest import REL_TOL, rel_err, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
sk = pytest.importorskip("row_gemv_decode_amd")

KINDS = ("f16", "bf16", "q8_0", "q4_0", "q2_0")


def _cases(count=60, seed=2026):
    rng = random.Random(seed)
    out = []
    for i in range(count):
        kind = KINDS[i % len(KINDS)]
        block = kind.startswith("q")
        k = rng.randrange(64, 3073, 32) if block else rng.randrange(8, 3073, 8)
        n = (rng.randrange(1, 4), rng.randrange(4, 129), rng.randrange(129, 701), rng.randrange(129, 701))[i % 4]
        m = rng.randrange(1, 17) if i % 2 == 0 else rng.randrange(17, 261)
        out_kind = "f32" if (i // 2) % 2 == 0 else "f16"
        out.append((i, kind, m, n, k, out_kind))
    return out


def _weight(kind, n, k, seed):
    if kind == "q8_0":
        qs, d = WL.gen_q8_0(n, k, seed, seed + 1)
        return (qs, d), (to_dev(qs, "i8"), to_dev(d, "f16"))
    if kind == "q4_0":
        qs, d = WL.gen_q4_0(n, k, seed, seed + 1)
        return (qs, d), (to_dev(qs, "u8"), to_dev(d, "f16"))
    if kind == "q2_0":
        qs, d = WL.gen_q2_0(n, k, seed, seed + 1)
        return (qs, d), (to_dev(qs, "u8"), to_dev(d, "f16"))
    W = WL.gen_matrix((n, k), kind, ("uniform", -0.05, 0.05), seed)
    return W, to_dev(W, kind)


@pytest.mark.parametrize("i,kind,m,n,k,out_kind", _cases())
def test_random_shape_parity(i, kind, m, n, k, out_kind):
    print(f"random shape {i}: {kind} m={m} n={n} k={k} out={out_kind}", flush=True)
    a_kind = "bf16" if kind == "bf16" else "f16"
    A = WL.gen_matrix((m, k), a_kind, ("normal", 1.0), 7000 + i)
    W, dW = _weight(kind, n, k, 7100 + 3 * i)
    dA = to_dev(A, a_kind)
    odt = torch.float32 if out_kind == "f32" else torch.float16
    max_m = max(m, 16)
    C = sk.mm(dA, dW, out_dtype=odt, max_m=max_m)
    single = sk.mm(dA[:1], dW, out_dtype=odt, max_m=max_m) if 1 < m <= 16 else None
    torch.cuda.synchronize()
    got = C.float().cpu().numpy()
    if kind.startswith("q"):
        qs, d = W
        ref = oracle.mm(A, a_kind, qs, kind, w_scales=d)
        absum = oracle.mm(A, a_kind, qs, kind, w_scales=d, absolute=True)
    else:
        ref = oracle.mm(A, a_kind, W, kind)
        absum = oracle.mm(A, a_kind, W, kind, absolute=True)
    bound = (k + 2) * 2.0 ** -24 * absum + 1e-30
    if out_kind == "f16":
        bound = bound * (1 + 2.0 ** -11) + 2.0 ** -11 * np.abs(ref) + 2.0 ** -24
    assert rel_err(got, ref) <= REL_TOL
    worst = np.argmax(np.abs(got - ref) - bound)
    assert np.all(np.abs(got - ref) <= bound), (np.unravel_index(worst, got.shape), got.flat[worst],
                                                ref.flat[worst], bound.flat[worst])
    if single is not None:
        row0 = C[:1].contiguous().view(torch.int16 if out_kind == "f16" else torch.int32)
        one = single.contiguous().view(torch.int16 if out_kind == "f16" else torch.int32)
        assert torch.equal(row0, one)


def _strided_cases(count=20, seed=2027):
    rng = random.Random(seed)
    out = []
    for i in range(count):
        kind = ("f16", "bf16", "q8_0")[i % 3]
        block = kind.startswith("q")
        k = rng.randrange(64, 2049, 32) if block else rng.randrange(8, 2049, 8)
        lda = k + 8 * rng.randrange(1, 9)          # rows stay 16-byte aligned
        n = (rng.randrange(1, 40), rng.randrange(40, 600))[i % 2]
        ldc = n + rng.randrange(1, 13)
        m = rng.randrange(1, 17) if i % 2 == 0 else rng.randrange(17, 200)
        out.append((i, kind, m, n, k, lda, ldc))
    return out


@pytest.mark.parametrize("i,kind,m,n,k,lda,ldc", _strided_cases())
def test_random_strided_shape_parity(i, kind, m, n, k, lda, ldc):
    """A rows at a stride lda > k and C rows at ldc > n (f32): the product
    meets the oracle and the columns past n keep their sentinel."""
    print(f"random strided {i}: {kind} m={m} n={n} k={k} lda={lda} ldc={ldc}", flush=True)
    a_kind = "bf16" if kind == "bf16" else "f16"
    Afull = WL.gen_matrix((m, lda), a_kind, ("normal", 1.0), 7500 + i)
    A = np.ascontiguousarray(Afull[:, :k])
    W, dW = _weight(kind, n, k, 7600 + 3 * i)
    code = {"f16": sk.F16, "bf16": sk.BF16, "q8_0": sk.Q8_0}[kind]
    plan = sk.Plan(n, k, max(m, 16), sk.BF16 if a_kind == "bf16" else sk.F16, code, sk.F32, lda=lda, ldc=ldc)
    C = torch.full((m, ldc), -7.0, dtype=torch.float32, device="cuda")
    if kind.startswith("q"):
        plan.run(m, to_dev(Afull, a_kind), dW[0], C, scales=dW[1])
    else:
        plan.run(m, to_dev(Afull, a_kind), dW, C)
    torch.cuda.synchronize()
    out = C.cpu().numpy()
    assert np.all(out[:, n:] == -7.0)
    got = out[:, :n]
    if kind.startswith("q"):
        ref = oracle.mm(A, a_kind, W[0], kind, w_scales=W[1])
        absum = oracle.mm(A, a_kind, W[0], kind, w_scales=W[1], absolute=True)
    else:
        ref = oracle.mm(A, a_kind, W, kind)
        absum = oracle.mm(A, a_kind, W, kind, absolute=True)
    assert rel_err(got, ref) <= REL_TOL
    assert np.all(np.abs(got - ref) <= (k + 2) * 2.0 ** -24 * absum + 1e-30)


def _topk_cases(count=30, seed=2028):
    rng = random.Random(seed)
    out = []
    for i in range(count):
        n = (rng.randrange(1, 65), rng.randrange(65, 1025), rng.randrange(1025, 1501))[i % 3]
        topk = rng.randrange(1, min(32, n) + 1)
        m = rng.randrange(1, 17)
        k = rng.randrange(8, 6145, 8)
        out.append((i, m, n, k, topk))
    return out


@pytest.mark.parametrize("i,m,n,k,topk", _topk_cases())
def test_random_router_topk(i, m, n, k, topk):
    """gemv_topk at random n (register and re-reading top-k paths), topk, m
    and k, with duplicated weight rows (equal logits): the logits meet the
    oracle, and the indices and values are the oracle's top-k of the GPU's
    own logits (value descending, ties to the lower column), bit for bit."""
    print(f"random top-k {i}: m={m} n={n} k={k} topk={topk}", flush=True)
    rng = np.random.default_rng(7800 + i)
    W = WL.gen_matrix((n, k), "bf16", ("normal", 0.02), 7900 + i)
    for _ in range(n // 8):
        src, dst = rng.integers(0, n, size=2)
        W[dst] = W[src]
    A = WL.gen_matrix((m, k), "bf16", ("normal", 1.0), 8000 + i)
    logits, idx, val = sk.gemv_topk(to_dev(A, "bf16"), to_dev(W, "bf16"), topk=topk, max_m=16)
    torch.cuda.synchronize()
    lg = logits.cpu().numpy()
    assert rel_err(lg, oracle.mm(A, "bf16", W, "bf16")) <= REL_TOL
    oi, ov = oracle.topk(lg.astype(np.float64), topk)
    assert np.array_equal(idx.cpu().numpy(), oi)
    assert np.array_equal(val.cpu().numpy().view(np.uint32), ov.astype(np.float32).view(np.uint32))
