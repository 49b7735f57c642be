"""GPU parity of the MoE combine (Strata PR #109, "What": one combine launch
for the window's tokens) against the CPU oracle.

Bars: max|out - ref| / max|ref| <= 2e-3 for fp32 output, and per element the
bound of a chain of topk + 1 fp32 fused multiply-adds, (topk + 2) * 2^-24 *
sum |w * y| (+ |g * s|), plus the output's own rounding for bf16; a token's
row is the same bits at every m.
"""
import numpy as np
import pytest

import oracle
import workloads as WL
from conftest import REL_TOL, bits_of, rel_err, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
sk = pytest.importorskip("row_gemv_decode_amd")


def _dev(x, kind):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda() if kind == "f32" else to_dev(x, "bf16")


def _abs_rows(x, kind):
    return np.abs(x) if kind == "f32" else (np.asarray(x, np.uint16) & np.uint16(0x7FFF))


def _case(m, topk, d, seed, kind="f32", out="f32", shared=True):
    y, w, sh, g = WL.gen_combine(m, topk, d, seed, kind)
    odt = torch.float32 if out == "f32" else torch.bfloat16
    got = sk.moe_combine(_dev(y, kind), torch.from_numpy(w).cuda(),
                         _dev(sh, kind) if shared else None,
                         torch.from_numpy(g).cuda() if shared else None, out_dtype=odt)
    torch.cuda.synchronize()
    ref = oracle.moe_combine(y, w, sh if shared else None, g if shared else None, kind=kind)
    absum = oracle.moe_combine(_abs_rows(y, kind), np.abs(w), _abs_rows(sh, kind) if shared else None,
                               np.abs(g) if shared else None, kind=kind)
    ulp = 0.0 if out == "f32" else 2.0 ** -8
    bound = (topk + 2) * 2.0 ** -24 * absum * (1 + ulp) + ulp * np.abs(ref) + 1e-30
    res = got.float().cpu().numpy()
    assert np.all(np.abs(res - ref) <= bound)
    if out == "f32":
        assert rel_err(res, ref) <= REL_TOL
    return got


@pytest.mark.parametrize("m", WL.COMBINE["ms"])
@pytest.mark.parametrize("kind,out", [("f32", "f32"), ("bf16", "f32"), ("f32", "bf16"), ("bf16", "bf16")])
def test_combine_workload_parity(m, kind, out):
    print(f"combine m={m} rows={kind} out={out}", flush=True)
    _case(m, WL.COMBINE["topk"], WL.COMBINE["d"], 6000 + m, kind, out)


@pytest.mark.parametrize("m", [1, 16])
def test_combine_without_shared_expert(m):
    _case(m, WL.COMBINE["topk"], WL.COMBINE["d"], 6100 + m, shared=False)


def test_combine_row_invariance():
    # a token's row does not depend on how many tokens the call has
    topk, d = WL.COMBINE["topk"], WL.COMBINE["d"]
    y, w, sh, g = WL.gen_combine(16, topk, d, 6201)
    dy, dw, ds, dg = (torch.from_numpy(a).cuda() for a in (y, w, sh, g))
    full = sk.moe_combine(dy, dw, ds, dg)
    for m in (1, 5, 11):
        part = sk.moe_combine(dy[:m].contiguous(), dw[:m].contiguous(), ds[:m].contiguous(), dg[:m].contiguous())
        torch.cuda.synchronize()
        assert np.array_equal(bits_of(part), bits_of(full[:m])), m


@pytest.mark.parametrize("m,topk,d", [(1, 1, 8), (3, 32, 8200), (2, 9, 520), (70000, 1, 8)])
def test_combine_edge_shapes(m, topk, d):
    # one expert and one lane of columns; the largest topk over a ragged last
    # workgroup of columns; a topk past one group of eight rows; more tokens
    # than the grid's y dimension takes (the workgroups loop over tokens)
    print(f"combine edge m={m} topk={topk} d={d}", flush=True)
    _case(m, topk, d, 6300 + m + topk)


def _random_combine_cases(count=24, seed=2029):
    import random

    rng = random.Random(seed)
    kinds = (("f32", "f32"), ("bf16", "f32"), ("f32", "bf16"), ("bf16", "bf16"))
    return [(i, rng.randrange(1, 65), rng.randrange(1, 33), rng.randrange(8, 12289, 8), *kinds[i % 4],
             i % 3 != 2) for i in range(count)]


@pytest.mark.parametrize("i,m,topk,d,kind,out,shared", _random_combine_cases())
def test_combine_random_shapes(i, m, topk, d, kind, out, shared):
    # seeded random tokens, topk, width, row and output types, with and
    # without the shared expert
    print(f"combine random {i}: m={m} topk={topk} d={d} rows={kind} out={out} shared={shared}", flush=True)
    _case(m, topk, d, 6400 + i, kind, out, shared)
