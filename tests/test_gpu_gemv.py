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


def _topk_case(m, n, k, seed, dup_cols=(), one_hot=False, max_m=16, flags=0, negative=False, topk=10):
    """Router-style inputs; dup_cols lists (src, dst) weight rows to duplicate
    (equal logits -> ties); one_hot makes A rows one-hot so logits are exact;
    negative sets every weight's sign bit."""
    W = WL.gen_matrix((n, k), "bf16", ("normal", 0.02), seed)
    if negative:
        W = W | np.uint16(0x8000)
    for src, dst in dup_cols:
        W[dst] = W[src]
    if one_hot:
        A = np.zeros((m, k), np.uint16)
        for r in range(m):
            A[r, (7 * r) % k] = 0x3F80  # bf16 1.0
    else:
        A = WL.gen_matrix((m, k), "bf16", ("normal", 1.0), seed + 1)
    logits, idx, val = sk.gemv_topk(to_dev(A, "bf16"), to_dev(W, "bf16"), topk=topk, max_m=max_m,
                                    flags=flags)
    torch.cuda.synchronize()
    lg = logits.cpu().numpy()
    ref = oracle.mm(A, "bf16", W, "bf16")
    assert rel_err(lg, ref) <= REL_TOL
    oi, ov = oracle.topk(lg.astype(np.float64), topk)
    assert np.array_equal(idx.cpu().numpy(), oi)
    assert np.array_equal(val.cpu().numpy().view(np.uint32), ov.astype(np.float32).view(np.uint32))
    return lg, idx.cpu().numpy()


@pytest.mark.parametrize("m", [1, 3, 8, 16])
def test_topk_ties_break_to_lower_index(m):
    # many duplicated weight rows: equal logits everywhere in the top of the list
    dups = [(5, 200), (5, 17), (40, 41), (40, 3), (100, 250), (100, 101), (9, 10)]
    lg, idx = _topk_case(m, 256, 5120, 301, dup_cols=dups)
    for src, dst in dups:
        assert np.array_equal(lg[:, src].view(np.uint32), lg[:, dst].view(np.uint32))


def test_topk_exact_logits_one_hot():
    # one-hot rows: logits are weight values exactly, so fp32 cannot reorder them
    _topk_case(4, 256, 5120, 311, one_hot=True)


@pytest.mark.parametrize("n", [64, 100, 128, 500, 512, 1000, 1024])
def test_topk_negative_logits_every_register_width(n):
    # all logits negative (the order keys flip their magnitude bits), exact
    # (one-hot rows), for each number of register slots per lane (1 .. 16)
    _, idx = _topk_case(3, n, 256, 341 + n, one_hot=True, negative=True, dup_cols=((1, n - 1),))


@pytest.mark.parametrize("n", [10, 130, 1100, 1500])
def test_topk_rows_beyond_register_cache(n):
    # n > 1024 exercises the re-read path of the top-k; n = 10 takes every column
    _topk_case(5, n, 512, 321 + n)


@pytest.mark.parametrize("n,topk", [(1, 1), (32, 32), (256, 32), (1100, 32), (256, 1)])
def test_topk_sizes_at_the_limits(n, topk):
    # one expert; topk = n; the largest topk in a register-cached row and on
    # the re-read path; topk = 1
    print(f"top-k n={n} topk={topk}", flush=True)
    _topk_case(4, n, 1024, 351 + n + topk, topk=topk, dup_cols=((0, n - 1),) if n > 2 else ())


def test_topk_on_gemm_path():
    # m > 16: the MFMA GEMM writes the logits, a second launch takes the top-k
    _topk_case(20, 256, 5120, 331, max_m=20)


def test_repeated_calls_leave_counters_ready():
    """k = 16384 splits k across workgroups: the workspace counters must be back
    at zero after every call, so repeated calls (with different m) reproduce
    their first results bit for bit."""
    n, k = 256, 16384
    W = to_dev(WL.gen_matrix((n, k), "bf16", ("normal", 0.02), 501), "bf16")
    A = to_dev(WL.gen_matrix((16, k), "bf16", ("normal", 1.0), 502), "bf16")
    plan = sk.Plan(n, k, 16, sk.BF16, sk.BF16, sk.F32)
    ws = sk.new_workspace(plan, A.device)
    assert ws is not None and "split_reduce=global" in plan.info(1)
    outs = []
    for rep in range(4):
        for m in (16, 3, 1):
            lg = torch.empty((m, n), dtype=torch.float32, device="cuda")
            idx = torch.empty((m, 10), dtype=torch.int32, device="cuda")
            val = torch.empty((m, 10), dtype=torch.float32, device="cuda")
            plan.run_topk(m, A[:m], W, lg, idx, val, 10, workspace=ws)
            outs.append((m, lg, idx))
    torch.cuda.synchronize()
    # the counters (the first 256 bytes, before the partials: 64 column
    # ranges of 4 columns) are back at zero
    head = ws[:256].cpu().numpy()
    assert not np.any(head), head[np.nonzero(head)][:8]
    first = {}
    for m, lg, idx in outs:
        if m not in first:
            first[m] = (lg.cpu().numpy().view(np.uint32), idx.cpu().numpy())
        else:
            assert np.array_equal(lg.cpu().numpy().view(np.uint32), first[m][0])
            assert np.array_equal(idx.cpu().numpy(), first[m][1])
    # and row invariance holds through the top-k path too
    l16, l1 = first[16][0], first[1][0]
    assert np.array_equal(l16[:1], l1)


def test_mm_run_equals_gemv_topk_logits():
    wl = WL.WORKLOADS["router_topk"]
    W = to_dev(WL.gen_w(wl), "bf16")
    A = to_dev(WL.gen_a(wl, 16), "bf16")
    for m in (1, 7, 16):
        C = sk.mm(A[:m], W, out_dtype=torch.float32, max_m=16)
        lg, _, _ = sk.gemv_topk(A[:m], W, topk=10, max_m=16)
        torch.cuda.synchronize()
        assert np.array_equal(C.cpu().numpy().view(np.uint32), lg.cpu().numpy().view(np.uint32))


@pytest.mark.parametrize("n,k", [(300, 1032), (1001, 2048), (256, 16384), (37, 4096)])
def test_split_shapes_parity_and_row_invariance(n, k):
    """k splits summed inside a workgroup (k = 1032: 3 splits, the last ending
    inside a chunk slot; 2048 and 4096: splits whose chunk slots cover k
    exactly, the kernels without tail handling) and across workgroups
    (k = 16384: 16 splits), with ragged column ranges; every row at m = 16
    equals its m = 1 call bit for bit."""
    print(f"split shapes n={n} k={k}", flush=True)
    W = WL.gen_matrix((n, k), "f16", ("uniform", -0.05, 0.05), 401 + k)
    A = WL.gen_matrix((16, k), "f16", ("normal", 1.0), 402 + k)
    dW, dA = to_dev(W, "f16"), to_dev(A, "f16")
    plan = sk.Plan(n, k, 16, sk.F16, sk.F16, sk.F32)
    c16 = torch.empty((16, n), dtype=torch.float32, device="cuda")
    plan.run(16, dA, dW, c16)
    singles = []
    for r in range(16):
        c1 = torch.empty((1, n), dtype=torch.float32, device="cuda")
        plan.run(1, dA[r:r + 1], dW, c1)
        singles.append(c1)
    torch.cuda.synchronize()
    got = c16.cpu().numpy()
    ref = oracle.mm(A, "f16", W, "f16")
    assert rel_err(got, ref) <= REL_TOL
    assert np.all(np.abs(got - ref) <= _f32_bound(A, "f16", W, "f16"))
    single = torch.cat(singles).cpu().numpy().view(np.uint32)
    assert np.array_equal(got.view(np.uint32), single)


@pytest.mark.parametrize("m", [1, 6, 16])
@pytest.mark.parametrize("k", [1032, 16384])
def test_topk_with_split_shapes(m, k):
    # the top-k handoff after splits summed inside (k = 1032) and across
    # (k = 16384) workgroups
    print(f"topk split m={m} k={k}", flush=True)
    _topk_case(m, 300, k, 411 + k + m)


@pytest.mark.parametrize("name", ["router_topk", "q8_0_n512"])
def test_row_invariance_at_the_workload_shape(name):
    """Row r of every output at m = 2, 4, 8, 16 equals the m = 1 call on that
    row, bit for bit (the Strata PR #109 page, "What": the batched window's
    outputs are bit-identical to the per-token calls) -- at the router's
    own shape (256 x 5120 bf16, k split in five inside a workgroup; logits,
    top-10 indices and values) and at the Q8_0 GEMV's (512 x 2560, codes
    dequantised in the load, f16 out)."""
    wl = WL.WORKLOADS[name]
    A = WL.gen_a(wl, 16)
    W = WL.gen_w(wl)
    dA = to_dev(A, wl.a_kind)
    if wl.w_kind == "q8_0":
        dW, dS = to_dev(W[0], "i8"), to_dev(W[1], "f16")
        plan = sk.Plan(wl.n, wl.k, 16, sk.F16, sk.Q8_0, sk.F16)
    else:
        dW, dS = to_dev(W, wl.w_kind), None
        plan = sk.Plan(wl.n, wl.k, 16, sk.BF16, sk.BF16, sk.F32)
    cdt = torch.float16 if wl.w_kind == "q8_0" else torch.float32

    def call(m, rows):
        C = torch.empty((m, wl.n), dtype=cdt, device="cuda")
        if wl.topk:
            idx = torch.empty((m, wl.topk), dtype=torch.int32, device="cuda")
            val = torch.empty((m, wl.topk), dtype=torch.float32, device="cuda")
            plan.run_topk(m, rows, dW, C, idx, val, wl.topk)
            return C, idx, val
        plan.run(m, rows, dW, C, scales=dS)
        return (C,)

    print(f"row invariance {name}: {plan.info(1)} | {plan.info(16)}", flush=True)
    singles = [call(1, dA[r:r + 1]) for r in range(16)]
    torch.cuda.synchronize()
    ref = [torch.cat([s[i] for s in singles]).contiguous() for i in range(len(singles[0]))]
    ref = [t.view(torch.int16 if t.dtype == torch.float16 else torch.int32).cpu().numpy() for t in ref]
    for m in (2, 4, 8, 16):
        outs = call(m, dA[:m])
        torch.cuda.synchronize()
        for i, t in enumerate(outs):
            got = t.contiguous().view(torch.int16 if t.dtype == torch.float16 else torch.int32).cpu().numpy()
            assert np.array_equal(got, ref[i][:m]), (name, m, i)


def _check_topk_against_fp64(ref, bound, gpu_idx, topk):
    """The bounded check of the top-k against fp64 logits.  Each GPU logit is
    within E (the row's largest fp32 summation bound) of its fp64 value, so
    the GPU's t-th pick has an fp64 value within 2E of the t-th largest fp64
    value, and where that value stands more than 2E away from both of its
    neighbours in fp64 order the pick is exactly its index."""
    m, n = ref.shape
    for r in range(m):
        E = float(np.max(bound[r]))
        order = np.lexsort((np.arange(n), -ref[r]))  # value desc, index asc
        s = ref[r][order]
        for t in range(topk):
            prev_gap = s[t - 1] - s[t] if t > 0 else np.inf
            next_gap = s[t] - s[t + 1] if t + 1 < n else np.inf
            g = int(gpu_idx[r, t])
            if min(prev_gap, next_gap) > 2 * E:
                assert g == int(order[t]), (r, t, g, int(order[t]))
            else:
                assert abs(ref[r][g] - s[t]) <= 2 * E, (r, t, g)


@pytest.mark.parametrize("m", [1, 5, 16])
def test_router_topk_against_fp64_logits(m):
    """Top-10 of the router workload against the oracle's fp64 logits (not
    the GPU's own): indices agree except among fp64 values closer than the
    rigorous fp32 summation bound."""
    wl = WL.WORKLOADS["router_topk"]
    W = WL.gen_w(wl)
    A = WL.gen_a(wl, 16)[:m]
    _, idx, _ = sk.gemv_topk(to_dev(A, "bf16"), to_dev(W, "bf16"), topk=10, max_m=16)
    torch.cuda.synchronize()
    ref = oracle.mm(A, "bf16", W, "bf16")
    _check_topk_against_fp64(ref, _f32_bound(A, "bf16", W, "bf16"), idx.cpu().numpy(), 10)


def test_topk_against_fp64_with_near_ties():
    """Near-ties in fp64 (weight rows that differ in one low bit) may come out
    in either order but must stay within the bound; exact duplicates keep
    the lower index first."""
    n, k, m = 256, 5120, 8
    W = WL.gen_matrix((n, k), "bf16", ("normal", 0.02), 361)
    for src, dst in ((3, 200), (50, 51), (77, 12)):
        W[dst] = W[src]
        W[dst, 0] ^= np.uint16(1)  # one ulp of one weight: a near-tie
    W[90] = W[91]                  # an exact tie
    A = WL.gen_matrix((m, k), "bf16", ("normal", 1.0), 362)
    _, idx, _ = sk.gemv_topk(to_dev(A, "bf16"), to_dev(W, "bf16"), topk=10, max_m=16)
    torch.cuda.synchronize()
    ref = oracle.mm(A, "bf16", W, "bf16")
    _check_topk_against_fp64(ref, _f32_bound(A, "bf16", W, "bf16"), idx.cpu().numpy(), 10)


@pytest.mark.parametrize("kind", ["gemv_global_split", "gemm_split_launch"])
def test_two_streams_at_once_use_their_own_workspaces(kind):
    """The binding's Plan hands each (device, stream) its own workspace, so
    runs of one plan on two streams in flight at once do not share arrival
    counters or partial sums: each stream's results equal the serial calls'
    bits, and every workspace's counters are back at zero afterwards."""
    if kind == "gemv_global_split":
        n, k, m, flags, cdt = 256, 16384, 16, 0, torch.float32
    else:
        n, k, m, flags, cdt = 96, 2560, 300, sk.GEMM_SPLIT_LAUNCH, torch.float16
    W = to_dev(WL.gen_matrix((n, k), "f16", ("normal", 0.02), 811), "f16")
    As = [to_dev(WL.gen_matrix((m, k), "f16", ("normal", 1.0), 812 + i), "f16") for i in range(2)]
    plan = sk.Plan(n, k, m, sk.F16, sk.F16, sk.F32 if cdt == torch.float32 else sk.F16, flags=flags)
    print(f"two streams {kind}: {plan.info(m)}", flush=True)
    serial = []
    for A in As:
        C = torch.empty((m, n), dtype=cdt, device="cuda")
        plan.run(m, A, W, C)
        serial.append(C)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [[torch.empty((m, n), dtype=cdt, device="cuda") for _ in range(6)] for _ in range(2)]
    for rep in range(6):  # interleaved enqueues: both streams have work in flight together
        for i in range(2):
            plan.run(m, As[i], W, outs[i][rep], stream=streams[i])
    torch.cuda.synchronize()
    ibits = torch.int32 if cdt == torch.float32 else torch.int16
    for i in range(2):
        ref = serial[i].view(ibits).cpu().numpy()
        for rep in range(6):
            assert np.array_equal(outs[i][rep].view(ibits).cpu().numpy(), ref), (i, rep)
        ws = plan.workspace(As[i].device, streams[i])
        assert ws is not None and ws.data_ptr() != plan.workspace(As[i].device, streams[1 - i]).data_ptr()
        if kind == "gemv_global_split":
            head = ws[:256].cpu().numpy()  # the arrival counters
            assert not np.any(head), head[np.nonzero(head)][:8]


_CODES = {"f16": sk.F16, "bf16": sk.BF16, "f32": sk.F32, "q2_0": sk.Q2_0}
_TORCH = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@pytest.mark.parametrize("akind,wkind,ckind,k", [
    ("bf16", "bf16", "f32", 5120),   # k split inside the workgroup (S = 5)
    ("f16", "f16", "f16", 512),      # unsplit k
    ("f32", "bf16", "bf16", 2048),   # fp32 rows rounded to bf16 as they load
    ("f16", "q2_0", "f16", 2560),    # a block-quantised weight
])
def test_row_groups_equal_single_row_calls(akind, wkind, ckind, k):
    """Eight columns fill a single workgroup, so the plan runs m rows as m
    workgroup rows of the one-row kernel.  A and C are strided (lda and ldc
    past the row), so each group's offsets are checked; every row must be
    its own m = 1 call bit for bit, and the oracle's product within 2e-3."""
    n, lda, ldc = 8, k + 24, 16   # every row pointer stays 16-byte aligned
    seed = 1400 + k
    if akind == "f32":
        A = WL.gen_matrix((16, k), "f32", ("normal", 1.0), seed)
        dA = torch.zeros((16, lda), dtype=torch.float32, device="cuda")
        dA[:, :k] = torch.from_numpy(A).cuda()
    else:
        A = WL.gen_matrix((16, k), akind, ("normal", 1.0), seed)
        dA = torch.zeros((16, lda), dtype=_TORCH[akind], device="cuda")
        dA[:, :k] = to_dev(A, akind)
    if wkind == "q2_0":
        qs, d = WL.gen_q2_0(n, k, seed + 1, seed + 2)
        dW, ds = to_dev(qs, "u8"), to_dev(d, "f16")
    else:
        W = WL.gen_matrix((n, k), wkind, ("normal", 0.02), seed + 1)
        dW, ds = to_dev(W, wkind), None
    plan = sk.Plan(n, k, 16, _CODES[akind], _CODES[wkind], {"f32": sk.F32, "f16": sk.F16, "bf16": sk.BF16}[ckind],
                   lda=lda, ldc=ldc)
    singles = torch.zeros((16, ldc), dtype=_TORCH[ckind], device="cuda")
    for r in range(16):
        plan.run(1, dA[r:r + 1], dW, singles[r:r + 1], scales=ds)
    for m in (2, 5, 16):
        info = plan.info(m)
        print(f"row groups {akind}/{wkind}/{ckind} k={k} m={m}: {info}", flush=True)
        assert f"row_groups={m} " in info, info
        C = torch.full((m, ldc), 7.0, dtype=_TORCH[ckind], device="cuda")
        plan.run(m, dA[:m], dW, C, scales=ds)
        torch.cuda.synchronize()
        assert np.array_equal(bits_of(C[:, :n]), bits_of(singles[:m, :n])), m
        assert np.all(C[:, n:].float().cpu().numpy() == 7.0), m   # nothing past column n
    if akind != "f32":
        got = singles[:, :n].float().cpu().numpy()
        ref = (oracle.mm(A, akind, qs, "q2_0", w_scales=d) if wkind == "q2_0"
               else oracle.mm(A, akind, W, wkind))
        assert rel_err(got, ref) <= REL_TOL


def test_row_groups_at_the_shard_shape_equal_single_row_calls():
    """608 x 896 (one GPU's share of the k = 896 weight under an 8-way column
    shard): the plan runs m rows as groups of 1, 2 or 4 rows (m = 2 .. 16;
    the 4-row kernel stages A in LDS).  A and C strided; every row at every
    m must be its own m = 1 call bit for bit."""
    wl = WL.WORKLOADS["gemv_k896_shard8"]
    n, k, lda, ldc = wl.n, wl.k, wl.k + 8, wl.n + 8
    A = WL.gen_a(wl, 16)
    dA = torch.zeros((16, lda), dtype=torch.float16, device="cuda")
    dA[:, :k] = to_dev(A, "f16")
    dW = to_dev(WL.gen_w(wl), "f16")
    plan = sk.Plan(n, k, 16, sk.F16, sk.F16, sk.F32, lda=lda, ldc=ldc)
    singles = torch.zeros((16, ldc), dtype=torch.float32, device="cuda")
    for r in range(16):
        plan.run(1, dA[r:r + 1], dW, singles[r:r + 1])
    grouped = 0
    for m in range(2, 17):
        info = plan.info(m)
        grouped += "row_groups=" in info
        print(f"shard m={m}: {info}", flush=True)
        C = torch.full((m, ldc), 7.0, dtype=torch.float32, device="cuda")
        plan.run(m, dA[:m], dW, C)
        torch.cuda.synchronize()
        assert np.array_equal(bits_of(C[:, :n]), bits_of(singles[:m, :n])), m
        assert np.all(C[:, n:].cpu().numpy() == 7.0), m
    assert grouped >= 6
    ref = oracle.mm(A, "f16", WL.gen_w(wl), "f16")
    assert rel_err(singles[:, :n].cpu().numpy(), ref) <= REL_TOL
