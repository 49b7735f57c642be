"""GPU parity of the Q2_0-style 2-bit block format (its definition: the
oracle's dequant_q2_0; the Q2_0 runs the Strata PR #109 page names in
"Measured" do not define it, so the format is fixed there) in every path
that reads it: the standalone dequant bitwise against the oracle for every
finite scale and code; the fused GEMV and GEMM against the oracle's
fp64 product within 2e-3, and bitwise equal to the f16 path on the
standalone-dequantised weight; row invariance in the GEMV regime; every GEMM
tile, M and launch shape giving the same bits."""
import numpy as np
import pytest

import oracle
import workloads as WL
from conftest import REL_TOL, bits_of, rel_err, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
sk = pytest.importorskip("row_gemv_decode_amd")


def _bound(A, qs, d):
    k = A.shape[1]
    return (k + 2) * 2.0 ** -24 * oracle.mm(A, "f16", qs, "q2_0", w_scales=d, absolute=True) + 1e-30


def test_q2_dequant_exhaustive_bitwise():
    """Every finite f16 scale x every 2-bit code, in each of the four bit
    positions of a byte."""
    d_all = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    d_all = d_all[((d_all >> 10) & 0x1F) != 0x1F]
    # byte b of a block holds codes b, b+1, b+2, b+3 (mod 4) from its lowest bits up
    byte = np.array([0xE4, 0x39, 0x4E, 0x93] * 2, np.uint8)
    n = d_all.size
    packed = np.broadcast_to(byte, (n, 8)).copy()
    packed = np.tile(packed, (1, 8))                      # 8 blocks of 32 per row
    d = np.repeat(d_all[:, None], 8, axis=1).copy()
    out = sk.dequant_q2_0(to_dev(packed, "u8"), to_dev(d, "f16"))
    torch.cuda.synchronize()
    ref = oracle.dequant_q2_0(packed, d)
    got = bits_of(out)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, [(hex(d[i, 0]), hex(got[i, j]), hex(ref[i, j])) for i, j in bad[:5]]


def _inputs(M, N, K, seed):
    A = WL.gen_matrix((M, K), "f16", ("normal", 1.0), seed)
    qs, d = WL.gen_q2_0(N, K, seed + 1, seed + 2)
    return A, qs, d


@pytest.mark.parametrize("m", [1, 4, 16])
def test_q2_gemv_workload_parity_and_fused_equals_unfused(m):
    wl = WL.WORKLOADS["q2_0_n512"]
    qs, d = WL.gen_w(wl)
    A = WL.gen_a(wl, 16)[:m]
    dq = (to_dev(qs, "u8"), to_dev(d, "f16"))
    print(f"q2_0_n512 gemv m={m}", flush=True)
    C = sk.mm(to_dev(A, "f16"), dq, out_dtype=torch.float16, max_m=16)
    w16 = sk.dequant_q2_0(*dq)
    C2 = sk.mm(to_dev(A, "f16"), w16, out_dtype=torch.float16, max_m=16)
    torch.cuda.synchronize()
    ref = oracle.mm(A, "f16", qs, "q2_0", w_scales=d)
    assert rel_err(C.float().cpu().numpy(), ref) <= REL_TOL
    assert np.array_equal(bits_of(C), bits_of(C2))


def test_q2_gemv_row_invariance_at_the_workload_shape():
    wl = WL.WORKLOADS["q2_0_n512"]
    qs, d = WL.gen_w(wl)
    dA = to_dev(WL.gen_a(wl, 16), "f16")
    dq, ds = to_dev(qs, "u8"), to_dev(d, "f16")
    plan = sk.Plan(wl.n, wl.k, 16, sk.F16, sk.Q2_0, sk.F16)
    singles = []
    for r in range(16):
        c1 = torch.empty((1, wl.n), dtype=torch.float16, device="cuda")
        plan.run(1, dA[r:r + 1], dq, c1, scales=ds)
        singles.append(c1)
    single = bits_of(torch.cat(singles))
    for m in (2, 4, 8, 16):
        cm = torch.empty((m, wl.n), dtype=torch.float16, device="cuda")
        plan.run(m, dA[:m], dq, cm, scales=ds)
        torch.cuda.synchronize()
        assert np.array_equal(bits_of(cm), single[:m]), m


@pytest.mark.parametrize("n,k", [(300, 1056), (256, 16384), (7, 96)])
def test_q2_gemv_split_shapes(n, k):
    # k split inside a workgroup (1056: 3 splits of T = 1), across workgroups
    # (16384), and a ragged tiny shape; f32 out within the summation bound
    A, qs, d = _inputs(16, n, k, 801 + k)
    C = sk.mm(to_dev(A, "f16"), (to_dev(qs, "u8"), to_dev(d, "f16")), out_dtype=torch.float32, max_m=16)
    torch.cuda.synchronize()
    got = C.cpu().numpy()
    ref = oracle.mm(A, "f16", qs, "q2_0", w_scales=d)
    assert rel_err(got, ref) <= REL_TOL
    assert np.all(np.abs(got - ref) <= _bound(A, qs, d))


def test_q2_gemm_workload_full_size_and_fused_equals_unfused():
    wl = WL.WORKLOADS["q2_0_n512"]
    qs, d = WL.gen_w(wl)
    A = WL.gen_a(wl, max(wl.ms))
    dA = to_dev(A, "f16")
    dq = (to_dev(qs, "u8"), to_dev(d, "f16"))
    w16 = sk.dequant_q2_0(*dq)
    for M in (m for m in wl.ms if m > 16):
        print(f"q2_0 GEMM M={M}", flush=True)
        C = sk.mm(dA[:M], dq, out_dtype=torch.float16, max_m=max(wl.ms))
        C2 = sk.mm(dA[:M], w16, out_dtype=torch.float16, max_m=max(wl.ms))
        torch.cuda.synchronize()
        assert np.array_equal(bits_of(C), bits_of(C2)), M
        rows = np.arange(M) if M == max(wl.ms) else np.unique(np.r_[0, M - 1, np.arange(0, M, 32)])
        ref = oracle.mm(A[rows], "f16", qs, "q2_0", w_scales=d)
        assert rel_err(C.float().cpu().numpy()[rows], ref) <= REL_TOL, M


@pytest.mark.parametrize("M,N,K", [(150, 200, 544), (70, 65, 96), (40, 130, 2592), (300, 96, 2560)])
def test_q2_gemm_every_tile_bitwise(M, N, K):
    """On every tile (ragged row and column tiles; K % 64 == 32 gives an odd
    scale count and a half k-tile; N = 96 takes the plan's k chunks) the
    fused Q2_0 GEMM gives the bits of the same tile on the dequantised f16
    weights, and every tile gives the same bits, within the oracle's fp32
    summation bound."""
    A, qs, d = _inputs(M, N, K, 901 + K)
    dA = to_dev(A, "f16")
    dq = (to_dev(qs, "u8"), to_dev(d, "f16"))
    w16 = sk.dequant_q2_0(*dq)
    ref = oracle.mm(A, "f16", qs, "q2_0", w_scales=d)
    bound = _bound(A, qs, d)
    first = None
    for tid in range(len(sk.gemm_tiles())):
        print(f"q2_0 tile {tid} {sk.gemm_tiles()[tid]} M={M} N={N} K={K}", flush=True)
        C = sk.mm(dA, dq, out_dtype=torch.float32, tile_id=tid)
        C2 = sk.mm(dA, w16, out_dtype=torch.float32, tile_id=tid)
        torch.cuda.synchronize()
        got = C.cpu().numpy()
        assert np.array_equal(got.view(np.uint32), C2.cpu().numpy().view(np.uint32)), tid
        assert np.all(np.abs(got - ref) <= bound), tid
        if first is None:
            first = got.view(np.uint32).copy()
        assert np.array_equal(got.view(np.uint32), first), tid


def test_q2_gemm_launch_shapes_and_m_invariance():
    N, K = 512, 2560
    A, qs, d = _inputs(306, N, K, 991)
    dA = to_dev(A, "f16")
    dq, ds = to_dev(qs, "u8"), to_dev(d, "f16")
    outs = {}
    for flag in (sk.GEMM_SPLIT_LAUNCH, sk.GEMM_ONE_LAUNCH, sk.GEMM_FOLD_LAUNCH):
        plan = sk.Plan(N, K, 306, sk.F16, sk.Q2_0, sk.F32, flags=flag)
        ws = plan.workspace(dA.device)
        for M in (17, 100, 306):
            print(f"q2_0 flag={flag} M={M}: {plan.info(M)}", flush=True)
            C = torch.empty((M, N), dtype=torch.float32, device="cuda")
            plan.run(M, dA[:M], dq, C, scales=ds, workspace=ws)
            torch.cuda.synchronize()
            outs[(flag, M)] = C.cpu().numpy().view(np.uint32)
    for M in (17, 100, 306):
        for flag in (sk.GEMM_ONE_LAUNCH, sk.GEMM_FOLD_LAUNCH):
            assert np.array_equal(outs[(sk.GEMM_SPLIT_LAUNCH, M)], outs[(flag, M)]), (flag, M)
        assert np.array_equal(outs[(sk.GEMM_SPLIT_LAUNCH, M)], outs[(sk.GEMM_SPLIT_LAUNCH, 306)][:M]), M


@pytest.mark.parametrize("n,k", [(1, 32), (5, 32), (33, 64), (3, 2080)])
@pytest.mark.parametrize("m", [1, 3, 16])
def test_q2_gemv_small_and_ragged_shapes(n, k, m):
    """The smallest block count (k = 32: one scale per row, four chunks), a
    single column, a ragged column count and an odd scale count, against the
    oracle and bitwise against the f16 path on the dequantised weight."""
    A, qs, d = _inputs(m, n, k, 1201 + 7 * n + k + m)
    dq = (to_dev(qs, "u8"), to_dev(d, "f16"))
    print(f"q2_0 gemv n={n} k={k} m={m}", flush=True)
    C = sk.mm(to_dev(A, "f16"), dq, out_dtype=torch.float32, max_m=16)
    C2 = sk.mm(to_dev(A, "f16"), sk.dequant_q2_0(*dq), out_dtype=torch.float32, max_m=16)
    torch.cuda.synchronize()
    got = C.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), C2.cpu().numpy().view(np.uint32))
    ref = oracle.mm(A, "f16", qs, "q2_0", w_scales=d)
    assert np.all(np.abs(got - ref) <= _bound(A, qs, d))
