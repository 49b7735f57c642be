"""GPU parity of the MFMA GEMM path (m >= 17) against the CPU oracle, and its
bitwise tile- and M-invariance (opus r35 track A, section 2: every tile of the
family gives the same bytes)."""
import numpy as np
import pytest

import oracle
import workloads as WL
from conftest import REL_TOL, bits_of, rel_err, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
sk = pytest.importorskip("row_gemv_decode_amd")

OUT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def _inputs(M, N, K, seed, kind="f16"):
    A = WL.gen_matrix((M, K), kind, ("normal", 1.0), seed)
    W = WL.gen_matrix((N, K), kind, ("normal", 0.02), seed + 1)
    return A, W


def _f32_bound(A, a_kind, W, w_kind, scales=None):
    k = A.shape[1]
    absum = oracle.mm(A, a_kind, W, w_kind, w_scales=scales, absolute=True)
    return (k + 2) * 2.0 ** -24 * absum + 1e-30


@pytest.mark.parametrize("M,N,K", [
    (17, 96, 2560), (150, 384, 2560), (306, 200, 512), (64, 64, 64), (33, 7680, 256),
    (40, 100, 520),   # K % 64 = 8: a partial last k-tile
    (200, 96, 72),    # one full and one partial k-tile
    (19, 33, 8),      # a single 8-wide chunk of k
    (257, 129, 136),  # every dimension one past a power of two
])
def test_gemm_parity_small(M, N, K):
    print(f"gemm M={M} N={N} K={K}", flush=True)
    A, W = _inputs(M, N, K, 100 + M)
    C = sk.mm(to_dev(A, "f16"), to_dev(W, "f16"), out_dtype=torch.float32)
    torch.cuda.synchronize()
    got = C.cpu().numpy()
    ref = oracle.mm(A, "f16", W, "f16")
    assert rel_err(got, ref) <= REL_TOL
    assert np.all(np.abs(got - ref) <= _f32_bound(A, "f16", W, "f16"))


@pytest.mark.parametrize("out", ["f32", "f16", "bf16"])
def test_gemm_bf16_parity_and_output_kinds(out):
    M, N, K = 90, 160, 328
    print(f"gemm bf16 -> {out}", flush=True)
    A, W = _inputs(M, N, K, 211, kind="bf16")
    C = sk.mm(to_dev(A, "bf16"), to_dev(W, "bf16"), out_dtype=OUT[out])
    torch.cuda.synchronize()
    got = C.float().cpu().numpy()
    ref = oracle.mm(A, "bf16", W, "bf16")
    if out == "bf16":
        # rounding to bf16 (8 significant bits) alone costs up to 2^-8 of an
        # element, more than the 2e-3 bar that the f32 and f16 outputs meet:
        # bound each element by that rounding of the fp32 sum plus the fp32
        # summation bound
        B = _f32_bound(A, "bf16", W, "bf16")
        assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + (1 + 2.0 ** -8) * B)
    else:
        assert rel_err(got, ref) <= REL_TOL
    if out != "f32":
        # the 16-bit output is the f32 result rounded to nearest even
        C32 = sk.mm(to_dev(A, "bf16"), to_dev(W, "bf16"), out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert np.array_equal(bits_of(C), bits_of(C32.to(OUT[out])))


def test_gemm_strided_a():
    # A is a column slice of a wider matrix: lda = 1032 > K = 1000
    M, N, K, LDA = 70, 90, 1000, 1032
    A_full, W = _inputs(M, N, LDA, 221)
    A = np.ascontiguousarray(A_full[:, :K])
    W = np.ascontiguousarray(W[:, :K])
    dA = to_dev(A_full, "f16")[:, :K]
    plan = sk.Plan(N, K, M, sk.F16, sk.F16, sk.F32, lda=LDA)
    C = torch.empty((M, N), dtype=torch.float32, device="cuda")
    plan.run(M, dA, to_dev(W, "f16"), C)
    torch.cuda.synchronize()
    assert rel_err(C.cpu().numpy(), oracle.mm(A, "f16", W, "f16")) <= REL_TOL


@pytest.mark.parametrize("N,flags", [(99, sk.GEMM_SPLIT_LAUNCH), (99, sk.GEMM_ONE_LAUNCH), (4003, 0)])
@pytest.mark.parametrize("ldc", [4104, 4108, 4105])
@pytest.mark.parametrize("out", ["f32", "f16", "bf16"])
def test_gemm_strided_c(N, flags, ldc, out):
    # C is a column slice of a wider buffer (ldc > N; N % 8 = 3, so a row's
    # last group of columns is partial; ldc a multiple of 8, of 4 only, and
    # odd): the stored values are the dense run's bits and the padding
    # columns keep their bytes.  N = 99 runs k in chunks (partial sums + a
    # reduce, or one launch folding them), N = 4003 whole.
    M, K = 150, 520
    A, W = _inputs(M, N, K, 231)
    dA, dW = to_dev(A, "f16"), to_dev(W, "f16")
    ck = {"f32": sk.F32, "f16": sk.F16, "bf16": sk.BF16}[out]
    dense = torch.empty((M, N), dtype=OUT[out], device="cuda")
    sk.Plan(N, K, M, sk.F16, sk.F16, ck, flags=flags).run(M, dA, dW, dense)
    full = torch.full((M, ldc), 7.0, dtype=OUT[out], device="cuda")
    plan = sk.Plan(N, K, M, sk.F16, sk.F16, ck, ldc=ldc, flags=flags)
    print(f"strided C N={N} ldc={ldc} out={out}: {plan.info(M)}", flush=True)
    plan.run(M, dA, dW, full)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(full[:, :N].contiguous()), bits_of(dense))
    assert torch.all(full[:, N:] == 7.0).item()
    ref = oracle.mm(A, "f16", W, "f16")
    got = dense.float().cpu().numpy()
    if out == "bf16":
        # bf16 keeps 8 significant bits: rounding alone may cost 2^-8 of an
        # element (more than the 2e-3 bar, which applies to the fp32 sums);
        # bound each element by that rounding of the fp32 result plus the
        # fp32 summation bound
        B = _f32_bound(A, "f16", W, "f16")
        assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + (1 + 2.0 ** -8) * B)
    else:
        assert rel_err(got, ref) <= REL_TOL


@pytest.mark.parametrize("M,N,K", [(150, 200, 512), (150, 200, 520), (300, 2048, 520)])
def test_gemm_every_tile_bitwise_equal(M, N, K):
    """Every tile gives the same bits: N = 200 with k cut into chunks (the
    plan's chunk launch per tile), N = 2048 with k whole."""
    A, W = _inputs(M, N, K, 7)
    dA, dW = to_dev(A, "f16"), to_dev(W, "f16")
    outs = []
    for tid in range(len(sk.gemm_tiles())):
        print(f"tile {tid} {sk.gemm_tiles()[tid]} N={N} K={K}", flush=True)
        C = sk.mm(dA, dW, out_dtype=torch.float32, tile_id=tid)
        torch.cuda.synchronize()
        outs.append(C.cpu().numpy().view(np.uint32))
    ref = oracle.mm(A, "f16", W, "f16")
    assert rel_err(outs[0].view(np.float32), ref) <= REL_TOL
    for tid, o in enumerate(outs):
        assert np.array_equal(o, outs[0]), sk.gemm_tiles()[tid]


def test_gemm_m_invariance():
    # row i of C is the same for every M >= 17 (the selector picks different
    # tiles as M grows)
    N, K = 640, 1032
    A, W = _inputs(700, N, K, 31)
    dA, dW = to_dev(A, "f16"), to_dev(W, "f16")
    plan = sk.Plan(N, K, 700, sk.F16, sk.F16, sk.F32)
    full = None
    for M in (700, 17, 100, 306, 520):
        print(f"M-invariance M={M}: {plan.info(M)}", flush=True)
        C = torch.empty((M, N), dtype=torch.float32, device="cuda")
        plan.run(M, dA[:M], dW, C)
        torch.cuda.synchronize()
        c = C.cpu().numpy().view(np.uint32)
        if full is None:
            full = c
        else:
            assert np.array_equal(c, full[:M]), M


def _checked_rows(M, M_max):
    """Every row at the workload's largest M; below it, one seeded row in
    every 32-row block (so every MFMA row block of every tile is seen) plus
    the first and the last row."""
    if M == M_max:
        return np.arange(M)
    rng = np.random.default_rng(7000 + M)
    rows = {0, M - 1}
    for b in range(0, M, 32):
        rows.add(int(rng.integers(b, min(b + 32, M))))
    return np.array(sorted(rows))


@pytest.mark.parametrize("name", ["narrow_n96", "wide_n7680"])
def test_gemm_workload_full_size(name):
    """Every configured M at full size, in the launch configuration the bench
    times (the plan's own tile); the oracle checks every row and column at
    the largest M, and a row of every 32-row block at the others."""
    wl = WL.WORKLOADS[name]
    W = WL.gen_w(wl)
    A = WL.gen_a(wl, max(wl.ms))
    dW, dA = to_dev(W, "f16"), to_dev(A, "f16")
    plan = sk.Plan(wl.n, wl.k, max(wl.ms), sk.F16, sk.F16, sk.F16)
    for M in wl.ms:
        print(f"{name} M={M}: {plan.info(M)}", flush=True)
        C = torch.empty((M, wl.n), dtype=torch.float16, device="cuda")
        plan.run(M, dA[:M], dW, C)
        torch.cuda.synchronize()
        rows = _checked_rows(M, max(wl.ms))
        got = C.float().cpu().numpy()[rows]
        ref = oracle.mm(A[rows], "f16", W, "f16")
        assert rel_err(got, ref) <= REL_TOL, M


def test_q8_gemm_full_size_and_fused_equals_unfused():
    wl = WL.WORKLOADS["q8_0_n512"]
    qs, d = WL.gen_w(wl)
    A = WL.gen_a(wl, max(wl.ms))
    dA = to_dev(A, "f16")
    dq = (to_dev(qs, "i8"), to_dev(d, "f16"))
    w16 = sk.dequant_q8_0(*dq)
    for M in (m for m in wl.ms if m > 16):
        print(f"q8_0 GEMM M={M}", flush=True)
        C = sk.mm(dA[:M], dq, out_dtype=torch.float16, max_m=max(wl.ms))
        C2 = sk.mm(dA[:M], w16, out_dtype=torch.float16, max_m=max(wl.ms))
        torch.cuda.synchronize()
        assert np.array_equal(bits_of(C), bits_of(C2)), M
        rows = _checked_rows(M, max(wl.ms))
        ref = oracle.mm(A[rows], "f16", qs, "q8_0", w_scales=d)
        assert rel_err(C.float().cpu().numpy()[rows], ref) <= REL_TOL, M


@pytest.mark.parametrize("M,N,K", [(150, 200, 544), (70, 65, 96), (40, 130, 2592)])
def test_q8_gemm_odd_scale_count_every_tile(M, N, K):
    """K % 64 == 32: each weight row has an odd number of scales, the last
    k-tile holds one.  On every tile (ragged last column tiles down to one
    row, the plan's k chunks on the narrow shapes) the fused Q8_0 GEMM gives
    the bits of the same tile on the dequantised f16 weights, within the fp32
    summation bound of the oracle."""
    A = WL.gen_matrix((M, K), "f16", ("normal", 1.0), 621 + K)
    qs, d = WL.gen_q8_0(N, K, 622 + K, 623 + K)
    dA = to_dev(A, "f16")
    dq = (to_dev(qs, "i8"), to_dev(d, "f16"))
    w16 = sk.dequant_q8_0(*dq)
    ref = oracle.mm(A, "f16", qs, "q8_0", w_scales=d)
    bound = (K + 2) * 2.0 ** -24 * oracle.mm(A, "f16", qs, "q8_0", w_scales=d, absolute=True) + 1e-30
    for tid in range(len(sk.gemm_tiles())):
        print(f"q8_0 odd scales tile {tid} {sk.gemm_tiles()[tid]} M={M} N={N} K={K}", flush=True)
        C = sk.mm(dA, dq, out_dtype=torch.float32, tile_id=tid)
        C2 = sk.mm(dA, w16, out_dtype=torch.float32, tile_id=tid)
        torch.cuda.synchronize()
        got = C.cpu().numpy()
        assert np.array_equal(got.view(np.uint32), C2.cpu().numpy().view(np.uint32)), tid
        assert np.all(np.abs(got - ref) <= bound), tid


@pytest.mark.parametrize("w_kind", ["f16", "q8_0"])
def test_chunked_one_launch_equals_split_launch(w_kind):
    """A plan that cuts k into chunks gives the same bits whether each chunk
    runs in its own block (partials + ordered reduce), one block folds the
    chunk sums in the same order, or the last block of each tile to finish
    folds them (one launch); K = 2600 leaves a short last chunk."""
    N, K = 256, 2560 if w_kind == "q8_0" else 2600
    A = WL.gen_matrix((300, K), "f16", ("normal", 1.0), 601)
    if w_kind == "q8_0":
        qs, d = WL.gen_q8_0(N, K, 602, 603)
        dW, scales, wk = to_dev(qs, "i8"), to_dev(d, "f16"), sk.Q8_0
        ref_all = oracle.mm(A, "f16", qs, "q8_0", w_scales=d)
    else:
        W = WL.gen_matrix((N, K), "f16", ("normal", 0.02), 602)
        dW, scales, wk = to_dev(W, "f16"), None, sk.F16
        ref_all = oracle.mm(A, "f16", W, "f16")
    dA = to_dev(A, "f16")
    outs = {}
    for flag in (sk.GEMM_SPLIT_LAUNCH, sk.GEMM_ONE_LAUNCH, sk.GEMM_FOLD_LAUNCH):
        plan = sk.Plan(N, K, 300, sk.F16, wk, sk.F32, flags=flag)
        ws = plan.workspace(dA.device)
        for M in (17, 64, 300):
            print(f"{w_kind} flag={flag} M={M}: {plan.info(M)}", flush=True)
            C = torch.empty((M, N), dtype=torch.float32, device="cuda")
            plan.run(M, dA[:M], dW, C, scales=scales, workspace=ws)
            torch.cuda.synchronize()
            outs[(flag, M)] = C.cpu().numpy()
    for M in (17, 64, 300):
        a, b = outs[(sk.GEMM_SPLIT_LAUNCH, M)], outs[(sk.GEMM_ONE_LAUNCH, M)]
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), M
        f = outs[(sk.GEMM_FOLD_LAUNCH, M)]
        assert np.array_equal(a.view(np.uint32), f.view(np.uint32)), ("fold", M)
        assert np.array_equal(a.view(np.uint32), outs[(sk.GEMM_SPLIT_LAUNCH, 300)][:M].view(np.uint32)), M
        assert rel_err(a, ref_all[:M]) <= REL_TOL


@pytest.mark.parametrize("w_kind", ["f16", "q8_0"])
def test_fold_launch_every_tile_and_repeated_calls(w_kind):
    """The fold launch on every tile that runs it (ragged row and column
    tiles, the workload's own k chunks) gives the split launch's bits, call
    after call on one workspace (its arrival counters are back at zero after
    each call: the next call's last block would be wrong otherwise)."""
    N, K, M = (96, 2560, 150) if w_kind == "f16" else (512, 2560, 306)
    A = WL.gen_matrix((M, K), "f16", ("normal", 1.0), 631)
    if w_kind == "q8_0":
        qs, d = WL.gen_q8_0(N, K, 632, 633)
        dW, scales, wk = to_dev(qs, "i8"), to_dev(d, "f16"), sk.Q8_0
    else:
        dW, scales, wk = to_dev(WL.gen_matrix((N, K), "f16", ("normal", 0.02), 632), "f16"), None, sk.F16
    dA = to_dev(A, "f16")
    ref = sk.Plan(N, K, M, sk.F16, wk, sk.F16, flags=sk.GEMM_SPLIT_LAUNCH)
    C0 = torch.empty((M, N), dtype=torch.float16, device="cuda")
    ref.run(M, dA, dW, C0, scales=scales)
    torch.cuda.synchronize()
    want = bits_of(C0)
    for tid, name in enumerate(sk.gemm_tiles()):
        plan = sk.Plan(N, K, M, sk.F16, wk, sk.F16, flags=sk.GEMM_FOLD_LAUNCH, tile_id=tid)
        if "launch=fold" not in plan.info(M):
            continue
        print(f"fold {w_kind} tile {name}: {plan.info(M)}", flush=True)
        ws = sk.new_workspace(plan, dA.device)
        for rep in range(3):
            for m in (M, 17):
                C = torch.empty((m, N), dtype=torch.float16, device="cuda")
                plan.run(m, dA[:m], dW, C, scales=scales, workspace=ws)
                torch.cuda.synchronize()
                if m == M:
                    assert np.array_equal(bits_of(C), want), (name, rep)
