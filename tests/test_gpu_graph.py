"""HIP-graph capture of every run shape (the bench times graph replays).

Each shape is captured once into a graph of several calls, then the graph is
replayed three times with eager calls of the same shape and host
synchronisations in between; every replay must reproduce the eager results
bit for bit.  This covers the run shapes that keep state in the caller's
workspace between calls (the arrival counters of a GEMV whose k is split across
workgroups, which the kernels reset) and the two-launch shapes (the GEMM's
k-chunk partials + ordered reduce, the router's GEMV + top-k, fp32 rows cast
into the workspace + the bf16 GEMV), the row-grouped launches and the gate as
one launch with the cast fused; none records a memset.
"""
import numpy as np
import pytest

import workloads as WL
from conftest import to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
sk = pytest.importorskip("row_gemv_decode_amd")


def _replay_matches_eager(fn, outs, calls=3, replays=3):
    """fn(i) enqueues call i and writes outs[i % len(outs)] (a tuple of tensors)."""
    for i in range(calls):  # eager reference
        fn(i)
    torch.cuda.synchronize()
    ref = [tuple(t.clone() for t in o) for o in outs]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn(0)  # warm on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            for i in range(calls):
                fn(i)
    torch.cuda.synchronize()
    for rep in range(replays):
        for o in outs:
            for t in o:
                t.fill_(7)  # a replay must rewrite every output
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            for t, tr in zip(o, r):
                assert torch.equal(t.view(torch.uint8), tr.view(torch.uint8)), rep
        for i in range(calls):  # the program's own eager work between replays
            fn(i)
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            for t, tr in zip(o, r):
                assert torch.equal(t.view(torch.uint8), tr.view(torch.uint8)), rep
    del g


@pytest.mark.parametrize("n,k,ms", [(256, 5120, (1, 8, 16)),    # k split in the workgroup
                                     (256, 16384, (1, 5, 16)),  # k split across workgroups (counters)
                                     (4864, 896, (2, 16)),      # unsplit, A staged in LDS
                                     (608, 896, (4, 8, 16)),    # unsplit, row groups of 1, 2, 4 rows
                                     (8, 5120, (2, 16))])       # one workgroup: a row group per row
def test_gemv_graph_replays(n, k, ms):
    print(f"graph gemv n={n} k={k}", flush=True)
    W = to_dev(WL.gen_matrix((n, k), "bf16", ("normal", 0.02), 701), "bf16")
    A = to_dev(WL.gen_matrix((16, k), "bf16", ("normal", 1.0), 702), "bf16")
    plan = sk.Plan(n, k, 16, sk.BF16, sk.BF16, sk.F32)
    ws = plan.workspace(A.device)
    outs = [(torch.empty((m, n), dtype=torch.float32, device="cuda"),) for m in ms]

    def fn(i):
        m = ms[i % len(ms)]
        plan.run(m, A[:m], W, outs[i % len(ms)][0], workspace=ws)
    _replay_matches_eager(fn, outs, calls=len(ms))
    if ws is not None:
        assert not torch.any(ws[:256]).item()  # counters back at zero


def test_router_topk_graph_replays():
    wl = WL.WORKLOADS["router_topk"]
    W = to_dev(WL.gen_w(wl), "bf16")
    A = to_dev(WL.gen_a(wl, 16), "bf16")
    plan = sk.Plan(wl.n, wl.k, 16, sk.BF16, sk.BF16, sk.F32)
    ms = (1, 2, 4, 8, 16)
    outs = [(torch.empty((m, wl.n), dtype=torch.float32, device="cuda"),
             torch.empty((m, 10), dtype=torch.int32, device="cuda"),
             torch.empty((m, 10), dtype=torch.float32, device="cuda")) for m in ms]

    def fn(i):
        m = ms[i % len(ms)]
        lg, idx, val = outs[i % len(ms)]
        plan.run_topk(m, A[:m], W, lg, idx, val, 10)
    _replay_matches_eager(fn, outs, calls=len(ms))


@pytest.mark.parametrize("flag", ["split", "one", "fold"])
def test_gemm_chunked_graph_replays(flag):
    # narrow N: k cut into chunks, as partials + reduce launch or one launch
    N, K = 96, 2560
    W = to_dev(WL.gen_matrix((N, K), "f16", ("normal", 0.02), 711), "f16")
    A = to_dev(WL.gen_matrix((600, K), "f16", ("normal", 1.0), 712), "f16")
    flags = {"split": sk.GEMM_SPLIT_LAUNCH, "one": sk.GEMM_ONE_LAUNCH, "fold": sk.GEMM_FOLD_LAUNCH}[flag]
    plan = sk.Plan(N, K, 600, sk.F16, sk.F16, sk.F16, flags=flags)
    ws = plan.workspace(A.device)
    ms = (17, 300, 600)
    for m in ms:
        print(f"graph gemm {flag} m={m}: {plan.info(m)}", flush=True)
    outs = [(torch.empty((m, N), dtype=torch.float16, device="cuda"),) for m in ms]

    def fn(i):
        m = ms[i % len(ms)]
        plan.run(m, A[:m], W, outs[i % len(ms)][0], workspace=ws)
    _replay_matches_eager(fn, outs, calls=len(ms))


@pytest.mark.parametrize("shape", ["cast_then_gemv", "fused"])
def test_gate_graph_replays(shape):
    wl = WL.WORKLOADS["scalar_gate"]
    W = to_dev(WL.gen_w(wl), "bf16")
    A = torch.from_numpy(np.ascontiguousarray(WL.gen_a(wl, 16))).cuda()
    ms = (1, 16)
    A16 = torch.empty((16, wl.k), dtype=torch.bfloat16, device="cuda")
    a_code = sk.F32 if shape == "fused" else sk.BF16
    plan = sk.Plan(wl.n, wl.k, 16, a_code, sk.BF16, sk.F32, flags=sk.EPILOGUE_SIGMOID)
    outs = [(torch.empty((m, wl.n), dtype=torch.float32, device="cuda"),) for m in ms]

    def fn(i):
        m = ms[i % len(ms)]
        if shape == "fused":
            plan.run(m, A[:m], W, outs[i % len(ms)][0])
        else:
            sk.cast_f32_bf16(A[:m], out=A16[:m])
            plan.run(m, A16[:m], W, outs[i % len(ms)][0])
    print(f"graph gate {shape}", flush=True)
    _replay_matches_eager(fn, outs, calls=len(ms))


def test_fp32_rows_cast_first_graph_replays():
    """fp32 rows, k split inside the workgroup, 256 columns: m = 11 and 16 run
    the cast into the workspace and the bf16 GEMV (two launches of one run),
    m = 1 the fused launch."""
    n, k = 256, 5120
    W = to_dev(WL.gen_matrix((n, k), "bf16", ("normal", 0.02), 721), "bf16")
    A = torch.from_numpy(np.ascontiguousarray(WL.gen_matrix((16, k), "f32", ("normal", 1.0), 722))).cuda()
    plan = sk.Plan(n, k, 16, sk.F32, sk.BF16, sk.F32)
    ws = plan.workspace(A.device)
    ms = (1, 11, 16)
    for m in ms:
        print(f"graph fp32 rows m={m}: {plan.info(m)}", flush=True)
    assert "a=f32(cast-launch) " in plan.info(16)
    outs = [(torch.empty((m, n), dtype=torch.float32, device="cuda"),) for m in ms]

    def fn(i):
        m = ms[i % len(ms)]
        plan.run(m, A[:m], W, outs[i % len(ms)][0], workspace=ws)
    _replay_matches_eager(fn, outs, calls=len(ms))
