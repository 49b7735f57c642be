"""skinny_mm_run_static, the run call that allocates nothing: its scratch is
the library's static device array instead of a caller's workspace.

On the GPU (through the C ABI): on two calls in a row, the second with a
smaller input, it gives skinny_mm_run's bits on every kind of run that needs
scratch -- a GEMV whose k splits are summed across workgroups (arrival
counters + partial sums), a GEMM whose k chunks run as separate blocks
(partial sums + the ordered reduce, or chunk sums folded by the last block
of each tile, with arrival counters), fp32 rows cast before the GEMV (cast
rows) -- and on a run that needs none; the results also meet the oracle's
bar.  The second GEMV call is right only if the first left its arrival
counters at zero.  On the host: sizes beyond the array are rejected before
any HIP call.
"""
import ctypes

import numpy as np
import pytest

import oracle
import workloads as WL
from conftest import REL_TOL, gpu_available, rel_err, to_dev

import row_gemv_decode_amd as sk

L = sk.lib()


def _static_status(plan, m, A, W, S, C, stream=None):
    return L.skinny_mm_run_static(plan.handle, m, A, W, S, C, stream)


@pytest.mark.skipif(gpu_available(), reason="made-up pointers must never reach a GPU")
def test_sizes_beyond_the_static_array_are_rejected_on_the_host():
    P, Pb, Pc = (ctypes.c_void_p(x << 20) for x in (1, 2, 3))
    # narrow N with its k chunks run as separate blocks: 4 chunks x M x 96
    # fp32 partials; M = 30000 needs 46.1 MB of the 31 MiB data region
    p = sk.Plan(96, 2560, 30000, sk.F16, sk.F16, sk.F16, flags=sk.GEMM_SPLIT_LAUNCH, num_cus=256)
    assert "launch=split" in p.info(30000) and " chunks=4 " in p.info(30000)
    assert _static_status(p, 30000, P, Pb, None, Pc) == sk.ERR_SCRATCH
    # argument errors come first, as in skinny_mm_run
    assert _static_status(p, 0, P, Pb, None, Pc) == sk.ERR_INVALID_ARG
    assert _static_status(p, 30000, None, Pb, None, Pc) == sk.ERR_INVALID_ARG
    # a GEMV whose k splits are summed across workgroups: 16 splits x n fp32
    # partials (256 MiB at n = 2^22; its 2 MiB of arrival counters would not
    # fit their region either)
    g = sk.Plan(1 << 22, 16384, 16, sk.F16, sk.F16, sk.F32, num_cus=256)
    assert "split_reduce=global" in g.info(1)
    assert _static_status(g, 1, P, Pb, None, Pc) == sk.ERR_SCRATCH


def _cases():
    # (label, plan kwargs, A kind, (m1, m2)): the second call is smaller
    return [
        ("gemv_global_split", dict(n=256, k=16384, a=sk.BF16, w=sk.BF16, c=sk.F32), "bf16", (16, 3)),
        ("gemm_split_launch", dict(n=96, k=2560, a=sk.F16, w=sk.F16, c=sk.F16,
                                   flags=sk.GEMM_SPLIT_LAUNCH), "f16", (700, 130)),
        ("gemm_split_q8", dict(n=512, k=2560, a=sk.F16, w=sk.Q8_0, c=sk.F16,
                               flags=sk.GEMM_SPLIT_LAUNCH), "f16", (306, 40)),
        ("gemm_fold_launch", dict(n=96, k=2560, a=sk.F16, w=sk.F16, c=sk.F16,
                                  flags=sk.GEMM_FOLD_LAUNCH), "f16", (700, 130)),
        ("fp32_rows_cast_first", dict(n=256, k=5120, a=sk.F32, w=sk.BF16, c=sk.F32), "f32", (16, 11)),
        ("no_scratch_gemm", dict(n=384, k=512, a=sk.F16, w=sk.F16, c=sk.F32), "f16", (150, 33)),
    ]


@pytest.mark.gpu
@pytest.mark.parametrize("label,kw,akind,ms", _cases(), ids=[c[0] for c in _cases()])
def test_static_run_equals_workspace_run(label, kw, akind, ms):
    import torch

    n, k = kw["n"], kw["k"]
    max_m = ms[0]
    seed = 900 + n + k
    if akind == "f32":
        A = np.random.default_rng(seed).standard_normal((max_m, k)).astype(np.float32)
        dA = torch.from_numpy(A).cuda()
    else:
        A = WL.gen_matrix((max_m, k), akind, ("normal", 1.0), seed)
        dA = to_dev(A, akind)
    if kw["w"] == sk.Q8_0:
        qs, d = WL.gen_q8_0(n, k, seed + 1, seed + 2)
        dW, dS = to_dev(qs, "i8"), to_dev(d, "f16")
        ref_all = oracle.mm(A, "f16", qs, "q8_0", w_scales=d)
    else:
        wk = "bf16" if kw["w"] == sk.BF16 else "f16"
        Wb = WL.gen_matrix((n, k), wk, ("normal", 0.02), seed + 1)
        dW, dS = to_dev(Wb, wk), None
        A16 = oracle.cast_bf16(A) if akind == "f32" else A  # fp32 rows reach the GEMV as bf16
        ref_all = oracle.mm(A16, "bf16" if akind == "f32" else akind, Wb, wk)
    plan = sk.Plan(n, k, max_m, kw["a"], kw["w"], kw["c"], flags=kw.get("flags", 0))
    cdt = {sk.F32: torch.float32, sk.F16: torch.float16}[kw["c"]]
    ws = sk.new_workspace(plan, dA.device)
    for m in ms:
        print(f"no-alloc {label} m={m}: {plan.info(m)}", flush=True)
        C_ws = torch.full((m, n), 3.0, dtype=cdt, device="cuda")
        C_st = torch.full((m, n), -5.0, dtype=cdt, device="cuda")
        plan.run(m, dA[:m], dW, C_ws, scales=dS, workspace=ws)
        plan.run_static(m, dA[:m], dW, C_st, scales=dS)
        torch.cuda.synchronize()
        a = C_ws.contiguous().view(torch.int16 if cdt == torch.float16 else torch.int32).cpu().numpy()
        b = C_st.contiguous().view(torch.int16 if cdt == torch.float16 else torch.int32).cpu().numpy()
        assert np.array_equal(a, b), (label, m)
        assert rel_err(C_st.float().cpu().numpy(), ref_all[:m]) <= REL_TOL, (label, m)
