"""GPU parity of the MFMA GEMM path (m >= 17) against the CPU oracle, and its
bitwise tile- and M-invariance."""
import numpy as np
import pytest

import oracle
import workloads as WL
from conftest import REL_TOL, bits_of, rel_err, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
sk = pytest.importorskip("row_gemv_decode_amd")


def _inputs(M, N, K, seed, kind="f16"):
    A = WL.gen_matrix((M, K), kind, ("normal", 1.0), seed)
    W = WL.gen_matrix((N, K), kind, ("normal", 0.02), seed + 1)
    return A, W


@pytest.mark.parametrize("M,N,K", [(17, 96, 2560), (150, 384, 2560), (306, 200, 512), (64, 64, 64), (33, 7680, 256)])
def test_gemm_parity_small(M, N, K):
    print(f"gemm M={M} N={N} K={K}", flush=True)
    A, W = _inputs(M, N, K, 100 + M)
    C = sk.mm(to_dev(A, "f16"), to_dev(W, "f16"), out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.mm(A, "f16", W, "f16")
    assert rel_err(C.cpu().numpy(), ref) <= REL_TOL


def test_gemm_every_tile_bitwise_equal():
    M, N, K = 150, 200, 512
    A, W = _inputs(M, N, K, 7)
    dA, dW = to_dev(A, "f16"), to_dev(W, "f16")
    outs = []
    for tid in range(len(sk.gemm_tiles())):
        print(f"tile {tid} {sk.gemm_tiles()[tid]}", flush=True)
        C = sk.mm(dA, dW, out_dtype=torch.float32, tile_id=tid)
        torch.cuda.synchronize()
        outs.append(C.cpu().numpy().view(np.uint32))
    ref = oracle.mm(A, "f16", W, "f16")
    assert rel_err(outs[0].view(np.float32), ref) <= REL_TOL
    for tid, o in enumerate(outs):
        assert np.array_equal(o, outs[0]), sk.gemm_tiles()[tid]
