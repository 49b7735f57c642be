"""CPU oracle for the weight-streaming skinny matmul (TEST INFRASTRUCTURE ONLY).

A plain fp64 C implementation (oracle.c) behind ctypes.  Only the tests, the
smoke check and the bench's CPU-baseline leg may import this package; the
library's product path never does, and this code shares nothing with it.

All 16-bit float arrays cross this boundary as raw bit patterns (numpy uint16).

What each function follows (page titles and sections; no code is taken from
the pages, which print none for these steps):
  mm          -- nx_batchscale_kat: C[m,n] = A[m,k] . W[k,n]; W stored [n][k]
  dequant     -- opus r35 track A, section 1 (`dq_f16` to f16 weights), with the
                 Q8_0-style format: blocks of 32 along k, int8 q, f16 scale d,
                 w = RNE_f16(d * q)
  dequant_q4_0 -- the 4-bit block format the Strata PR #109 page names
                 ("Measured": IQ3_S, Q2_0) but does not define, fixed here as
                 Q4_0-style: blocks of 32 along k, one f16 scale d, 4-bit
                 codes q two per byte (even k low nibble), w = RNE_f16(d*(q-8))
  dequant_q2_0 -- the 2-bit block format the same page names (Q2_0 runs) but
                 does not define, fixed here as the 2-bit counterpart: blocks
                 of 32 along k, one f16 scale d, 2-bit codes q four per byte
                 (element kk at bits 2*(kk%4)), w = RNE_f16(d*(q-2))
  topk        -- Strata PR #109, "What" (router top-10 per token), ties to the
                 lower index
  cast_bf16   -- Strata PR #109, "What" (the bf16 cast of the window's rows):
                 fp32 to bf16, round to nearest, ties to even
  sigmoid, gate -- Strata PR #109, "What" (the shared expert's scalar gate: a
                 multi-row GEMV, then a sigmoid): gate = 1 / (1 + e^-(a . w))
  moe_combine -- Strata PR #109, "What" (the MoE combine, one launch over the
                 window's tokens): each token's output row is its experts'
                 output rows weighted by its routing weights, plus the shared
                 expert's row times its gate.  The page does not say how the
                 routing weights are formed, so they are an input.
"""
import ctypes
import os

import numpy as np

from . import build as _build

F16, BF16, Q8_0, Q4_0, Q2_0 = 1, 2, 4, 5, 6
_KINDS = {"f16": F16, "bf16": BF16, "q8_0": Q8_0, "q4_0": Q4_0, "q2_0": Q2_0}
# stored codes per byte of the packed block formats
_CODES_PER_BYTE = {"q8_0": 1, "q4_0": 2, "q2_0": 4}

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_build.LIB):
        _build.build()
    lib = ctypes.CDLL(_build.LIB)
    i64, i32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
    lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_to_f64.restype = ctypes.c_double
    lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_f64.restype = ctypes.c_double
    lib.oracle_f64_to_f16_rne.argtypes = [ctypes.c_double]
    lib.oracle_f64_to_f16_rne.restype = ctypes.c_uint16
    lib.oracle_dequant_q8_0.argtypes = [i64, i64, vp, vp, vp]
    lib.oracle_dequant_q8_0.restype = ctypes.c_int
    lib.oracle_dequant_q4_0.argtypes = [i64, i64, vp, vp, vp]
    lib.oracle_dequant_q4_0.restype = ctypes.c_int
    lib.oracle_dequant_q2_0.argtypes = [i64, i64, vp, vp, vp]
    lib.oracle_dequant_q2_0.restype = ctypes.c_int
    lib.oracle_mm.argtypes = [i64, i64, i64, ctypes.c_int, vp, i64, ctypes.c_int, vp, vp, vp,
                              i64, ctypes.c_int, ctypes.c_int]
    lib.oracle_mm.restype = ctypes.c_int
    lib.oracle_topk.argtypes = [i64, i64, vp, i64, i32, vp, vp]
    lib.oracle_topk.restype = ctypes.c_int
    lib.oracle_f64_to_bf16_rne.argtypes = [ctypes.c_double]
    lib.oracle_f64_to_bf16_rne.restype = ctypes.c_uint16
    lib.oracle_cast_f32_bf16.argtypes = [i64, vp, vp]
    lib.oracle_cast_f32_bf16.restype = None
    lib.oracle_sigmoid.argtypes = [i64, vp, vp]
    lib.oracle_sigmoid.restype = None
    _lib = lib
    return lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def f16_to_f64(bits) -> float:
    return _load().oracle_f16_to_f64(int(bits))


def bf16_to_f64(bits) -> float:
    return _load().oracle_bf16_to_f64(int(bits))


def f64_to_f16_rne(x: float) -> int:
    return int(_load().oracle_f64_to_f16_rne(float(x)))


def decode(bits: np.ndarray, kind: str) -> np.ndarray:
    """fp64 values of an array of f16 / bf16 bit patterns (elementwise)."""
    lib = _load()
    fn = lib.oracle_bf16_to_f64 if kind == "bf16" else lib.oracle_f16_to_f64
    flat = np.ascontiguousarray(bits, dtype=np.uint16).ravel()
    lut = np.array([fn(v) for v in range(65536)], dtype=np.float64)
    return lut[flat].reshape(np.shape(bits))


def dequant_q8_0(qs: np.ndarray, d: np.ndarray) -> np.ndarray:
    """f16 bits [n][k] of RNE_f16(d[j][kk/32] * qs[j][kk])."""
    qs = np.ascontiguousarray(qs, dtype=np.int8)
    d = np.ascontiguousarray(d, dtype=np.uint16)
    n, k = qs.shape
    assert d.shape == (n, k // 32), (d.shape, qs.shape)
    out = np.empty((n, k), dtype=np.uint16)
    rc = _load().oracle_dequant_q8_0(n, k, _ptr(qs), _ptr(d), _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle_dequant_q8_0 failed ({rc})")
    return out


def dequant_q4_0(qs: np.ndarray, d: np.ndarray) -> np.ndarray:
    """f16 bits [n][k] of RNE_f16(d[j][kk/32] * (q - 8)), q the 4-bit code of
    element kk: the low nibble of qs[j][kk/2] for even kk, the high for odd."""
    qs = np.ascontiguousarray(qs, dtype=np.uint8)
    d = np.ascontiguousarray(d, dtype=np.uint16)
    n, kh = qs.shape
    k = 2 * kh
    assert d.shape == (n, k // 32), (d.shape, qs.shape)
    out = np.empty((n, k), dtype=np.uint16)
    rc = _load().oracle_dequant_q4_0(n, k, _ptr(qs), _ptr(d), _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle_dequant_q4_0 failed ({rc})")
    return out


def dequant_q2_0(qs: np.ndarray, d: np.ndarray) -> np.ndarray:
    """f16 bits [n][k] of RNE_f16(d[j][kk/32] * (q - 2)), q the 2-bit code of
    element kk: bits 2*(kk%4) and 2*(kk%4)+1 of qs[j][kk/4]."""
    qs = np.ascontiguousarray(qs, dtype=np.uint8)
    d = np.ascontiguousarray(d, dtype=np.uint16)
    n, kq = qs.shape
    k = 4 * kq
    assert d.shape == (n, k // 32), (d.shape, qs.shape)
    out = np.empty((n, k), dtype=np.uint16)
    rc = _load().oracle_dequant_q2_0(n, k, _ptr(qs), _ptr(d), _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle_dequant_q2_0 failed ({rc})")
    return out


def mm(A: np.ndarray, a_kind: str, W: np.ndarray, w_kind: str, w_scales=None,
       threads=None, absolute=False) -> np.ndarray:
    """fp64 C[m][n] = sum_kk A[i][kk] * W[j][kk] (W stored [n][k]).

    A: uint16 bits [m][k]; W: uint16 bits [n][k], or int8 codes [n][k] for
    q8_0, packed 4-bit codes uint8 [n][k/2] for q4_0 or packed 2-bit codes
    uint8 [n][k/4] for q2_0, each with w_scales uint16 bits [n][k/32].
    absolute=True returns sum |A| * |W| instead (the fp32 rounding-error
    yardstick).
    """
    A = np.ascontiguousarray(A, dtype=np.uint16)
    m, k = A.shape
    if w_kind in _CODES_PER_BYTE:
        W = np.ascontiguousarray(W, dtype=np.int8 if w_kind == "q8_0" else np.uint8)
        w_scales = np.ascontiguousarray(w_scales, dtype=np.uint16)
        sp = _ptr(w_scales)
    else:
        W = np.ascontiguousarray(W, dtype=np.uint16)
        sp = None
    n, k2 = W.shape
    k2 *= _CODES_PER_BYTE.get(w_kind, 1)
    assert k2 == k, (A.shape, W.shape)
    C = np.zeros((m, n), dtype=np.float64)
    t = default_threads() if threads is None else int(threads)
    rc = _load().oracle_mm(m, n, k, _KINDS[a_kind], _ptr(A), k, _KINDS[w_kind], _ptr(W), sp,
                           _ptr(C), n, t, 1 if absolute else 0)
    if rc != 0:
        raise ValueError(f"oracle_mm failed ({rc})")
    return C


def topk(logits: np.ndarray, k: int):
    """Per-row top-k: (idx int32 [m][k], val fp64 [m][k]), value desc, index asc."""
    L = np.ascontiguousarray(logits, dtype=np.float64)
    m, n = L.shape
    idx = np.empty((m, k), dtype=np.int32)
    val = np.empty((m, k), dtype=np.float64)
    rc = _load().oracle_topk(m, n, _ptr(L), n, k, _ptr(idx), _ptr(val))
    if rc != 0:
        raise ValueError(f"oracle_topk failed ({rc})")
    return idx, val


def f64_to_bf16_rne(x: float) -> int:
    return int(_load().oracle_f64_to_bf16_rne(float(x)))


def cast_bf16(x: np.ndarray) -> np.ndarray:
    """bf16 bits of every fp32 value of x, rounded to nearest, ties to even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().oracle_cast_f32_bf16(x.size, _ptr(x), _ptr(out))
    return out


def sigmoid(x: np.ndarray) -> np.ndarray:
    """fp64 1 / (1 + e^-x), elementwise."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty(x.shape, dtype=np.float64)
    _load().oracle_sigmoid(x.size, _ptr(x), _ptr(y))
    return y


def gate(A_f32: np.ndarray, W: np.ndarray, w_kind: str = "bf16", threads=None) -> np.ndarray:
    """The scalar gate over fp32 rows: sigmoid(cast_bf16(A) . W) in fp64,
    W stored [n][k] (n = 1 for a scalar gate)."""
    return sigmoid(mm(cast_bf16(A_f32), "bf16", W, w_kind, threads=threads))


def _row_values(x: np.ndarray, kind: str) -> np.ndarray:
    """fp64 values of fp32 values ("f32") or bf16 bit patterns ("bf16")."""
    if kind == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    return decode(x, "bf16")


def moe_combine(y: np.ndarray, w: np.ndarray, shared=None, gate=None, kind: str = "f32") -> np.ndarray:
    """fp64 out[t][c] = sum over i of w[t][i] * y[t][i][c], plus gate[t] * shared[t][c]
    when the shared expert's row is given.

    y: [m][topk][d] expert output rows, w: [m][topk] fp32 routing weights,
    shared: [m][d] or None, gate: [m] fp32 (with shared); y and shared are
    fp32 values (kind "f32") or bf16 bit patterns (kind "bf16").  Every
    product of two fp32 values is exact in fp64; the experts are added in
    order i = 0 .. topk - 1, then the shared term.
    """
    Y = _row_values(y, kind)
    Wt = np.asarray(w, dtype=np.float32).astype(np.float64)
    m, topk, d = Y.shape
    assert Wt.shape == (m, topk)
    out = np.zeros((m, d), dtype=np.float64)
    for i in range(topk):
        out += Wt[:, i:i + 1] * Y[:, i, :]
    if shared is not None:
        S = _row_values(shared, kind)
        G = np.asarray(gate, dtype=np.float32).astype(np.float64)
        assert S.shape == (m, d) and G.shape == (m,)
        out += G[:, None] * S
    return out
