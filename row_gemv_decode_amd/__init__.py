"""Thin Python binding of libskinny.so, the MI355X weight-streaming skinny matmul.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI (include/skinny.h).  PyTorch supplies device memory
and the current stream; nothing here computes a result, and there is no CPU
fallback -- importing this package fails loudly when the library is missing.

    C = mm(A, W)                       # f16/bf16 rows x [n][k] weight
    C = mm(A, (qs, d))                 # Q8_0-style weight: int8 codes, f16 scales
                                       # (Q4_0 / Q2_0: packed uint8 codes)
    logits, idx, val = gemv_topk(A, W, topk=10)
    w16 = dequant_q8_0(qs, d)

W is stored [n][k] (k-contiguous): stored row j is column j of the logical
W[k, n] in C[m, n] = A[m, k] . W[k, n].
"""
import ctypes
import os

# torch first: it brings its own HIP runtime (soname libamdhip64.so.7); loaded
# afterwards, libskinny.so binds to that same runtime, so torch's streams and
# device memory are the library's.  Loaded the other way round the process
# would hold two HIP runtimes that do not share devices or streams.
import torch  # noqa: F401

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libskinny.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python -m row_gemv_decode_amd.build` "
        "(or __graft_entry__.build()); there is no fallback implementation")

_lib = ctypes.CDLL(LIB_PATH)

# --- C ABI mirror -----------------------------------------------------------
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_ALIGNMENT, ERR_SHAPE, ERR_HIP, ERR_WORKSPACE, ERR_SCRATCH = range(8)
F16, BF16, F32, Q8_0, Q4_0, Q2_0 = 1, 2, 3, 4, 5, 6
# stored codes per byte of the block-quantised weight kinds
CODES_PER_BYTE = {Q8_0: 1, Q4_0: 2, Q2_0: 4}
FORCE_GEMV, FORCE_GEMM, GEMM_SPLIT_LAUNCH, GEMM_ONE_LAUNCH = 0x1, 0x2, 0x4, 0x8
EPILOGUE_SIGMOID = 0x10
GEMM_FOLD_LAUNCH = 0x20
GEMV_MAX_M = 16
TOPK_MAX = 32

EXPORTS = (
    "skinny_mm_plan", "skinny_mm_plan_destroy", "skinny_mm_workspace_size", "skinny_mm_run",
    "gemv_topk_run", "skinny_dequant_q8_0_run", "skinny_dequant_q4_0_run", "skinny_dequant_q2_0_run",
    "skinny_mm_plan_info",
    "skinny_gemm_tile_count",
    "skinny_gemm_tile_name", "skinny_status_string", "skinny_abi_version", "skinny_cast_f32_bf16_run",
    "skinny_moe_combine_run", "skinny_mm_run_static",
)
STATIC_SCRATCH_BYTES = 32 << 20
STATIC_COUNTER_BYTES = 1 << 20


class MMDesc(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("a_dtype", ctypes.c_int32),
        ("w_dtype", ctypes.c_int32),
        ("c_dtype", ctypes.c_int32),
        ("max_m", ctypes.c_int64),
        ("n", ctypes.c_int64),
        ("k", ctypes.c_int64),
        ("lda", ctypes.c_int64),
        ("ldc", ctypes.c_int64),
        ("flags", ctypes.c_uint32),
        ("tile_id", ctypes.c_int32),
        ("num_cus", ctypes.c_int32),
    ]


_vp, _i64, _i32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
_lib.skinny_mm_plan.argtypes = [ctypes.POINTER(MMDesc), ctypes.POINTER(_vp)]
_lib.skinny_mm_plan.restype = ctypes.c_int
_lib.skinny_mm_plan_destroy.argtypes = [_vp]
_lib.skinny_mm_plan_destroy.restype = None
_lib.skinny_mm_workspace_size.argtypes = [_vp, ctypes.POINTER(_sz)]
_lib.skinny_mm_workspace_size.restype = ctypes.c_int
_lib.skinny_mm_run.argtypes = [_vp, _i64, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.skinny_mm_run.restype = ctypes.c_int
_lib.skinny_mm_run_static.argtypes = [_vp, _i64, _vp, _vp, _vp, _vp, _vp]
_lib.skinny_mm_run_static.restype = ctypes.c_int
_lib.gemv_topk_run.argtypes = [_vp, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _sz, _vp]
_lib.gemv_topk_run.restype = ctypes.c_int
_lib.skinny_dequant_q8_0_run.argtypes = [_i64, _i64, _vp, _vp, _vp, _vp]
_lib.skinny_dequant_q8_0_run.restype = ctypes.c_int
_lib.skinny_dequant_q4_0_run.argtypes = [_i64, _i64, _vp, _vp, _vp, _vp]
_lib.skinny_dequant_q4_0_run.restype = ctypes.c_int
_lib.skinny_dequant_q2_0_run.argtypes = [_i64, _i64, _vp, _vp, _vp, _vp]
_lib.skinny_dequant_q2_0_run.restype = ctypes.c_int
_lib.skinny_cast_f32_bf16_run.argtypes = [_i64, _vp, _vp, _vp]
_lib.skinny_cast_f32_bf16_run.restype = ctypes.c_int
_lib.skinny_moe_combine_run.argtypes = [_i64, _i64, _i32, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _vp]
_lib.skinny_moe_combine_run.restype = ctypes.c_int
_lib.skinny_mm_plan_info.argtypes = [_vp, _i64, ctypes.c_char_p, _sz]
_lib.skinny_mm_plan_info.restype = ctypes.c_int
_lib.skinny_gemm_tile_count.argtypes = []
_lib.skinny_gemm_tile_count.restype = _i32
_lib.skinny_gemm_tile_name.argtypes = [_i32]
_lib.skinny_gemm_tile_name.restype = ctypes.c_char_p
_lib.skinny_status_string.argtypes = [ctypes.c_int]
_lib.skinny_status_string.restype = ctypes.c_char_p
_lib.skinny_abi_version.argtypes = []
_lib.skinny_abi_version.restype = _i32


class SkinnyError(RuntimeError):
    def __init__(self, status: int, where: str = ""):
        self.status = int(status)
        msg = _lib.skinny_status_string(self.status).decode()
        super().__init__(f"{where}: {msg} (status {self.status})" if where else msg)


def _check(status: int, where: str):
    if status != OK:
        raise SkinnyError(status, where)


def lib() -> ctypes.CDLL:
    return _lib


def abi_version() -> int:
    return int(_lib.skinny_abi_version())


def gemm_tiles():
    return [_lib.skinny_gemm_tile_name(i).decode() for i in range(_lib.skinny_gemm_tile_count())]


# --- torch plumbing ---------------------------------------------------------
def _torch():
    import torch
    return torch


def _dtype_code(t, what):
    torch = _torch()
    if t == torch.float16:
        return F16
    if t == torch.bfloat16:
        return BF16
    if t == torch.float32:
        return F32
    raise TypeError(f"{what}: unsupported dtype {t}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


class Plan:
    """A skinny_mm_plan: host-only, immutable, reusable across streams (the
    workspaces it hands out are kept per device and stream)."""

    def __init__(self, n, k, max_m, a_dtype=F16, w_dtype=F16, c_dtype=F32, lda=0, ldc=0,
                 flags=0, tile_id=-1, num_cus=0):
        d = MMDesc(ctypes.sizeof(MMDesc), a_dtype, w_dtype, c_dtype, max_m, n, k, lda, ldc,
                   flags, tile_id, num_cus)
        h = ctypes.c_void_p()
        _check(_lib.skinny_mm_plan(ctypes.byref(d), ctypes.byref(h)), "skinny_mm_plan")
        self._h = h
        self.n, self.k, self.max_m = n, k, max_m
        self.a_dtype, self.w_dtype, self.c_dtype = a_dtype, w_dtype, c_dtype
        self.lda, self.ldc = lda or k, ldc or n
        sz = ctypes.c_size_t()
        _check(_lib.skinny_mm_workspace_size(self._h, ctypes.byref(sz)), "skinny_mm_workspace_size")
        self.workspace_bytes = int(sz.value)
        self._ws = {}

    @property
    def handle(self):
        return self._h

    def info(self, m: int) -> str:
        buf = ctypes.create_string_buffer(256)
        _check(_lib.skinny_mm_plan_info(self._h, m, buf, 256), "skinny_mm_plan_info")
        return buf.value.decode()

    def workspace(self, device, stream=None):
        """A zero-initialised device workspace of this plan for one (device,
        stream) pair (None when none is needed).  Runs on one stream are
        ordered, so they may share it; runs on different streams may be in
        flight at once and must not (the workspace holds arrival counters and
        partial sums), so every stream gets its own.  It is allocated and
        zero-filled on that stream, so the fill precedes the stream's first
        run.  Each plan keeps its own: one plan's counters must not be
        overwritten by another plan's partial sums."""
        if self.workspace_bytes == 0:
            return None
        torch = _torch()
        dev = torch.device(device)
        if stream is None:
            stream = torch.cuda.current_stream(dev)
        key = (str(dev), int(stream.cuda_stream))
        ws = self._ws.get(key)
        if ws is None:
            with torch.cuda.stream(stream):
                ws = torch.zeros(self.workspace_bytes, dtype=torch.uint8, device=dev)
            self._ws[key] = ws
        return ws

    def _resolve(self, A, workspace, stream):
        torch = _torch()
        if stream is None:
            stream = torch.cuda.current_stream(A.device)
        ws = workspace if workspace is not None else self.workspace(A.device, stream)
        nbytes = 0 if ws is None else ws.numel() * ws.element_size()
        return ws, nbytes, ctypes.c_void_p(stream.cuda_stream)

    def run(self, m, A, W, C, scales=None, workspace=None, stream=None):
        ws, nbytes, st = self._resolve(A, workspace, stream)
        _check(_lib.skinny_mm_run(self._h, m, _ptr(A), _ptr(W), _ptr(scales), _ptr(C), _ptr(ws),
                                  nbytes, st), "skinny_mm_run")

    def run_topk(self, m, A, W, logits, idx, val, topk, scales=None, workspace=None, stream=None):
        ws, nbytes, st = self._resolve(A, workspace, stream)
        _check(_lib.gemv_topk_run(self._h, m, _ptr(A), _ptr(W), _ptr(scales), _ptr(logits),
                                  _ptr(idx), _ptr(val), topk, _ptr(ws), nbytes, st),
               "gemv_topk_run")

    def run_static(self, m, A, W, C, scales=None, stream=None):
        """skinny_mm_run_static: the run without a workspace argument (the
        library's own static scratch; calls in flight at once on one GPU race)."""
        torch = _torch()
        if stream is None:
            stream = torch.cuda.current_stream(A.device)
        _check(_lib.skinny_mm_run_static(self._h, m, _ptr(A), _ptr(W), _ptr(scales), _ptr(C),
                                         ctypes.c_void_p(stream.cuda_stream)), "skinny_mm_run_static")

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _lib is not None:
            try:
                _lib.skinny_mm_plan_destroy(h)
            except Exception:  # interpreter shutdown
                pass
            self._h = None


def new_workspace(plan, device):
    """A fresh zero-filled workspace for `plan` (None when it needs none)."""
    torch = _torch()
    if plan.workspace_bytes == 0:
        return None
    return torch.zeros(plan.workspace_bytes, dtype=torch.uint8, device=device)


_plan_cache = {}


def _dense(where, **tensors):
    """The library reads every tensor as a dense row-major block: reject views
    with other strides instead of reading them wrongly."""
    for name, t in tensors.items():
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{where}: {name} must be contiguous (pass a Plan with lda/ldc for strided rows)")


def _weight_kind(W, k):
    """(dtype code, weight or codes, scales or None) of a weight for reduction
    length k.  Packed uint8 codes are Q4_0 when a row holds k/2 bytes and
    Q2_0 when it holds k/4."""
    torch = _torch()
    if isinstance(W, tuple):
        qs, d = W
        if qs.dtype not in (torch.int8, torch.uint8) or d.dtype != torch.float16 or qs.dim() != 2:
            raise TypeError("a block-quantised weight is (int8 codes [n][k] (Q8_0), or uint8 packed "
                            "4-bit codes [n][k/2] (Q4_0) or 2-bit codes [n][k/4] (Q2_0), float16 "
                            "scales [n][k/32])")
        if qs.dtype == torch.int8:
            kind = Q8_0
        else:
            kind = Q4_0 if 2 * qs.shape[1] == k else Q2_0
        if qs.shape[1] * CODES_PER_BYTE[kind] != k or tuple(d.shape) != (qs.shape[0], k // 32):
            raise ValueError(f"block-quantised weight: codes {tuple(qs.shape)} and scales {tuple(d.shape)} "
                             f"do not fit k = {k}")
        _dense("block-quantised weight", codes=qs, scales=d)
        return kind, qs, d
    _dense("weight", W=W)
    return _dtype_code(W.dtype, "W"), W, None


def get_plan(n, k, max_m, a_dtype, w_dtype, c_dtype, flags=0, tile_id=-1) -> Plan:
    key = (n, k, max_m, a_dtype, w_dtype, c_dtype, flags, tile_id)
    p = _plan_cache.get(key)
    if p is None:
        p = Plan(n, k, max_m, a_dtype, w_dtype, c_dtype, flags=flags, tile_id=tile_id)
        _plan_cache[key] = p
    return p


def mm(A, W, out=None, out_dtype=None, flags=0, tile_id=-1, max_m=None, stream=None):
    """C = A . W^T_storage for A [m][k] (f16/bf16, contiguous rows) and W [n][k]
    (same dtype), or W = (qs int8 [n][k], d f16 [n][k/32]) for Q8_0, or
    W = (qs uint8 [n][k/2] packed 4-bit codes, d f16 [n][k/32]) for Q4_0, or
    W = (qs uint8 [n][k/4] packed 2-bit codes, d f16 [n][k/32]) for Q2_0."""
    torch = _torch()
    m, k = A.shape
    wk, Wt, scales = _weight_kind(W, k)
    n = Wt.shape[0]
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype or torch.float32, device=A.device)
    _dense("mm", A=A, out=out)
    plan = get_plan(n, k, max_m or m, _dtype_code(A.dtype, "A"), wk, _dtype_code(out.dtype, "C"),
                    flags, tile_id)
    plan.run(m, A, Wt, out, scales=scales, stream=stream)
    return out


def gemv_topk(A, W, topk=10, flags=0, max_m=None, stream=None):
    """(logits f32 [m][n], idx int32 [m][topk], val f32 [m][topk]) of the router step."""
    torch = _torch()
    m, k = A.shape
    wk, Wt, scales = _weight_kind(W, k)
    n = Wt.shape[0]
    logits = torch.empty((m, n), dtype=torch.float32, device=A.device)
    idx = torch.empty((m, topk), dtype=torch.int32, device=A.device)
    val = torch.empty((m, topk), dtype=torch.float32, device=A.device)
    _dense("gemv_topk", A=A)
    plan = get_plan(n, k, max_m or m, _dtype_code(A.dtype, "A"), wk, F32, flags)
    plan.run_topk(m, A, Wt, logits, idx, val, topk, scales=scales, stream=stream)
    return logits, idx, val


def dequant_q2_0(qs, d, out=None, stream=None):
    """f16 [n][k] weight of a Q2_0-style (packed codes uint8 [n][k/4], scales) pair."""
    torch = _torch()
    n, kq = qs.shape
    if out is None:
        out = torch.empty((n, 4 * kq), dtype=torch.float16, device=qs.device)
    _dense("dequant_q2_0", qs=qs, d=d, out=out)
    _check(_lib.skinny_dequant_q2_0_run(n, 4 * kq, _ptr(qs), _ptr(d), _ptr(out), _stream(stream)),
           "skinny_dequant_q2_0_run")
    return out


def dequant_q4_0(qs, d, out=None, stream=None):
    """f16 [n][k] weight of a Q4_0-style (packed codes uint8 [n][k/2], scales) pair."""
    torch = _torch()
    n, kh = qs.shape
    if out is None:
        out = torch.empty((n, 2 * kh), dtype=torch.float16, device=qs.device)
    _dense("dequant_q4_0", qs=qs, d=d, out=out)
    _check(_lib.skinny_dequant_q4_0_run(n, 2 * kh, _ptr(qs), _ptr(d), _ptr(out), _stream(stream)),
           "skinny_dequant_q4_0_run")
    return out


def dequant_q8_0(qs, d, out=None, stream=None):
    """f16 [n][k] weight of a Q8_0-style (codes, scales) pair."""
    torch = _torch()
    n, k = qs.shape
    if out is None:
        out = torch.empty((n, k), dtype=torch.float16, device=qs.device)
    _dense("dequant_q8_0", qs=qs, d=d, out=out)
    _check(_lib.skinny_dequant_q8_0_run(n, k, _ptr(qs), _ptr(d), _ptr(out), _stream(stream)),
           "skinny_dequant_q8_0_run")
    return out


def cast_f32_bf16(x, out=None, stream=None):
    """bf16 copy of a contiguous fp32 tensor (round to nearest even), one launch."""
    torch = _torch()
    if x.dtype != torch.float32 or not x.is_contiguous():
        raise TypeError("cast_f32_bf16 takes a contiguous float32 tensor")
    if out is None:
        out = torch.empty(x.shape, dtype=torch.bfloat16, device=x.device)
    _check(_lib.skinny_cast_f32_bf16_run(x.numel(), _ptr(x), _ptr(out), _stream(stream)),
           "skinny_cast_f32_bf16_run")
    return out


def moe_combine(rows, weights, shared=None, gate=None, out=None, out_dtype=None, stream=None):
    """MoE combine: out[t] = sum_i weights[t][i] * rows[t][i] (+ gate[t] * shared[t]),
    rows [m][topk][d] float32 or bfloat16 (contiguous), weights float32 [m][topk],
    shared [m][d] like rows and gate float32 [m] (both or neither); one launch."""
    torch = _torch()
    m, topk, d = rows.shape
    if out is None:
        out = torch.empty((m, d), dtype=out_dtype or torch.float32, device=rows.device)
    _dense("moe_combine", rows=rows, weights=weights, shared=shared, gate=gate, out=out)
    if weights.dtype != torch.float32 or tuple(weights.shape) != (m, topk):
        raise ValueError("moe_combine: weights must be float32 [m][topk]")
    if shared is not None and (tuple(shared.shape) != (m, d) or shared.dtype != rows.dtype):
        raise ValueError("moe_combine: shared must be [m][d] with the rows' dtype")
    if gate is not None and (gate.dtype != torch.float32 or tuple(gate.shape) != (m,)):
        raise ValueError("moe_combine: gate must be float32 [m]")
    if tuple(out.shape) != (m, d):
        raise ValueError("moe_combine: out must be [m][d]")
    _check(_lib.skinny_moe_combine_run(m, d, topk, _ptr(rows), _ptr(weights), _ptr(shared), _ptr(gate),
                                       _dtype_code(rows.dtype, "rows"), _ptr(out),
                                       _dtype_code(out.dtype, "out"), _stream(stream)),
           "skinny_moe_combine_run")
    return out


def gate(A, W, max_m=None, out=None, stream=None):
    """Scalar gate of fp32 window rows: sigmoid(bf16(A) . W) for A [m][k] fp32
    (contiguous rows) and W bf16 [n][k] (n = 1 for one gate per row), in one
    GEMV launch that rounds A to bf16 as it loads it and applies the sigmoid
    as it stores."""
    torch = _torch()
    m, k = A.shape
    n = W.shape[0]
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=A.device)
    _dense("gate", A=A, out=out)
    plan = get_plan(n, k, max_m or m, _dtype_code(A.dtype, "A"), _dtype_code(W.dtype, "W"),
                    _dtype_code(out.dtype, "C"), EPILOGUE_SIGMOID)
    plan.run(m, A, W, out, stream=stream)
    return out
