"""Pins of the CPU oracle to things other than itself (CPU only).

Every check below compares the oracle with an independent source: the hand
examples in tests/golden/ (each file cites the page passage it follows), exact
integer / rational arithmetic, numpy's and Python's own routines (f16 casts,
BLAS dgemm, math.fsum, sorted), or closed forms.  They are chosen so that a
plausible slip in the oracle -- a dropped term, a swapped operand, a wrong
sign, an off-by-one in the block index, round-toward-zero instead of
round-to-nearest-even -- fails at least one of them.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads as WL
from conftest import golden_lines

F16_ALL = np.arange(65536, dtype=np.uint32).astype(np.uint16)


def np_f16(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def np_bf16(bits):
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def rounding_bound(k, abs_sum):
    """Rigorous bound on |fl_fp64(sum) - exact| for a sequential sum of k exact
    products: gamma_k * sum|a*w| with unit roundoff u = 2^-53."""
    u = 2.0 ** -53
    return (k * u / (1 - k * u)) * abs_sum * 1.0000001 + 1e-300


# ---------------------------------------------------------------------------
# scalar formats
# ---------------------------------------------------------------------------

def test_f16_decode_matches_numpy_all_patterns():
    got = oracle.decode(F16_ALL, "f16")
    ref = np_f16(F16_ALL)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_bf16_decode_matches_float32_upper_half_all_patterns():
    got = oracle.decode(F16_ALL, "bf16")
    ref = np_bf16(F16_ALL)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_f64_to_f16_rne_matches_numpy_on_random_and_edge_values():
    rng = np.random.default_rng(7)
    mags = np.concatenate([
        2.0 ** rng.uniform(-30, 17, 20000),        # subnormal .. overflow
        np.array([65504.0, 65519.99, 65520.0, 65535.0, 2.0 ** -24, 2.0 ** -25,
                  2.0 ** -25 * 1.0000001, 3 * 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 * (1 - 2 ** -12),
                  1.0 + 2 ** -11, 1.0 + 3 * 2 ** -11, 0.0]),
    ])
    vals = np.concatenate([mags, -mags])
    got = np.array([oracle.f64_to_f16_rne(v) for v in vals], dtype=np.uint16)
    with np.errstate(over="ignore"):
        ref = vals.astype(np.float16).view(np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(vals[i], hex(got[i]), hex(ref[i])) for i in bad[:5]]


# ---------------------------------------------------------------------------
# dequant
# ---------------------------------------------------------------------------

def test_dequant_golden_values():
    rows = [line.split() for line in golden_lines("dequant_q8_0_rne.txt")]
    for d_hex, q, exp_hex in rows:
        qs = np.zeros((1, 32), np.int8)
        qs[0, 5] = int(q)
        d = np.array([[int(d_hex, 16)]], np.uint16)
        out = oracle.dequant_q8_0(qs, d)
        assert out[0, 5] == int(exp_hex, 16), (d_hex, q, hex(out[0, 5]), exp_hex)
        assert out[0, 0] == 0  # q = 0 -> +0


def test_dequant_exhaustive_every_finite_scale_every_code():
    """All 63488 finite f16 scales x all 256 int8 codes against numpy's
    correctly rounded float64 -> float16 cast of the exact product."""
    d_all = F16_ALL[((F16_ALL >> 10) & 0x1F) != 0x1F]          # finite scales
    codes = np.arange(-128, 128, dtype=np.int16).astype(np.int8)  # 256 codes = 8 blocks
    n = d_all.size
    qs = np.broadcast_to(codes, (n, 256)).copy()
    d = np.repeat(d_all[:, None], 8, axis=1)
    got = oracle.dequant_q8_0(qs, d)
    exact = np_f16(d_all)[:, None] * codes.astype(np.float64)[None, :]
    with np.errstate(over="ignore"):
        ref = exact.astype(np.float16).view(np.uint16)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, bad[:5]


def test_dequant_uses_the_scale_of_each_32_block():
    # distinct scales per block: a wrong block index (kk/16, kk/64, kk%32) fails
    k = 128
    qs = np.ones((2, k), np.int8)
    d = WL.to_f16_bits(np.array([[1.0, 2.0, 4.0, 8.0], [0.5, 0.25, 0.125, 16.0]]))
    out = np_f16(oracle.dequant_q8_0(qs, d))
    expect = np.repeat(np_f16(d), 32, axis=1)
    assert np.array_equal(out, expect)


# ---------------------------------------------------------------------------
# matmul
# ---------------------------------------------------------------------------

def _parse_matrix(s):
    return np.array([[float(x) for x in row.split()] for row in s.split(";")])


def test_hand_example_2x3x4():
    lines = dict(line.split(":", 1) for line in golden_lines("hand_2x3x4.txt"))
    A = _parse_matrix(lines["A"])
    Wl = _parse_matrix(lines["W_logical"])
    C = _parse_matrix(lines["C"])
    for kind in ("f16", "bf16"):
        got = oracle.mm(WL.to_bits(A, kind), kind, WL.to_bits(Wl.T.copy(), kind), kind)
        assert np.array_equal(got, C), (kind, got)
    # padding k with zeros (the GPU path needs k % 8 == 0) leaves C unchanged
    Ap = np.zeros((2, 8)); Ap[:, :3] = A
    Wp = np.zeros((4, 8)); Wp[:, :3] = Wl.T
    got = oracle.mm(WL.to_f16_bits(Ap), "f16", WL.to_f16_bits(Wp), "f16")
    assert np.array_equal(got, C)


@pytest.mark.parametrize("kind", ["f16", "bf16"])
@pytest.mark.parametrize("shape", [(1, 1, 1), (2, 3, 5), (3, 7, 16), (5, 4, 33)])
def test_brute_force_exact_rationals(kind, shape):
    m, n, k = shape
    A = WL.gen_matrix((m, k), kind, ("normal", 1.0), 11 + m)
    W = WL.gen_matrix((n, k), kind, ("normal", 0.02), 13 + n)
    got = oracle.mm(A, kind, W, kind, threads=2)
    dec = np_bf16 if kind == "bf16" else np_f16
    a, w = dec(A), dec(W)
    for i in range(m):
        for j in range(n):
            exact = sum(Fraction(a[i, t]) * Fraction(w[j, t]) for t in range(k))
            abs_sum = float(sum(abs(Fraction(a[i, t]) * Fraction(w[j, t])) for t in range(k)))
            err = abs(Fraction(got[i, j]) - exact)
            assert float(err) <= rounding_bound(k, abs_sum), (i, j, float(err))


def test_brute_force_exact_rationals_q8_0():
    m, n, k = 3, 5, 64
    A = WL.gen_matrix((m, k), "f16", ("normal", 1.0), 21)
    qs, d = WL.gen_q8_0(n, k, 22, 23)
    got = oracle.mm(A, "f16", qs, "q8_0", w_scales=d)
    a = np_f16(A)
    # dequant by numpy's correctly rounded cast (independent of the oracle's)
    w = (np.repeat(np_f16(d), 32, axis=1) * qs.astype(np.float64)).astype(np.float16).astype(np.float64)
    for i in range(m):
        for j in range(n):
            exact = sum(Fraction(a[i, t]) * Fraction(w[j, t]) for t in range(k))
            abs_sum = float(sum(abs(Fraction(a[i, t]) * Fraction(w[j, t])) for t in range(k)))
            assert float(abs(Fraction(got[i, j]) - exact)) <= rounding_bound(k, abs_sum)


def _exact_int64(a_f64, w_f64):
    """Exact C for f16-valued inputs: every f16 value is an integer multiple of
    2^-24, so scaled by 2^24 both operands are int64 and C*2^48 is an exact
    int64 product (guarded against overflow)."""
    ai = np.rint(a_f64 * 2.0 ** 24).astype(np.int64)
    wi = np.rint(w_f64 * 2.0 ** 24).astype(np.int64)
    assert np.array_equal(ai.astype(np.float64) * 2.0 ** -24, a_f64)
    assert np.array_equal(wi.astype(np.float64) * 2.0 ** -24, w_f64)
    k = ai.shape[1]
    assert float(np.abs(ai).max()) * float(np.abs(wi).max()) * k < 2.0 ** 62
    c = ai @ wi.T
    ca = np.abs(ai) @ np.abs(wi).T
    return c, ca  # both scaled by 2^48


@pytest.mark.parametrize("name,rows,cols", [
    ("gemv_k896", 16, None),          # the whole m=16 output
    ("narrow_n96", 64, None),
    ("wide_n7680", 6, None),
    ("q8_0_n512", 16, None),
    ("q4_0_n512", 16, None),
    ("q2_0_n512", 16, None),
])
def test_exact_int64_at_workload_shapes(name, rows, cols):
    wl = WL.WORKLOADS[name]
    A = WL.gen_a(wl, rows)
    W = WL.gen_w(wl)
    if wl.w_kind == "q8_0":
        qs, d = W
        got = oracle.mm(A, "f16", qs, "q8_0", w_scales=d)
        w = (np.repeat(np_f16(d), 32, axis=1) * qs.astype(np.float64)).astype(np.float16).astype(np.float64)
    elif wl.w_kind == "q4_0":
        qs, d = W
        got = oracle.mm(A, "f16", qs, "q4_0", w_scales=d)
        q = np.empty((wl.n, wl.k), np.float64)
        q[:, 0::2], q[:, 1::2] = qs & 0x0F, qs >> 4
        w = (np.repeat(np_f16(d), 32, axis=1) * (q - 8.0)).astype(np.float16).astype(np.float64)
    elif wl.w_kind == "q2_0":
        qs, d = W
        got = oracle.mm(A, "f16", qs, "q2_0", w_scales=d)
        w = (np.repeat(np_f16(d), 32, axis=1) * (_unpack_q2(qs) - 2.0)).astype(np.float16).astype(np.float64)
    else:
        got = oracle.mm(A, wl.a_kind, W, wl.w_kind)
        w = np_f16(W)
    c, ca = _exact_int64(np_f16(A), w)
    exact = c.astype(np.float64) * 2.0 ** -48  # within one rounding of exact
    abs_sum = ca.astype(np.float64) * 2.0 ** -48
    bound = rounding_bound(wl.k, abs_sum) + np.abs(exact) * 2.0 ** -52
    assert np.all(np.abs(got - exact) <= bound)
    # and as a sanity check the error really is tiny relative to the output scale
    assert np.max(np.abs(got - exact)) / np.max(np.abs(exact)) < 1e-13


def test_bf16_router_against_fsum():
    """bf16 products are exact in fp64 (8 + 8 significant bits), so math.fsum
    of the products is the exactly rounded C; sampled rows of the router."""
    wl = WL.WORKLOADS["router_topk"]
    A = WL.gen_a(wl, 16)[[0, 7, 15]]
    W = WL.gen_w(wl)
    got = oracle.mm(A, "bf16", W, "bf16")
    a, w = np_bf16(A), np_bf16(W)
    for i in range(A.shape[0]):
        prods = a[i][None, :] * w           # exact
        for j in range(0, wl.n, 5):
            exact = math.fsum(prods[j].tolist())
            bound = rounding_bound(wl.k, math.fsum(np.abs(prods[j]).tolist())) + abs(exact) * 2.0 ** -52
            assert abs(got[i, j] - exact) <= bound, (i, j)


def test_matches_blas_dgemm():
    wl = WL.WORKLOADS["wide_n7680"]
    A = WL.gen_a(wl, 40)
    W = WL.gen_w(wl, n=300)
    got = oracle.mm(A, "f16", W, "f16")
    a, w = np_f16(A), np_f16(W)
    ref = a @ w.T
    abs_sum = np.abs(a) @ np.abs(w).T
    assert np.all(np.abs(got - ref) <= 2 * rounding_bound(wl.k, abs_sum))


def test_absolute_mode_is_sum_of_magnitudes():
    A = WL.gen_matrix((4, 96), "f16", ("normal", 1.0), 31)
    W = WL.gen_matrix((9, 96), "f16", ("normal", 0.1), 32)
    got = oracle.mm(A, "f16", W, "f16", absolute=True)
    _, ca = _exact_int64(np_f16(A), np_f16(W))
    exact = ca.astype(np.float64) * 2.0 ** -48
    assert np.all(np.abs(got - exact) <= rounding_bound(96, exact) + exact * 2.0 ** -52)


def test_one_hot_rows_pick_weight_columns_exactly():
    wl = WL.WORKLOADS["gemv_k896"]
    W = WL.gen_w(wl, n=50)
    A = np.zeros((3, wl.k)); A[0, 0] = 1.0; A[1, 517] = 1.0; A[2, wl.k - 1] = -1.0
    got = oracle.mm(WL.to_f16_bits(A), "f16", W, "f16")
    w = np_f16(W)
    assert np.array_equal(got[0], w[:, 0])
    assert np.array_equal(got[1], w[:, 517])
    assert np.array_equal(got[2], -w[:, wl.k - 1])


def test_zero_a_gives_positive_zero():
    W = WL.gen_matrix((7, 64), "bf16", ("normal", 0.02), 41)
    got = oracle.mm(np.zeros((2, 64), np.uint16), "bf16", W, "bf16")
    assert np.all(got == 0) and not np.any(np.signbit(got))


def test_thread_count_does_not_change_bits():
    wl = WL.WORKLOADS["gemv_k896"]
    A = WL.gen_a(wl, 5)
    W = WL.gen_w(wl, n=333)
    c1 = oracle.mm(A, "f16", W, "f16", threads=1)
    c7 = oracle.mm(A, "f16", W, "f16", threads=7)
    assert np.array_equal(c1, c7)


# ---------------------------------------------------------------------------
# top-k
# ---------------------------------------------------------------------------

def test_topk_golden():
    for line in golden_lines("topk_ties.txt"):
        body = line.split(":", 1)[1]
        vals, k, idx, top = [s.strip() for s in body.split(";")]
        logits = np.array([[float(v) for v in vals.split()]])
        gi, gv = oracle.topk(logits, int(k))
        assert gi[0].tolist() == [int(x) for x in idx.split()]
        ev = [float(x) for x in top.split()]
        assert gv[0].tolist() == ev
        assert np.signbit(gv[0]).tolist() == np.signbit(ev).tolist()


def test_topk_matches_python_sorted_with_many_ties():
    rng = np.random.default_rng(5)
    for trial in range(20):
        n = int(rng.integers(10, 300))
        k = int(rng.integers(1, min(n, 32) + 1))
        logits = rng.integers(-4, 5, size=(3, n)).astype(np.float64) / 4  # heavy ties
        logits[logits == 0] *= rng.choice([-1.0, 1.0], size=int((logits == 0).sum()))
        gi, gv = oracle.topk(logits, k)
        for r in range(3):
            order = sorted(range(n), key=lambda j: (-logits[r, j], j))[:k]
            assert gi[r].tolist() == order
            assert np.array_equal(gv[r], logits[r, order])


# --- the window-row cast and the scalar gate (Strata PR #109, "What": the bf16
# cast of the window's rows; the shared expert's gate, a GEMV then a sigmoid)

def _f32(bits):
    return np.asarray(bits, dtype=np.uint32).view(np.float32)


@pytest.mark.parametrize("value,bits", [
    (1.0, 0x3F80),
    (1.0 + 2.0 ** -8, 0x3F80),                  # halfway between 1 and 1 + 2^-7: to even
    (1.0 + 3 * 2.0 ** -8, 0x3F82),              # halfway, odd lower neighbour: up
    (1.0 + 2.0 ** -8 + 2.0 ** -20, 0x3F81),     # just above halfway: up
    (-(1.0 + 2.0 ** -8), 0xBF80),
    (-0.0, 0x8000),
    (2.0 ** -133, 0x0001),                      # smallest subnormal
    (2.0 ** -134, 0x0000),                      # halfway between 0 and it: to even (0)
    (3 * 2.0 ** -134, 0x0002),                  # halfway between 1 and 2 units: to even (2)
    (2.0 ** -126 - 2.0 ** -134, 0x0080),        # rounds up into the first normal
    ((2 - 2.0 ** -7) * 2.0 ** 127, 0x7F7F),     # largest finite
    ((2 - 2.0 ** -8) * 2.0 ** 127, 0x7F80),     # halfway past it, odd: to infinity
    (float(np.finfo(np.float32).max), 0x7F80),
])
def test_bf16_rne_hand_values(value, bits):
    assert oracle.f64_to_bf16_rne(value) == bits
    assert oracle.cast_bf16(np.array([value], np.float32))[0] == bits


def test_bf16_cast_keeps_every_finite_bf16_value():
    # each finite bf16 value, widened to fp32 by numpy's bit placement, casts back to itself
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = ((pats >> 7) & 0xFF) != 0xFF
    x = (pats.astype(np.uint32) << 16).view(np.float32)
    got = oracle.cast_bf16(x)
    assert np.array_equal(got[finite], pats[finite])


def test_bf16_cast_matches_torch_cpu_rne():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(77)
    raw = rng.integers(0, 2 ** 32, 200_000, dtype=np.uint64).astype(np.uint32)
    raw = raw[((raw >> 23) & 0xFF) != 0xFF]  # finite fp32 patterns of every size
    mags = np.ldexp(rng.random(50_000) + 0.5, rng.integers(-140, 128, 50_000)) * rng.choice([-1, 1], 50_000)
    x = np.concatenate([_f32(raw), mags.astype(np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.cast_bf16(x), want)


def test_sigmoid_closed_forms_and_library():
    special = pytest.importorskip("scipy.special")
    assert oracle.sigmoid(np.array([0.0]))[0] == 0.5
    l3 = math.log(3.0)
    y = oracle.sigmoid(np.array([l3, -l3]))
    assert abs(y[0] - 0.75) < 1e-15 and abs(y[1] - 0.25) < 1e-15
    x = np.random.default_rng(5).normal(0, 8, 10_000)
    y, yn = oracle.sigmoid(x), oracle.sigmoid(-x)
    assert np.max(np.abs(y + yn - 1.0)) < 1e-15
    assert np.max(np.abs(y - special.expit(x))) < 1e-15
    assert np.all(np.diff(oracle.sigmoid(np.sort(x))) >= 0)  # monotone


def test_gate_hand_example():
    # row 0: the cast drops 2^-8 from the first value, so a . w = 1 exactly;
    # row 1: a . w = 0, the gate is one half; row 2: -ln-free check, 3 - 3 = 0
    one_bf16 = 0x3F80
    w = np.array([[one_bf16, 0x3F00, 0x4000, 0x4040, 0, 0, 0, 0]], np.uint16)  # 1, 0.5, 2, 3
    A = np.array([[1 + 2.0 ** -8, 2.0, -0.5, 0.0, 9.0, 9.0, 9.0, 9.0],
                  [1.0, 0.0, -0.5, 0.0, 0.0, 0.0, 0.0, 0.0],
                  [0.0, 6.0, 0.0, -1.0, 0.0, 0.0, 0.0, 0.0]], np.float32)
    g = oracle.gate(A, w)
    assert g.shape == (3, 1)
    assert abs(g[0, 0] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-15
    assert g[1, 0] == 0.5 and g[2, 0] == 0.5


# --- the MoE combine ---------------------------------------------------------

def test_moe_combine_hand_example():
    # 0.5 * [1, 2, 3] + 0.25 * [4, 5, 6] + 2 * [1, 1, 1]: distinct values so a
    # transposed y (token / expert / column) or a dropped term shows
    y = np.array([[[1, 2, 3], [4, 5, 6]]], np.float32)
    w = np.array([[0.5, 0.25]], np.float32)
    out = oracle.moe_combine(y, w, np.ones((1, 3), np.float32), np.array([2.0], np.float32))
    assert out.tolist() == [[3.5, 4.25, 5.0]]
    assert oracle.moe_combine(y, w).tolist() == [[1.5, 2.25, 3.0]]  # no shared expert


def test_moe_combine_one_hot_weights_pick_an_expert_row():
    y, _, sh, _ = WL.gen_combine(3, 4, 64, 4401)
    for j in range(4):
        w = np.zeros((3, 4), np.float32)
        w[:, j] = 1.0
        out = oracle.moe_combine(y, w, sh, np.zeros(3, np.float32))
        assert np.array_equal(out, y[:, j, :].astype(np.float64))


def test_moe_combine_brute_force_exact_rationals():
    # dyadic inputs: every product and sum is exact in fp64, so the oracle
    # must equal exact rational arithmetic in Python, term by term
    rng = np.random.default_rng(4411)
    m, topk, d = 3, 5, 7
    y = (rng.integers(-64, 65, size=(m, topk, d)) / 16.0).astype(np.float32)
    w = (rng.integers(0, 33, size=(m, topk)) / 32.0).astype(np.float32)
    sh = (rng.integers(-64, 65, size=(m, d)) / 8.0).astype(np.float32)
    g = (rng.integers(0, 17, size=m) / 16.0).astype(np.float32)
    out = oracle.moe_combine(y, w, sh, g)
    for t in range(m):
        for c in range(d):
            exact = sum(Fraction(float(w[t, i])) * Fraction(float(y[t, i, c])) for i in range(topk))
            exact += Fraction(float(g[t])) * Fraction(float(sh[t, c]))
            assert Fraction(out[t, c]) == exact


def test_moe_combine_linear_in_weights_and_bf16_rows():
    # linear in w (dyadic: exact); bf16 rows give the values of their bit patterns
    rng = np.random.default_rng(4421)
    y = (rng.integers(-8, 9, size=(2, 3, 16)) / 4.0).astype(np.float32)
    w1 = (rng.integers(0, 9, size=(2, 3)) / 8.0).astype(np.float32)
    w2 = (rng.integers(0, 9, size=(2, 3)) / 8.0).astype(np.float32)
    assert np.array_equal(oracle.moe_combine(y, w1 + w2), oracle.moe_combine(y, w1) + oracle.moe_combine(y, w2))
    yb = WL.to_bits(y.astype(np.float64), "bf16")  # these values are exact in bf16
    assert np.array_equal(oracle.moe_combine(yb, w1, kind="bf16"), oracle.moe_combine(y, w1))


# ---------------------------------------------------------------------------
# Q4_0-style dequant (4-bit codes, two per byte)
# ---------------------------------------------------------------------------

def _q4_block(element, q, rows=1):
    """One 32-weight block whose codes are all 8 (weight 0) but `element`'s."""
    codes = np.full((rows, 32), 8, np.uint8)
    codes[:, element] = q
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def test_dequant_q4_0_golden_values():
    rows = [line.split() for line in golden_lines("dequant_q4_0_rne.txt")]
    for d_hex, q, element, exp_hex in rows:
        e = int(element)
        out = oracle.dequant_q4_0(_q4_block(e, int(q)), np.array([[int(d_hex, 16)]], np.uint16))
        assert out[0, e] == int(exp_hex, 16), (d_hex, q, e, hex(out[0, e]), exp_hex)
        # every other element holds code 8: a zero weight with d's sign
        others = np.delete(out[0], e)
        assert np.all(others == (0x8000 if int(d_hex, 16) & 0x8000 else 0)), (d_hex, q, e)


def test_dequant_q4_0_nibble_order():
    # element 2i in the low nibble of byte i, element 2i + 1 in the high nibble
    codes = np.arange(32, dtype=np.uint8) % 16          # element kk has code kk % 16
    packed = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)[None, :]
    assert packed[0, 0] == 0x10 and packed[0, 1] == 0x32   # elements 0,1 and 2,3
    out = np_f16(oracle.dequant_q4_0(packed, WL.to_f16_bits(np.array([[1.0]]))))
    assert np.array_equal(out[0], (codes.astype(np.float64) - 8.0))


def test_dequant_q4_0_exhaustive_every_finite_scale_every_code():
    """All 63488 finite f16 scales x all 16 codes (in both nibble positions)
    against numpy's correctly rounded float64 -> float16 cast of the exact
    product d * (q - 8)."""
    d_all = F16_ALL[((F16_ALL >> 10) & 0x1F) != 0x1F]
    codes = np.concatenate([np.arange(16), np.arange(16)[::-1]]).astype(np.uint8)  # 32 = one block
    n = d_all.size
    packed = np.broadcast_to((codes[0::2] | (codes[1::2] << 4)).astype(np.uint8), (n, 16)).copy()
    d = d_all[:, None].copy()
    got = oracle.dequant_q4_0(packed, d)
    exact = np_f16(d_all)[:, None] * (codes.astype(np.float64) - 8.0)[None, :]
    with np.errstate(over="ignore"):
        ref = exact.astype(np.float16).view(np.uint16)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, bad[:5]


def test_dequant_q4_0_uses_the_scale_of_each_32_block():
    k = 128
    packed = np.full((2, k // 2), 0x99, np.uint8)         # every code 9: weight = d
    d = WL.to_f16_bits(np.array([[1.0, 2.0, 4.0, 8.0], [0.5, 0.25, 0.125, 16.0]]))
    out = np_f16(oracle.dequant_q4_0(packed, d))
    assert np.array_equal(out, np.repeat(np_f16(d), 32, axis=1))


def test_brute_force_exact_rationals_q4_0():
    m, n, k = 3, 5, 64
    A = WL.gen_matrix((m, k), "f16", ("normal", 1.0), 31)
    qs, d = WL.gen_q4_0(n, k, 32, 33)
    got = oracle.mm(A, "f16", qs, "q4_0", w_scales=d)
    a = np_f16(A)
    # unpack the nibbles and dequant by numpy's correctly rounded cast
    q = np.empty((n, k), np.float64)
    q[:, 0::2] = qs & 0x0F
    q[:, 1::2] = qs >> 4
    w = (np.repeat(np_f16(d), 32, axis=1) * (q - 8.0)).astype(np.float16).astype(np.float64)
    for i in range(m):
        for j in range(n):
            exact = sum(Fraction(a[i, t]) * Fraction(w[j, t]) for t in range(k))
            abs_sum = float(sum(abs(Fraction(a[i, t]) * Fraction(w[j, t])) for t in range(k)))
            assert float(abs(Fraction(got[i, j]) - exact)) <= rounding_bound(k, abs_sum)


def test_q4_0_generator_codes_and_scales():
    qs, d = WL.gen_q4_0(8, 64, 41, 42)
    assert qs.shape == (8, 32) and qs.dtype == np.uint8 and d.shape == (8, 2)
    q = np.concatenate([qs & 0x0F, qs >> 4])
    assert q.min() == 0 and q.max() == 15
    assert np.all((np_f16(d) >= 1e-3 - 1e-6) & (np_f16(d) <= 2e-3 + 1e-6))


# ---------------------------------------------------------------------------
# Q2_0-style dequant (2-bit codes, four per byte)
# ---------------------------------------------------------------------------

def _unpack_q2(qs):
    """fp64 codes [rows][4 * bytes]: element kk from bits 2*(kk%4) of byte kk//4."""
    q = np.empty((qs.shape[0], 4 * qs.shape[1]), np.float64)
    for p in range(4):
        q[:, p::4] = (qs >> (2 * p)) & 0x3
    return q


def _q2_block(element, q, rows=1):
    """One 32-weight block whose codes are all 2 (weight 0) but `element`'s,
    packed byte by byte."""
    packed = np.full((rows, 8), 0xAA, np.uint8)            # 0b10101010: four codes 2
    b, p = divmod(element, 4)
    packed[:, b] = (0xAA & ~(0x3 << (2 * p)) | (q << (2 * p))) & 0xFF
    return packed


def test_dequant_q2_0_golden_values():
    rows = [line.split() for line in golden_lines("dequant_q2_0_rne.txt")]
    assert len(rows) == 17
    for d_hex, q, element, exp_hex in rows:
        e = int(element)
        with np.errstate(over="ignore"):
            out = oracle.dequant_q2_0(_q2_block(e, int(q)), np.array([[int(d_hex, 16)]], np.uint16))
        assert out[0, e] == int(exp_hex, 16), (d_hex, q, e, hex(out[0, e]), exp_hex)
        # every other element holds code 2: a zero weight with d's sign
        others = np.delete(out[0], e)
        assert np.all(others == (0x8000 if int(d_hex, 16) & 0x8000 else 0)), (d_hex, q, e)


def test_dequant_q2_0_bit_order():
    ones = WL.to_f16_bits(np.array([[1.0]]))
    # byte 0x1b = 0b00_01_10_11: element 0 (lowest bits) code 3, element 1 code 2,
    # element 2 code 1, element 3 (highest bits) code 0
    out = np_f16(oracle.dequant_q2_0(np.full((1, 8), 0x1B, np.uint8), ones))
    assert np.array_equal(out[0, :8], [1.0, 0.0, -1.0, -2.0, 1.0, 0.0, -1.0, -2.0])
    # byte 0xe4 = 0b11_10_01_00: element kk has code kk % 4
    out = np_f16(oracle.dequant_q2_0(np.full((1, 8), 0xE4, np.uint8), ones))
    assert np.array_equal(out[0], np.arange(32) % 4 - 2.0)


def test_dequant_q2_0_exhaustive_every_finite_scale_every_code():
    """All 63488 finite f16 scales x all 4 codes in each of the four bit
    positions of a byte, against numpy's correctly rounded float64 -> float16
    cast of the exact product d * (q - 2) (overflow to inf included)."""
    d_all = F16_ALL[((F16_ALL >> 10) & 0x1F) != 0x1F]
    codes = np.array([(kk % 4 + kk // 4) % 4 for kk in range(32)], np.uint8)  # byte b holds codes b..b+3 rotated
    byte = [int(codes[4 * b] | (codes[4 * b + 1] << 2) | (codes[4 * b + 2] << 4) | (codes[4 * b + 3] << 6))
            for b in range(8)]
    assert byte[:4] == [0xE4, 0x39, 0x4E, 0x93]
    n = d_all.size
    packed = np.broadcast_to(np.array(byte, np.uint8), (n, 8)).copy()
    d = d_all[:, None].copy()
    got = oracle.dequant_q2_0(packed, d)
    exact = np_f16(d_all)[:, None] * (codes.astype(np.float64) - 2.0)[None, :]
    with np.errstate(over="ignore"):
        ref = exact.astype(np.float16).view(np.uint16)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, bad[:5]


def test_dequant_q2_0_uses_the_scale_of_each_32_block():
    k = 128
    packed = np.full((2, k // 4), 0xFF, np.uint8)         # every code 3: weight = d
    d = WL.to_f16_bits(np.array([[1.0, 2.0, 4.0, 8.0], [0.5, 0.25, 0.125, 16.0]]))
    out = np_f16(oracle.dequant_q2_0(packed, d))
    assert np.array_equal(out, np.repeat(np_f16(d), 32, axis=1))


def test_brute_force_exact_rationals_q2_0():
    m, n, k = 3, 5, 64
    A = WL.gen_matrix((m, k), "f16", ("normal", 1.0), 34)
    qs, d = WL.gen_q2_0(n, k, 35, 36)
    got = oracle.mm(A, "f16", qs, "q2_0", w_scales=d)
    a = np_f16(A)
    w = (np.repeat(np_f16(d), 32, axis=1) * (_unpack_q2(qs) - 2.0)).astype(np.float16).astype(np.float64)
    for i in range(m):
        for j in range(n):
            exact = sum(Fraction(a[i, t]) * Fraction(w[j, t]) for t in range(k))
            abs_sum = float(sum(abs(Fraction(a[i, t]) * Fraction(w[j, t])) for t in range(k)))
            assert float(abs(Fraction(got[i, j]) - exact)) <= rounding_bound(k, abs_sum)


def test_q2_0_generator_codes_and_scales():
    qs, d = WL.gen_q2_0(8, 64, 43, 44)
    assert qs.shape == (8, 16) and qs.dtype == np.uint8 and d.shape == (8, 2)
    q = _unpack_q2(qs)
    assert q.min() == 0 and q.max() == 3
    assert np.all((np_f16(d) >= 1e-3 - 1e-6) & (np_f16(d) <= 2e-3 + 1e-6))
