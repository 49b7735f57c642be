"""The C ABI on the host (CPU only): the library loads, exports every entry
point include/skinny.h declares, validates every argument before any HIP
call, and plans the documented GEMV split and GEMM tile for each shape.

Plans are made with num_cus = 256 (an MI355X), which skips the device query,
so nothing here touches a GPU; runs are only called with arguments that fail
validation, which returns before any launch.
"""
import ctypes
import os
import re

import pytest

import row_gemv_decode_amd as sk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "skinny.h")
L = sk.lib()


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"SKINNY_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)


def plan(n=4864, k=896, max_m=16, a=sk.F16, w=sk.F16, c=sk.F32, **kw):
    kw.setdefault("num_cus", 256)
    return sk.Plan(n, k, max_m, a, w, c, **kw)


def plan_status(**fields):
    d = sk.MMDesc(ctypes.sizeof(sk.MMDesc), sk.F16, sk.F16, sk.F32, 16, 4864, 896, 0, 0, 0, -1, 256)
    for name, value in fields.items():
        setattr(d, name, value)
    h = ctypes.c_void_p()
    st = L.skinny_mm_plan(ctypes.byref(d), ctypes.byref(h))
    if st == sk.OK:
        L.skinny_mm_plan_destroy(h)
    return st


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) == 16, names
    assert set(names) == set(sk.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_abi_version_and_status_strings():
    assert sk.abi_version() == 1
    for st in range(8):
        assert L.skinny_status_string(st)
    assert L.skinny_status_string(99) == b"unknown status"
    assert ctypes.sizeof(sk.MMDesc) == 72  # layout shared with the C header


def test_tile_table():
    names = sk.gemm_tiles()
    assert len(names) == L.skinny_gemm_tile_count() == 18
    for nm in names:
        tm, rest = nm.split("x", 1)
        tn, w = rest.split("_w")
        wm, wn = w.split("x")
        assert int(tm) % (32 * int(wm)) == 0 and int(tn) % (32 * int(wn)) == 0
    assert L.skinny_gemm_tile_name(-1) is None and L.skinny_gemm_tile_name(18) is None


@pytest.mark.parametrize("fields,status", [
    (dict(struct_size=8), sk.ERR_INVALID_ARG),
    (dict(a_dtype=sk.F32), sk.ERR_UNSUPPORTED),
    (dict(a_dtype=sk.F16, w_dtype=sk.BF16), sk.ERR_UNSUPPORTED),
    (dict(a_dtype=sk.BF16, w_dtype=sk.F16), sk.ERR_UNSUPPORTED),
    (dict(a_dtype=sk.BF16, w_dtype=sk.Q8_0), sk.ERR_UNSUPPORTED),
    (dict(c_dtype=sk.Q8_0), sk.ERR_UNSUPPORTED),
    (dict(max_m=0), sk.ERR_INVALID_ARG),
    (dict(n=0), sk.ERR_INVALID_ARG),
    (dict(k=4), sk.ERR_INVALID_ARG),
    (dict(k=900), sk.ERR_SHAPE),
    (dict(w_dtype=sk.Q8_0, k=904), sk.ERR_SHAPE),
    (dict(lda=800), sk.ERR_SHAPE),
    (dict(lda=900), sk.ERR_ALIGNMENT),
    (dict(ldc=100), sk.ERR_SHAPE),
    (dict(flags=0x40), sk.ERR_UNSUPPORTED),                           # an unknown flag
    (dict(flags=sk.GEMM_FOLD_LAUNCH), sk.OK),
    (dict(flags=sk.GEMM_FOLD_LAUNCH | sk.GEMM_SPLIT_LAUNCH), sk.ERR_INVALID_ARG),  # two shapes forced
    (dict(flags=sk.GEMM_FOLD_LAUNCH | sk.GEMM_ONE_LAUNCH), sk.ERR_INVALID_ARG),
    (dict(flags=sk.EPILOGUE_SIGMOID, a_dtype=sk.BF16, w_dtype=sk.BF16), sk.OK),  # the gate
    (dict(flags=sk.EPILOGUE_SIGMOID), sk.ERR_UNSUPPORTED),            # f16 weights: no gate
    (dict(flags=sk.EPILOGUE_SIGMOID, a_dtype=sk.BF16, w_dtype=sk.BF16, c_dtype=sk.BF16), sk.ERR_UNSUPPORTED),
    (dict(flags=sk.EPILOGUE_SIGMOID, a_dtype=sk.BF16, w_dtype=sk.BF16, max_m=17), sk.ERR_UNSUPPORTED),
    (dict(flags=sk.EPILOGUE_SIGMOID | sk.FORCE_GEMM, a_dtype=sk.BF16, w_dtype=sk.BF16), sk.ERR_UNSUPPORTED),
    (dict(flags=sk.FORCE_GEMV | sk.FORCE_GEMM), sk.ERR_INVALID_ARG),
    (dict(flags=sk.FORCE_GEMV, max_m=17), sk.ERR_INVALID_ARG),
    (dict(tile_id=18), sk.ERR_INVALID_ARG),
    (dict(tile_id=-2), sk.ERR_INVALID_ARG),
    (dict(num_cus=-1), sk.ERR_INVALID_ARG),
    (dict(max_m=64, k=(1 << 20) + 8), sk.ERR_SHAPE),          # GEMM path: k <= 2^20
    (dict(max_m=16, k=(1 << 20) + 8), sk.OK),                 # GEMV only: fine
    (dict(w_dtype=sk.Q8_0, k=32, max_m=17), sk.ERR_SHAPE),    # Q8_0 GEMM: k >= 64
    (dict(max_m=(1 << 31) - 1, n=(1 << 31) - 1), sk.ERR_SHAPE),  # GEMM: max_m * n <= 2^50
    (dict(max_m=16, n=(1 << 31) - 1), sk.OK),                # GEMV only: fine
    (dict(a_dtype=sk.F32, w_dtype=sk.BF16), sk.OK),           # fp32 rows, cast on load
    (dict(a_dtype=sk.F32, w_dtype=sk.BF16, flags=sk.EPILOGUE_SIGMOID), sk.OK),  # the one-launch gate
    (dict(a_dtype=sk.F32, w_dtype=sk.BF16, max_m=17), sk.ERR_UNSUPPORTED),      # GEMV regime only
    (dict(a_dtype=sk.F32, w_dtype=sk.BF16, flags=sk.FORCE_GEMM), sk.ERR_UNSUPPORTED),
    (dict(a_dtype=sk.F32, w_dtype=sk.F16), sk.ERR_UNSUPPORTED),                # bf16 weights only
    (dict(a_dtype=sk.F32, w_dtype=sk.Q8_0), sk.ERR_UNSUPPORTED),
    (dict(w_dtype=sk.Q8_0, k=32, flags=sk.FORCE_GEMM), sk.ERR_SHAPE),
    (dict(w_dtype=sk.Q8_0, k=32, max_m=16), sk.OK),           # GEMV only: fine
    (dict(w_dtype=sk.Q8_0, k=96, max_m=17), sk.OK),           # an odd number of scales
    (dict(ldc=4870), sk.OK),                                   # any ldc >= n
    (dict(lda=904), sk.OK),
])
def test_plan_validation(fields, status):
    assert plan_status(**fields) == status


def test_plan_null_arguments():
    h = ctypes.c_void_p()
    assert L.skinny_mm_plan(None, ctypes.byref(h)) == sk.ERR_INVALID_ARG
    d = sk.MMDesc(ctypes.sizeof(sk.MMDesc), sk.F16, sk.F16, sk.F32, 16, 64, 64, 0, 0, 0, -1, 256)
    assert L.skinny_mm_plan(ctypes.byref(d), None) == sk.ERR_INVALID_ARG
    L.skinny_mm_plan_destroy(None)  # ignored


@pytest.mark.parametrize("k,T,S", [(896, 2, 1), (5120, 2, 5), (2560, 1, 5), (8, 1, 1), (1024, 2, 1),
                                   (1032, 1, 3), (16384, 2, 16), (4600, 2, 5), (8192, 2, 8), (8200, 1, 17)])
def test_gemv_split_depends_on_k_only(k, T, S):
    for n in (1, 256, 4864):
        for m in (1, 7, 16):
            info = plan(n=n, k=k).info(m)
            assert f"T={T} S={S}" in info, info


def test_paths_by_m():
    p = plan(max_m=64)
    for m in range(1, 17):
        assert p.info(m).startswith("path=gemv")
    for m in (17, 31, 64):
        assert p.info(m).startswith("path=gemm")
    assert plan(max_m=8, flags=sk.FORCE_GEMM).info(3).startswith("path=gemm")
    assert plan(max_m=16, flags=sk.FORCE_GEMV).info(16).startswith("path=gemv")


def test_workspace_sizes():
    # router: its 5 k splits are summed inside a workgroup; the top-k is a
    # second launch: no workspace
    assert plan(n=256, k=5120, a=sk.BF16, w=sk.BF16).workspace_bytes == 0
    assert plan(n=4864, k=896).workspace_bytes == 0
    # k = 16384: 16 splits are summed across workgroups through fp32 partials
    # (16 splits x 16 rows x 256 columns), then 64 range counters (4 columns
    # per wave) rounded to 256 B
    assert plan(n=256, k=16384).workspace_bytes == 16 * 16 * 256 * 4 + 256
    # the partials are sized for the plan's largest GEMV m
    assert plan(n=256, k=16384, max_m=3).workspace_bytes == 16 * 3 * 256 * 4 + 256
    # GEMM-only plan: none
    assert plan(max_m=64, flags=sk.FORCE_GEMM).workspace_bytes == 0


@pytest.mark.parametrize("k,S,shape,reduce", [
    (896, 1, "x 4 waves", "none"),     # no split: 4 waves of separate columns
    (2048, 2, "x 8 waves", "in-block"),  # 2 splits x 4 column ranges
    (1032, 3, "x 6 waves", "in-block"),  # 3 splits x 2 ranges
    (5120, 5, "x 5 waves", "in-block"),  # the router: one range of 5 splits
    (16384, 16, "x 4 waves", "global"),  # too many splits for one workgroup
])
def test_gemv_block_shape(k, S, shape, reduce):
    info = plan(n=256, k=k).info(4)
    assert f"S={S} " in info and f"{shape} split_reduce={reduce} " in info, info


@pytest.mark.parametrize("n,k,m,tile", [
    # the measured winners on MI355X (cold weights, K = 2560)
    (7680, 2560, 150, "128x64_w2x2"),
    (7680, 2560, 306, "128x96_w4x1"),
    (7680, 2560, 448, "128x128_w2x2"),
    (7680, 2560, 520, "192x96_w6x1"),    # 3 row tiles x 80 = 240 blocks (192 x 128: 180)
    (7680, 2560, 700, "192x128_w2x2"),
    (7680, 2560, 1050, "192x192_w3x2"),  # 240 blocks (192 x 256: 180; 256 x 256: 150)
    (7680, 2560, 2048, "256x256_w2x4"),
    (96, 2560, 1024, "32x64_w1x2"),      # narrow N: four k chunks, one block per chunk
    (96, 2560, 2048, "64x64_w2x2"),      # (the same launch shape, 64-row tiles)
])
def test_tile_selector_picks(n, k, m, tile):
    assert f"name={tile} " in plan(n=n, k=k, max_m=2048).info(m)


@pytest.mark.parametrize("n,k,splits", [(96, 2560, 4), (256, 2560, 4), (512, 2560, 4), (7680, 2560, 1),
                                        (200, 512, 2), (200, 64, 1), (4864, 896, 1)])
def test_gemm_split_depends_on_n_k_only(n, k, splits):
    # narrow N splits k so that enough blocks exist at moderate M; the split
    # is fixed per plan (never per M), so rows stay M-invariant
    for m in (17, 300, 2048):
        info = plan(n=n, k=k, max_m=2048).info(m)
        assert f" chunks={splits} " in info, info


@pytest.mark.parametrize("n,k,m,cpw", [
    (4864, 896, 1, 1), (4864, 896, 8, 1), (4864, 896, 9, 2), (4864, 896, 16, 2),  # unsplit k
    (2048, 2048, 16, 2), (1024, 4096, 1, 2),                                      # k split in the workgroup
    (256, 5120, 1, 1), (256, 5120, 16, 1),                                        # the router
    (256, 16384, 1, 4), (4864, 16384, 16, 8),                                     # k split across workgroups
])
def test_gemv_columns_per_wave_by_m(n, k, m, cpw):
    # about eight waves per CU when k is split in the workgroup, sixteen (up to
    # m = 8) or eight (above) for an unsplit k, four when k is split across
    # workgroups; never more than eight columns
    assert f" cpw={cpw} " in plan(n=n, k=k).info(m)


def test_gemm_split_workspace():
    # chunks x M x N fp32 partial sums for the split launch, sized for max_m;
    # the one-launch shape needs none
    p = plan(n=512, k=2560, max_m=2048)
    assert p.workspace_bytes == 4 * 2048 * 512 * 4
    s = plan(n=512, k=2560, max_m=2048, flags=sk.GEMM_SPLIT_LAUNCH)
    assert " launch=split " in s.info(17) and s.info(17).endswith(" workspace=139264")  # 4 * 17 * 512 * 4
    o = plan(n=512, k=2560, max_m=2048, flags=sk.GEMM_ONE_LAUNCH)
    assert " launch=one " in o.info(17) and o.info(17).endswith(" workspace=0")
    # a tile without room for two accumulator sets always splits
    big = plan(n=512, k=2560, max_m=2048, flags=sk.GEMM_ONE_LAUNCH, tile_id=0)
    assert " launch=split " in big.info(300)
    # narrow N: 4 chunks of 10 k-tiles
    assert plan(n=96, k=2560, max_m=2048).workspace_bytes == 4 * 2048 * 96 * 4
    assert plan_status(flags=sk.GEMM_SPLIT_LAUNCH | sk.GEMM_ONE_LAUNCH) == sk.ERR_INVALID_ARG


def _est(info):
    return float(info.split("est_us=")[1].split()[0])


def test_tile_cost_counts_padded_tail_blocks():
    """opus r35 track A, section 2: a tile whose last row-block is mostly
    padding loses.  The cost model charges a padded tail block in full: one
    row past a multiple of the tile costs a whole extra row of blocks."""
    for tid, name in enumerate(sk.gemm_tiles()):
        tm = int(name.split("x")[0])
        p = plan(n=7680, k=2560, max_m=4096, tile_id=tid)
        m = 8 * tm
        assert _est(p.info(m + 1)) >= _est(p.info(m)), name
        # padded rows cost nothing extra until the next block boundary
        assert _est(p.info(m + 1)) == _est(p.info(m + tm)), name


def test_tile_selector_counts_the_padded_tail():
    """At M = 192 a 128-row tile leaves a half-padded second row of blocks.
    The selector charges that padding in full and still picks the 128-row
    tile, because MI355X measured it faster there (22.1 us against 29.6 us
    for 64 x 64 at N = 7680, K = 2560); one row more than a whole 128-row
    block, though, costs a whole extra round."""
    p = plan(n=7680, k=2560, max_m=2048, tile_id=6)  # 128x64_w2x2
    assert _est(p.info(192)) == _est(p.info(256))
    assert _est(p.info(129)) == _est(p.info(256))
    assert "name=128x64_w2x2 " in plan(n=7680, k=2560, max_m=2048).info(192)


def test_forced_tile_is_used():
    for tid, name in enumerate(sk.gemm_tiles()):
        assert f"tile={tid} name={name} " in plan(max_m=64, tile_id=tid).info(40)


# --- run validation (returns before any HIP call) ---------------------------
def _gpu_present():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


# The validation tests below pass made-up device pointers and expect every
# call to be rejected on the host.  Should a case ever pass validation by
# mistake it would launch on them, so they run only where no GPU is present.
fake_pointers = pytest.mark.skipif(_gpu_present(), reason="made-up pointers must never reach a GPU")

P16 = ctypes.c_void_p(1 << 20)   # aligned, never dereferenced
P16b = ctypes.c_void_p(2 << 20)
P16c = ctypes.c_void_p(3 << 20)
ODD = ctypes.c_void_p((1 << 20) + 2)


def run(p, m, A=P16, W=P16b, S=None, C=P16c, ws=None, nbytes=0):
    return L.skinny_mm_run(p.handle if p is not None else None, m, A, W, S, C, ws, nbytes, None)


@fake_pointers
def test_run_validation():
    p = plan()
    assert run(None, 1) == sk.ERR_INVALID_ARG
    assert run(p, 0) == sk.ERR_INVALID_ARG
    assert run(p, 17) == sk.ERR_INVALID_ARG
    assert run(p, 1, A=None) == sk.ERR_INVALID_ARG
    assert run(p, 1, W=None) == sk.ERR_INVALID_ARG
    assert run(p, 1, C=None) == sk.ERR_INVALID_ARG
    assert run(p, 1, S=P16) == sk.ERR_INVALID_ARG          # scales only for Q8_0
    assert run(p, 1, A=ODD) == sk.ERR_ALIGNMENT
    assert run(p, 1, W=ODD) == sk.ERR_ALIGNMENT
    assert run(p, 1, C=ODD) == sk.ERR_ALIGNMENT
    q = plan(n=512, k=2560, w=sk.Q8_0, c=sk.F16)
    assert run(q, 1) == sk.ERR_INVALID_ARG                 # Q8_0 needs scales
    assert run(q, 1, S=ODD) == sk.ERR_ALIGNMENT
    # splits summed across workgroups: partials need the workspace
    # (every case here must fail validation: the pointers are not real)
    g = plan(n=256, k=16384)
    assert run(g, 4, ws=None, nbytes=0) == sk.ERR_WORKSPACE
    assert run(g, 16, ws=P16, nbytes=g.workspace_bytes - 16) == sk.ERR_WORKSPACE  # m = 16 needs it all
    assert run(g, 4, ws=ODD, nbytes=g.workspace_bytes) == sk.ERR_ALIGNMENT
    # a GEMM that splits k needs the workspace for its partial sums
    h = plan(n=512, k=2560, max_m=64, flags=sk.GEMM_SPLIT_LAUNCH)
    assert run(h, 40, ws=None, nbytes=0) == sk.ERR_WORKSPACE
    assert run(h, 64, ws=P16, nbytes=h.workspace_bytes - 16) == sk.ERR_WORKSPACE


def topk_run(p, m, logits=P16c, idx=P16, val=P16b, k=10, ws=P16, nbytes=1 << 20):
    return L.gemv_topk_run(p.handle, m, P16, P16b, None, logits, idx, val, k, ws, nbytes, None)


@fake_pointers
def test_run_rejects_a_gemv_of_more_than_2_31_waves():
    # 2^21 k splits x 2^28 column ranges: the wave count would not fit 32 bits
    p = plan(n=(1 << 31) - 1, k=(1 << 31) - 8, a=sk.BF16, w=sk.BF16)
    assert "path=gemv" in p.info(1)
    assert run(p, 1) == sk.ERR_SHAPE


@fake_pointers
def test_topk_validation():
    p = plan(n=256, k=5120, a=sk.BF16, w=sk.BF16)
    assert topk_run(p, 1, idx=None) == sk.ERR_INVALID_ARG
    assert topk_run(p, 1, val=None) == sk.ERR_INVALID_ARG
    assert topk_run(p, 1, k=0) == sk.ERR_INVALID_ARG
    assert topk_run(p, 1, k=33) == sk.ERR_INVALID_ARG
    assert topk_run(p, 1, idx=ODD) == sk.ERR_ALIGNMENT
    g = plan(n=256, k=16384)  # splits summed across workgroups need the workspace
    assert topk_run(g, 1, ws=None, nbytes=0) == sk.ERR_WORKSPACE
    small = plan(n=8, k=64)
    assert topk_run(small, 1, k=9) == sk.ERR_INVALID_ARG   # topk > n
    f16out = plan(n=256, k=5120, a=sk.BF16, w=sk.BF16, c=sk.F16)
    assert topk_run(f16out, 1) == sk.ERR_UNSUPPORTED
    gated = plan(n=256, k=5120, a=sk.BF16, w=sk.BF16, flags=sk.EPILOGUE_SIGMOID)
    assert topk_run(gated, 1) == sk.ERR_UNSUPPORTED      # no top-k of gate values


@fake_pointers
def test_cast_validation():
    f = L.skinny_cast_f32_bf16_run
    assert f(0, P16, P16b, None) == sk.ERR_INVALID_ARG
    assert f((1 << 40) + 1, P16, P16b, None) == sk.ERR_INVALID_ARG
    assert f(8, None, P16b, None) == sk.ERR_INVALID_ARG
    assert f(8, P16, None, None) == sk.ERR_INVALID_ARG
    assert f(8, ODD, P16b, None) == sk.ERR_ALIGNMENT
    assert f(8, P16, ctypes.c_void_p((2 << 20) + 2), None) == sk.ERR_ALIGNMENT
    base = 1 << 20
    # overlapping ranges: in [base, base + 4 * count), out [o, o + 2 * count)
    assert f(64, ctypes.c_void_p(base), ctypes.c_void_p(base + 128), None) == sk.ERR_INVALID_ARG
    assert f(64, ctypes.c_void_p(base + 96), ctypes.c_void_p(base), None) == sk.ERR_INVALID_ARG


def test_row_groups_for_a_few_workgroups():
    # the gate (n = 1: one workgroup of five waves at m = 1) runs the one-row
    # kernel in m workgroup rows: fused fp32 rows at every m, no workspace
    g = plan(n=1, k=5120, a=sk.F32, w=sk.BF16, flags=sk.EPILOGUE_SIGMOID)
    assert "row_groups" not in g.info(1)
    for m in (2, 11, 16):
        info = g.info(m)
        assert f"row_groups={m} " in info and f"blocks={m} x 5 waves" in info, info
        assert "a=f32(fused) " in info and "workspace=0" in info, info
    assert g.workspace_bytes == 0
    # up to half the CUs: 64 columns at k = 5120 make 64 one-row workgroups
    assert "row_groups=2 " in plan(n=64, k=5120, a=sk.BF16, w=sk.BF16).info(2)
    assert "row_groups" not in plan(n=64, k=5120, a=sk.BF16, w=sk.BF16).info(3)
    # unsplit k: the smallest power-of-two rows per group whose groups keep
    # the launch within ten waves per CU (608 one-row waves at 608 x 896)
    shard = plan(n=608, k=896)
    for m, groups in ((2, 2), (3, 3), (4, 4), (6, 3), (8, 4), (16, 4)):
        assert f"row_groups={groups} " in shard.info(m), (m, shard.info(m))
    for m in (1, 5, 13):
        assert "row_groups" not in shard.info(m), m   # no power of two divides into few enough groups
    assert "row_groups" not in plan(n=4864, k=896).info(16)
    # never with a k split across workgroups, nor for wide grids
    assert "row_groups" not in plan(n=2, k=16384, a=sk.BF16, w=sk.BF16).info(4)
    assert "row_groups" not in plan(n=256, k=5120, a=sk.BF16, w=sk.BF16).info(2)


def test_gate_plan_info():
    g = plan(n=1, k=5120, a=sk.BF16, w=sk.BF16, flags=sk.EPILOGUE_SIGMOID)
    assert " epilogue=sigmoid " in g.info(16) and "path=gemv" in g.info(16)
    assert "epilogue" not in plan(n=1, k=5120, a=sk.BF16, w=sk.BF16).info(1)


def test_fp32_rows_shape_by_m():
    # fp32 A: fused into the GEMV while A is staged in LDS (unsplit k) or
    # m <= 10; above that (k split) the rows are cast into the workspace first
    g = plan(n=256, k=5120, a=sk.F32, w=sk.BF16)
    assert "a=f32(fused) " in g.info(10) and "workspace=0" in g.info(10)
    assert "a=f32(cast-launch) " in g.info(11)
    assert f"workspace={11 * 5120 * 2}" in g.info(11)  # 112640 B, a multiple of 256
    assert g.workspace_bytes == 16 * 5120 * 2
    assert plan(n=256, k=5120, max_m=10, a=sk.F32, w=sk.BF16).workspace_bytes == 0
    # lda > k: rows 0..m-2 at full stride, the last one up to k, rounded to 256 B
    r = plan(n=256, k=5120, lda=5128, a=sk.F32, w=sk.BF16)
    assert r.workspace_bytes == -(-(15 * 5128 + 5120) * 2 // 256) * 256
    # k split across workgroups: the cast rows follow the counters and partials
    q = plan(n=256, k=16384, a=sk.F32, w=sk.BF16)
    assert q.workspace_bytes == 16 * 16 * 256 * 4 + 256 + 16 * 16384 * 2
    # unsplit k (k <= 1024): always fused
    u = plan(n=4864, k=896, a=sk.F32, w=sk.BF16)
    assert "a=f32(fused) " in u.info(16) and u.workspace_bytes == 0


@fake_pointers
def test_moe_combine_validation():
    # every case fails before any launch (the pointers are made up)
    f = L.skinny_moe_combine_run
    P16d = ctypes.c_void_p(4 << 20)
    P4 = ctypes.c_void_p((5 << 20) + 4)  # 4-byte aligned only

    def call(m=4, d=64, topk=10, rows=P16, w=P16b, sh=None, g=None, rk=sk.F32, out=P16c, ok=sk.F32):
        return f(m, d, topk, rows, w, sh, g, rk, out, ok, None)
    assert call(rows=None) == sk.ERR_INVALID_ARG
    assert call(w=None) == sk.ERR_INVALID_ARG
    assert call(out=None) == sk.ERR_INVALID_ARG
    assert call(sh=P16d) == sk.ERR_INVALID_ARG             # shared rows without a gate
    assert call(g=P4) == sk.ERR_INVALID_ARG                # a gate without shared rows
    assert call(m=0) == sk.ERR_INVALID_ARG
    assert call(d=0) == sk.ERR_INVALID_ARG
    assert call(topk=0) == sk.ERR_INVALID_ARG
    assert call(topk=33) == sk.ERR_INVALID_ARG
    assert call(m=(1 << 31) - 1, topk=32, d=1 << 40) == sk.ERR_INVALID_ARG  # m * topk * d > 2^56
    assert call(d=12) == sk.ERR_SHAPE                      # d % 8 != 0
    assert call(rk=sk.F16) == sk.ERR_UNSUPPORTED
    assert call(ok=sk.F16) == sk.ERR_UNSUPPORTED
    assert call(rows=ODD) == sk.ERR_ALIGNMENT
    assert call(out=ODD) == sk.ERR_ALIGNMENT
    assert call(w=ctypes.c_void_p((2 << 20) + 2)) == sk.ERR_ALIGNMENT
    assert call(sh=ODD, g=P4) == sk.ERR_ALIGNMENT
    assert call(out=P16) == sk.ERR_INVALID_ARG             # out over the expert rows
    assert call(sh=P16c, g=P4) == sk.ERR_INVALID_ARG       # out over the shared rows
    assert call(w=ctypes.c_void_p((3 << 20) + 64)) == sk.ERR_INVALID_ARG  # out over the weights


@fake_pointers
@pytest.mark.parametrize("f", [L.skinny_dequant_q8_0_run, L.skinny_dequant_q4_0_run,
                               L.skinny_dequant_q2_0_run])
def test_dequant_validation(f):
    assert f(0, 64, P16, P16b, P16c, None) == sk.ERR_INVALID_ARG
    assert f(4, 16, P16, P16b, P16c, None) == sk.ERR_INVALID_ARG
    assert f(4, 80, P16, P16b, P16c, None) == sk.ERR_SHAPE
    assert f(4, 64, None, P16b, P16c, None) == sk.ERR_INVALID_ARG
    assert f(4, 64, ODD, P16b, P16c, None) == sk.ERR_ALIGNMENT


@pytest.mark.parametrize("w", [sk.Q4_0, sk.Q2_0])
@pytest.mark.parametrize("fields,status", [
    (dict(n=512, k=2560, c_dtype=sk.F16), sk.OK),
    (dict(k=2568), sk.ERR_SHAPE),                     # k % 32 != 0
    (dict(a_dtype=sk.BF16), sk.ERR_UNSUPPORTED),      # f16 rows only
    (dict(k=32, max_m=17), sk.ERR_SHAPE),             # the GEMM needs k >= 64
    (dict(k=32, max_m=16), sk.OK),                    # the GEMV does not
])
def test_packed_block_plan_validation(w, fields, status):
    assert plan_status(w_dtype=w, **fields) == status


def test_unknown_weight_dtype():
    assert plan_status(w_dtype=7) == sk.ERR_UNSUPPORTED


@fake_pointers
@pytest.mark.parametrize("w", [sk.Q4_0, sk.Q2_0])
def test_packed_block_run_needs_scales(w):
    q = plan(n=512, k=2560, w=w, c=sk.F16)
    assert run(q, 1) == sk.ERR_INVALID_ARG                 # block formats need scales
    assert run(q, 1, S=ODD) == sk.ERR_ALIGNMENT


def test_plan_info_validation():
    p = plan()
    buf = ctypes.create_string_buffer(8)
    assert L.skinny_mm_plan_info(p.handle, 0, buf, 8) == sk.ERR_INVALID_ARG
    assert L.skinny_mm_plan_info(p.handle, 1, None, 8) == sk.ERR_INVALID_ARG
    assert L.skinny_mm_plan_info(p.handle, 1, buf, 8) == sk.OK  # truncated, NUL-terminated
    assert len(buf.value) == 7


def test_binding_rejects_strided_views_before_any_call():
    # CPU tensors: each check raises before a pointer reaches the library
    torch = pytest.importorskip("torch")
    A = torch.zeros(16, 8, dtype=torch.float16).t()  # [8][16], not contiguous
    W = torch.zeros(4, 16, dtype=torch.float16)
    with pytest.raises(ValueError, match="A must be contiguous"):
        sk.mm(A, W)
    with pytest.raises(ValueError, match="W must be contiguous"):
        sk.mm(torch.zeros(2, 4, dtype=torch.float16), torch.zeros(4, 8, dtype=torch.float16)[:, ::2])
    with pytest.raises(ValueError, match="A must be contiguous"):
        sk.gemv_topk(A.to(torch.bfloat16), W.to(torch.bfloat16), topk=2)
    with pytest.raises(ValueError, match="A must be contiguous"):
        sk.gate(torch.zeros(16, 8).t(), torch.zeros(1, 16, dtype=torch.bfloat16))
    y = torch.zeros(2, 3, 16)
    with pytest.raises(ValueError, match="rows must be contiguous"):
        sk.moe_combine(y.transpose(1, 2).contiguous().transpose(1, 2), torch.zeros(2, 3))
    with pytest.raises(ValueError, match="weights must be float32"):
        sk.moe_combine(y, torch.zeros(2, 4))
    with pytest.raises(ValueError, match="shared must be"):
        sk.moe_combine(y, torch.zeros(2, 3), torch.zeros(2, 8), torch.zeros(2))


def test_fold_launch_plan_and_workspace():
    # the fold launch runs only when asked for; its workspace holds one arrival
    # counter per tile (before the chunk sums) and TM x TN fp32 per tile and chunk
    n, k, max_m = 96, 2560, 2048
    base = plan(n=n, k=k, max_m=max_m)
    fold = plan(n=n, k=k, max_m=max_m, flags=sk.GEMM_FOLD_LAUNCH)
    for m in (17, 512, 2048):
        assert "launch=fold" not in base.info(m)
        info = fold.info(m)
        assert "launch=fold" in info, info
        tile = info.split(" name=")[1].split()[0]
        tm, tn = (int(x) for x in tile.split("_")[0].split("x"))
        tiles = -(-m // tm) * -(-n // tn)
        ws = int(info.split("workspace=")[1].split()[0])
        # counters for the most tiles any foldable tile has at max_m (32 x 64: 64 x 2)
        chunks = int(info.split(" chunks=")[1].split()[0])
        assert ws >= 64 * 2 * 4 + tiles * chunks * tm * tn * 4
        assert fold.workspace_bytes >= ws
    # a tile that cannot fold (two accumulator sets do not fit) takes the split launch
    big = plan(n=n, k=k, max_m=max_m, flags=sk.GEMM_FOLD_LAUNCH, tile_id=0)
    assert "launch=split" in big.info(512)
