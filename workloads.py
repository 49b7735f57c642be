"""Seeded synthetic inputs for the skinny-matmul workloads.

This module only draws random numbers and stores them in the input formats
(f16 / bf16 bit patterns, int8 codes); it holds none of the method's
arithmetic.  Both the CPU oracle's tests and the GPU path's tests and bench
take their inputs from here, so the two sides see identical bits.

Every draw comes from numpy's PCG64 (`numpy.random.default_rng(seed)`) in
float64 and is rounded once to the storage format (numpy's f16 cast, torch's
bf16 cast; both round to nearest even).  Seeds: W = 1000*c + 0,
A = 1000*c + 1, Q8_0 scales = 1000*c + 2, with c the workload's index.

The workloads stand in for the pages' measurements:
  gemv_k896     -- the nx_batchscale_kat page: synthetic W at the FFN inner
                   dimension k = 896, m swept to see whether W is amortised.
  gemv_k896_shard8 -- one GPU's share of it under an 8-way column shard
                   (n = 608, W = the first 608 rows of gemv_k896's W).
  router_topk   -- Strata PR #109 ("What"): the bf16 router GEMV (a 2.6 MB
                   weight) with a per-token top-10, rows = window tokens.
  narrow_n96    -- opus r35 track A, section 2, the N = 96, K = 2560 table.
  wide_n7680    -- opus r35 track A, section 2, big-N GEMMs with ragged M.
  q8_0_n512     -- opus r35 track A, section 1: a 512 x 2560 block-quantised
                   weight (the router that `dq_f16` dequantises), Q8_0-style.
  scalar_gate   -- Strata PR #109 ("What"): the shared expert's scalar gate over
                   the window's fp32 rows (n = 1, the router's k = 5120); the
                   rows are kept in fp32 (A ~N(0,1) stored as float32).
  q4_0_n512     -- the q8_0_n512 shape with a 4-bit Q4_0-style weight (the
                   4-bit block formats the Strata PR #109 page names, "Measured",
                   without a definition; the format is fixed by the oracle);
                   seed base 7.
  q2_0_n512     -- the q8_0_n512 shape with a 2-bit Q2_0-style weight (the
                   Strata PR #109 page, "Measured", names Q2_0 runs without a
                   definition; the format is fixed by the oracle); seed base 8.
  moe_combine   -- Strata PR #109 ("What"): the MoE combine over the window's
                   tokens, each with the router's top-10 experts' output rows
                   (d = 5120, the router's k), routing weights, the shared
                   expert's row and its scalar gate; seed base 6 (gen_combine).
No dataset, prompt or model from the pages exists here or is recreated.
"""
from dataclasses import dataclass
from typing import Optional, Tuple

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    index: int          # seed base c (seeds 1000*c + {0,1,2})
    n: int              # output columns (rows of the stored [n][k] weight)
    k: int              # reduction length
    a_kind: str         # "f16" | "bf16" | "f32"
    w_kind: str         # "f16" | "bf16" | "q8_0" | "q4_0" | "q2_0"
    c_kind: str         # "f32" | "f16"
    ms: Tuple[int, ...]  # row counts swept
    w_dist: Tuple       # ("uniform", lo, hi) | ("normal", sd) | (block format, dlo, dhi)
    topk: Optional[int] = None

    @property
    def w_bytes(self) -> int:
        if self.w_kind == "q8_0":
            return self.n * self.k + self.n * (self.k // 32) * 2
        if self.w_kind == "q4_0":
            return self.n * self.k // 2 + self.n * (self.k // 32) * 2
        if self.w_kind == "q2_0":
            return self.n * self.k // 4 + self.n * (self.k // 32) * 2
        return self.n * self.k * 2


WORKLOADS = {
    w.name: w
    for w in (
        Workload("gemv_k896", 0, 4864, 896, "f16", "f16", "f32", (1, 2, 4, 8, 16),
                 ("uniform", -0.05, 0.05)),
        # one GPU's share of gemv_k896 sharded by output columns over eight
        # GPUs: the same seed, so W is the first 608 rows of gemv_k896's W
        Workload("gemv_k896_shard8", 0, 608, 896, "f16", "f16", "f32", (1, 2, 4, 8, 16),
                 ("uniform", -0.05, 0.05)),
        Workload("router_topk", 1, 256, 5120, "bf16", "bf16", "f32", (1, 2, 4, 8, 16),
                 ("normal", 0.02), topk=10),
        Workload("narrow_n96", 2, 96, 2560, "f16", "f16", "f16",
                 (512, 640, 768, 1024, 1983, 2048), ("normal", 0.02)),
        Workload("wide_n7680", 3, 7680, 2560, "f16", "f16", "f16",
                 (150, 192, 306, 448, 520, 700, 1050, 1983, 2048), ("normal", 0.02)),
        Workload("q8_0_n512", 4, 512, 2560, "f16", "q8_0", "f16", (1, 4, 16, 306, 2048),
                 ("q8_0", 1e-3, 2e-3)),
        Workload("scalar_gate", 5, 1, 5120, "f32", "bf16", "f32", (1, 2, 4, 8, 16),
                 ("normal", 0.02)),
        Workload("q4_0_n512", 7, 512, 2560, "f16", "q4_0", "f16", (1, 4, 16, 306, 2048),
                 ("q4_0", 1e-3, 2e-3)),
        Workload("q2_0_n512", 8, 512, 2560, "f16", "q2_0", "f16", (1, 4, 16, 306, 2048),
                 ("q2_0", 1e-3, 2e-3)),
    )
}


def to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Store float64 draws as IEEE binary16 bit patterns (round to nearest even)."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Store float64 draws as bfloat16 bit patterns (via float32, torch's RNE cast)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def to_bits(x: np.ndarray, kind: str) -> np.ndarray:
    """The storage form: f16 / bf16 bit patterns, or float32 values for "f32"."""
    if kind == "f32":
        return np.asarray(x, dtype=np.float32)
    return to_bf16_bits(x) if kind == "bf16" else to_f16_bits(x)


def draw(shape, dist, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    if dist[0] == "uniform":
        return rng.uniform(dist[1], dist[2], size=shape)
    if dist[0] == "normal":
        return rng.normal(0.0, dist[1], size=shape)
    raise ValueError(dist)


def gen_q8_0(n: int, k: int, seed_q: int, seed_d: int, dlo=1e-3, dhi=2e-3):
    """Q8_0-style weight: int8 codes ~U{-127..127} [n][k], f16 scales ~U(dlo, dhi) [n][k/32]."""
    assert k % 32 == 0
    qs = np.random.default_rng(seed_q).integers(-127, 128, size=(n, k), dtype=np.int8)
    d = to_f16_bits(np.random.default_rng(seed_d).uniform(dlo, dhi, size=(n, k // 32)))
    return qs, d


def gen_q4_0(n: int, k: int, seed_q: int, seed_d: int, dlo=1e-3, dhi=2e-3):
    """Q4_0-style weight: 4-bit codes ~U{0..15} packed two per byte (element kk
    of a row in byte kk // 2, the low nibble for even kk) [n][k/2] uint8, and
    f16 scales ~U(dlo, dhi) [n][k/32]."""
    assert k % 32 == 0
    q = np.random.default_rng(seed_q).integers(0, 16, size=(n, k), dtype=np.uint8)
    qs = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    d = to_f16_bits(np.random.default_rng(seed_d).uniform(dlo, dhi, size=(n, k // 32)))
    return qs, d


def gen_q2_0(n: int, k: int, seed_q: int, seed_d: int, dlo=1e-3, dhi=2e-3):
    """Q2_0-style weight: 2-bit codes ~U{0..3} packed four per byte (element kk
    of a row in byte kk // 4 at bits 2 * (kk % 4)) [n][k/4] uint8, and f16
    scales ~U(dlo, dhi) [n][k/32]."""
    assert k % 32 == 0
    q = np.random.default_rng(seed_q).integers(0, 4, size=(n, k), dtype=np.uint8)
    qs = (q[:, 0::4] | (q[:, 1::4] << 2) | (q[:, 2::4] << 4) | (q[:, 3::4] << 6)).astype(np.uint8)
    d = to_f16_bits(np.random.default_rng(seed_d).uniform(dlo, dhi, size=(n, k // 32)))
    return qs, d


def gen_w(wl: Workload, n: Optional[int] = None):
    """The workload's stored weight [n][k]: uint16 bits, or (qs, d) for the block formats."""
    n = wl.n if n is None else n
    c = wl.index
    if wl.w_kind == "q8_0":
        return gen_q8_0(n, wl.k, 1000 * c + 0, 1000 * c + 2, wl.w_dist[1], wl.w_dist[2])
    if wl.w_kind == "q4_0":
        return gen_q4_0(n, wl.k, 1000 * c + 0, 1000 * c + 2, wl.w_dist[1], wl.w_dist[2])
    if wl.w_kind == "q2_0":
        return gen_q2_0(n, wl.k, 1000 * c + 0, 1000 * c + 2, wl.w_dist[1], wl.w_dist[2])
    return to_bits(draw((n, wl.k), wl.w_dist, 1000 * c + 0), wl.w_kind)


def gen_a(wl: Workload, rows: int) -> np.ndarray:
    """A [rows][k] ~N(0,1) as bits (float32 values for an "f32" workload).  Smaller m take a prefix of these rows, so the
    same token rows appear at every m."""
    return to_bits(draw((rows, wl.k), ("normal", 1.0), 1000 * wl.index + 1), wl.a_kind)


def gen_matrix(shape, kind: str, dist, seed: int) -> np.ndarray:
    """A free-form f16 / bf16 matrix for tests at other shapes."""
    return to_bits(draw(shape, dist, seed), kind)


# the MoE combine's workload: top-10 experts per token, rows of the router's
# k = 5120, the window's token counts
COMBINE = {"index": 6, "topk": 10, "d": 5120, "ms": (1, 2, 4, 8, 16)}


def gen_combine(m: int, topk: int, d: int, seed: int, kind: str = "f32"):
    """Inputs of the MoE combine for m tokens: expert output rows y [m][topk][d]
    ~N(0, 0.5), routing weights w [m][topk] ~U(0, 0.2) (fp32), the shared
    expert's rows s [m][d] ~N(0, 0.5) and its gate g [m] ~U(0, 1) (fp32); y
    and s stored as `kind` ("f32" values or "bf16" bits).  Seeds seed + 0..3;
    smaller m are not prefixes (draw for the largest m and slice)."""
    y = to_bits(draw((m, topk, d), ("normal", 0.5), seed), kind)
    w = np.random.default_rng(seed + 1).uniform(0.0, 0.2, size=(m, topk)).astype(np.float32)
    sh = to_bits(draw((m, d), ("normal", 0.5), seed + 2), kind)
    g = np.random.default_rng(seed + 3).uniform(0.0, 1.0, size=m).astype(np.float32)
    return y, w, sh, g
