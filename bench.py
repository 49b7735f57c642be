"""Benchmark of the weight-streaming skinny matmul on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--rounds R] [--no-sweep] [--no-cpu]

Headline step (the router workload, Strata PR #109 "What"): one decode
window sweep -- gemv_topk_run at m = 1, 2, 4, 8, 16 rows, each on a cold copy
of the bf16 router weight [256 x 5120] -- so `value` is the weight bytes the
step streams per second (weight-GB/s), with us_per_row for every m alongside
(nx_batchscale_kat: print every m, not one ratio).

Timing: inputs are resident in HBM before the timed region.  Each weight
copy comes from a rotating pool larger than the 256 MiB Infinity Cache, so
every call streams its weight from HBM.  The K timed steps are captured once
as a HIP graph (the library's runs allocate nothing and never synchronise, so
they capture) and replayed between two events after a synchronize, which
removes Python's per-launch cost from a region whose kernels take a few
microseconds each.

The roofline object is the step's dominant kernel, the router GEMV: the same
K cold-weight steps captured with only the GEMV launch of each call, timed
the same way (algorithmic bytes W + A + logits per launch / launch time).

The sweep times every workload at every m the same way (min and median over
interleaved rounds, opus r35 track A section 2's method), and reports
us_per_row, weight-GB/s, HBM and MFMA roofline fractions.

cpu_baseline: the CPU oracle (fp64, plain C) timed on this host's cores on a
bounded sample of the headline step; its outputs also check the GPU's on the
same sample (the run exits non-zero on a mismatch).

Prints one JSON line on stdout; progress goes to stderr.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense f16/bf16 MFMA, published
POOL_BYTES = 640 << 20       # rotating weight pool, > 256 MiB Infinity Cache
HEADLINE = "router_topk"
HEADLINE_MS = (1, 2, 4, 8, 16)
TOPK = 10


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--rounds", type=int, default=9)
    p.add_argument("--no-sweep", action="store_true")
    p.add_argument("--sweep-only", default=None, metavar="NAME[,NAME...]",
                   help="sweep only these workloads ('moe_combine' names the combine rows)")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--oracle-seconds", type=float, default=0.25,
                   help="CPU-oracle budget per sweep row (a sample of rows, scaled to the call)")
    p.add_argument("--tiles", default=None, metavar="WORKLOAD",
                   help="time every GEMM tile (and, for a plan that cuts k into chunks, each of "
                        "the split, one-launch and fold shapes) at every m > 16 of WORKLOAD (cold "
                        "weights and A, HIP-graph replay, min of 5) and print one JSON line per "
                        "m; the measurements behind the tile selector's cost table")
    p.add_argument("--only", default=None, metavar="WORKLOAD:M[,M...][:TILE]",
                   help="profiling mode: run one workload at the given m values (cycled; "
                        "optionally a forced GEMM tile id) --steps times eagerly, print the "
                        "timing and exit.  'copy:BYTES' runs a plain device copy of BYTES "
                        "instead (the calibration for the HBM byte counters)")
    return p.parse_args()


def run_tiles(name):
    """Time every GEMM tile at every m > 16 of one workload."""
    import torch

    import row_gemv_decode_amd as sk
    import workloads as WL

    wl = WL.WORKLOADS[name]
    inp = Inputs(wl, torch, max(wl.ms), pool_bytes=512 << 20)
    a, w, c = dtype_codes(sk, wl)
    cdt = torch.float32 if wl.c_kind == "f32" else torch.float16
    chunked = "chunks=1 " not in sk.Plan(wl.n, wl.k, max(wl.ms), a, w, c).info(max(wl.ms))
    shapes = (((sk.GEMM_SPLIT_LAUNCH, "split"), (sk.GEMM_ONE_LAUNCH, "one"), (sk.GEMM_FOLD_LAUNCH, "fold"))
              if chunked else ((0, "plain"),))
    nA = len(inp.As)
    for m in [x for x in wl.ms if x > 16]:
        C = torch.empty((m, wl.n), dtype=cdt, device="cuda")
        row = {"workload": name, "m": m, "us": {}}
        for tid, tname in enumerate(sk.gemm_tiles()):
            for flag, sname in shapes:
                plan = sk.Plan(wl.n, wl.k, max(wl.ms), a, w, c, tile_id=tid, flags=flag)
                if f"launch={sname}" not in plan.info(m):
                    continue  # the tile has no such launch shape
                ws = plan.workspace(inp.A.device)
                L = min(len(inp.W), 64)

                def fn(i, plan=plan, ws=ws):
                    W = inp.W[i % len(inp.W)]
                    A = inp.As[i % nA]
                    if wl.w_kind in BLOCK_KINDS:
                        plan.run(m, A[:m], W[0], C, scales=W[1], workspace=ws)
                    else:
                        plan.run(m, A[:m], W, C, workspace=ws)
                g = capture(torch, fn, L)
                row["us"][f"{tname}/{sname}"] = round(time_graph(torch, g, L, 5)[0], 2)
                del g
        row["selector"] = sk.Plan(wl.n, wl.k, max(wl.ms), a, w, c).info(m)
        print(json.dumps(row), flush=True)
        del C


def run_only(spec, steps, warmup):
    """Profiling mode: `steps` eager calls of one workload (m values cycled,
    each call on the next cold copy of the weight and of A), for rocprofv3
    kernel traces and counter passes; or a plain copy of a known size for
    calibration.  NAME_f16_twin runs a block-quantised workload on the f16
    dequantisation of its weight."""
    import torch

    import row_gemv_decode_amd as sk
    import workloads as WL

    parts = spec.split(":")
    if parts[0] == "copy":
        nbytes = int(parts[1])
        src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").random_()
        dst = torch.empty_like(src)
        for _ in range(warmup):
            dst.copy_(src)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        us = (time.perf_counter() - t0) * 1e6 / steps
        print(json.dumps({"only": spec, "bytes_read": nbytes, "bytes_written": nbytes,
                          "us_per_copy": round(us, 2)}), flush=True)
        return
    if parts[0] == "moe_combine":
        cfg = WL.COMBINE
        ms = [int(x) for x in parts[1].split(",")]
        topk, d = cfg["topk"], cfg["d"]
        y, w, sh, g = WL.gen_combine(max(ms), topk, d, 1000 * cfg["index"])
        copies = max(2, POOL_BYTES // (y.nbytes + w.nbytes + sh.nbytes + g.nbytes))
        dev = [tuple(torch.from_numpy(a).cuda() for a in (y, w, sh, g)) for _ in range(copies)]
        outs = {m: torch.empty((m, d), dtype=torch.float32, device="cuda") for m in ms}

        def call_c(i):
            m = ms[i % len(ms)]
            dy, dw, ds, dg = dev[i % copies]
            sk.moe_combine(dy[:m], dw[:m], ds[:m], dg[:m], out=outs[m])
        for i in range(warmup):
            call_c(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            call_c(warmup + i)
        torch.cuda.synchronize()
        us = (time.perf_counter() - t0) * 1e6 / steps
        print(json.dumps({"only": spec, "calls": steps, "us_per_call_eager": round(us, 3)}), flush=True)
        return
    twin = parts[0].endswith("_f16_twin")  # a block-quantised workload on its f16 dequantisation
    wl = WL.WORKLOADS[parts[0][:-len("_f16_twin")] if twin else parts[0]]
    ms = [int(x) for x in parts[1].split(",")]
    tile = int(parts[2]) if len(parts) > 2 else -1
    inp = Inputs(wl, torch, max(ms))
    if twin:
        import dataclasses

        deq = block_dequant(sk, wl.w_kind)
        inp.W = [deq(qs, d) for qs, d in inp.W]
        wl = dataclasses.replace(wl, w_kind="f16")
    a, w, c = dtype_codes(sk, wl)
    gate = wl.a_kind == "f32"  # the scalar gate: one GEMV, cast on load, sigmoid on store
    plan = sk.Plan(wl.n, wl.k, max(max(ms), max(wl.ms)), a, w, c, tile_id=tile,
                   flags=sk.EPILOGUE_SIGMOID if gate else 0)
    ws = plan.workspace(inp.A.device)
    cdt = torch.float32 if wl.c_kind == "f32" else torch.float16
    outs = {m: (torch.empty((m, wl.n), dtype=cdt, device="cuda"),
                torch.empty((m, TOPK), dtype=torch.int32, device="cuda"),
                torch.empty((m, TOPK), dtype=torch.float32, device="cuda")) for m in ms}

    def call(i):
        m = ms[i % len(ms)]
        C, idx, val = outs[m]
        W = inp.W[i % len(inp.W)]
        A = inp.As[i % len(inp.As)]
        if wl.w_kind in BLOCK_KINDS:
            plan.run(m, A[:m], W[0], C, scales=W[1], workspace=ws)
        elif wl.topk:
            plan.run_topk(m, A[:m], W, C, idx, val, TOPK, workspace=ws)
        else:
            plan.run(m, A[:m], W, C, workspace=ws)

    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        call(warmup + i)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    alg = sum(call_bytes(wl, m, bool(wl.topk)) for m in ms) / len(ms)
    print(json.dumps({"only": spec, "plans": {m: plan.info(m) for m in ms}, "calls": steps,
                      "us_per_call_eager": round(us, 3), "alg_bytes_per_call": alg}), flush=True)


# ---------------------------------------------------------------------------
# inputs
# ---------------------------------------------------------------------------
class Inputs:
    """Device copies of one workload: a rotating pool of (weight, A) copies.

    Every call of a timed loop takes the next copy, so neither operand is
    cache-warm: the pool (A at the largest m plus the weight, times the copy
    count) is larger than the 256 MiB Infinity Cache.  For the GEMV
    workloads A is tiny and the pool is nearly all weight; for the narrow-N
    and Q8_0 GEMMs at large M, A is most of the bytes and rotates with W.
    A is copy 0 of the rows (the headline step uses it)."""

    def __init__(self, wl, torch, max_rows, pool_bytes=POOL_BYTES):
        import numpy as np
        import workloads as WL

        self.wl = wl
        W = WL.gen_w(wl)
        A = WL.gen_a(wl, max_rows)
        self.A_bits = A
        self.W_bits = W

        def dev16(bits, kind):
            t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
            return t.view(torch.bfloat16 if kind == "bf16" else torch.float16).cuda()

        if wl.a_kind == "f32":
            self.A = torch.from_numpy(np.ascontiguousarray(A, dtype=np.float32)).cuda()
        else:
            self.A = dev16(A, wl.a_kind)
        a_bytes = self.A.numel() * self.A.element_size()
        copies = max(2, int(pool_bytes // max(1, wl.w_bytes + a_bytes)))
        self.As = [self.A] + [self.A.clone() for _ in range(copies - 1)]
        if wl.w_kind in BLOCK_KINDS:
            qs, d = W
            q0 = torch.from_numpy(qs).cuda()
            d0 = dev16(d, "f16")
            self.W = [(q0.clone(), d0.clone()) for _ in range(copies)]
        else:
            w0 = dev16(W, wl.w_kind)
            self.W = [w0.clone() for _ in range(copies)]
        self.scales = None


# block-quantised weight kinds: (codes, scales) pairs with a fused path and a
# standalone dequant to f16
BLOCK_KINDS = ("q8_0", "q4_0", "q2_0")


def block_dequant(sk, kind):
    return {"q8_0": sk.dequant_q8_0, "q4_0": sk.dequant_q4_0, "q2_0": sk.dequant_q2_0}[kind]


def dtype_codes(sk, wl):
    # fp32 rows (the gate) are rounded to bf16 by the GEMV as it loads them
    a = {"bf16": sk.BF16, "f32": sk.F32}.get(wl.a_kind, sk.F16)
    w = {"f16": sk.F16, "bf16": sk.BF16, "q8_0": sk.Q8_0, "q4_0": sk.Q4_0, "q2_0": sk.Q2_0}[wl.w_kind]
    c = sk.F32 if wl.c_kind == "f32" else sk.F16
    return a, w, c


def call_bytes(wl, m, with_topk=False):
    """Algorithmic HBM bytes of one call: the weight once, A once, C once."""
    c_elem = 4 if wl.c_kind == "f32" else 2
    a_elem = 4 if wl.a_kind == "f32" else 2
    b = wl.w_bytes + m * wl.k * a_elem + m * wl.n * c_elem
    if with_topk:
        b += m * TOPK * 8
    return b


# ---------------------------------------------------------------------------
# timing helpers
# ---------------------------------------------------------------------------
def capture(torch, fn, count):
    """Capture `count` calls fn(i) into one HIP graph.

    The caller must keep every tensor fn touches alive for as long as the
    graph is replayed: torch.cuda.graph() empties the allocator cache when a
    capture starts, so a buffer freed after an earlier capture can be unmapped
    while that earlier graph still writes to it."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(2):  # warm the path on the capture stream
            fn(i)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            for i in range(count):
                fn(i)
    torch.cuda.synchronize()
    return g


def time_graph(torch, g, count, rounds):
    """Per-call microseconds of a graph of `count` calls: (min, median) over rounds."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    g.replay()
    torch.cuda.synchronize()
    res = []
    for _ in range(rounds):
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        res.append(e0.elapsed_time(e1) * 1e3 / count)
    res.sort()
    return res[0], res[len(res) // 2]


# ---------------------------------------------------------------------------
# the headline step
# ---------------------------------------------------------------------------
class RouterStep:
    def __init__(self, sk, torch, inp):
        wl = inp.wl
        self.inp = inp
        self.plan = sk.Plan(wl.n, wl.k, max(HEADLINE_MS), sk.BF16, sk.BF16, sk.F32)
        self.ws = self.plan.workspace(inp.A.device)
        self.out = {}
        for m in HEADLINE_MS:
            self.out[m] = (torch.empty((m, wl.n), dtype=torch.float32, device="cuda"),
                           torch.empty((m, TOPK), dtype=torch.int32, device="cuda"),
                           torch.empty((m, TOPK), dtype=torch.float32, device="cuda"))
        self.calls = 0

    def call(self, m, copy):
        lg, idx, val = self.out[m]
        self.plan.run_topk(m, self.inp.A[:m], self.inp.W[copy % len(self.inp.W)], lg, idx, val, TOPK,
                           workspace=self.ws)

    def gemv_call(self, m, copy):
        # the step's dominant kernel alone: the GEMV launch of the same call
        lg, _, _ = self.out[m]
        self.plan.run(m, self.inp.A[:m], self.inp.W[copy % len(self.inp.W)], lg, workspace=self.ws)

    def step(self, i, fn=None):
        fn = fn or self.call
        base = i * len(HEADLINE_MS)
        for j, m in enumerate(HEADLINE_MS):
            fn(m, base + j)

    def bytes_per_step(self):
        return sum(call_bytes(self.inp.wl, m, True) for m in HEADLINE_MS)

    def gemv_bytes_per_step(self):
        return sum(call_bytes(self.inp.wl, m, False) for m in HEADLINE_MS)

    def weight_bytes_per_step(self):
        return self.inp.wl.w_bytes * len(HEADLINE_MS)


# ---------------------------------------------------------------------------
# sweep over every workload and m
# ---------------------------------------------------------------------------
def oracle_call_time(wl, m, inp, budget_s):
    """The CPU oracle's time for one call of this workload at m rows, on this
    host's cores, beside the GPU's: the oracle (fp64, plain C) runs on the
    first r <= m rows of the same inputs, r chosen so the sample costs about
    budget_s, and its time is scaled by m / r (every row is the same work).
    The top-k (router) and the sigmoid (gate) are part of the timed call."""
    import oracle

    threads = oracle.default_threads()
    flops_per_row = 2.0 * wl.n * wl.k
    rows = max(1, min(m, int(budget_s * 2.0e9 * threads / flops_per_row)))
    A = inp.A_bits[:rows]
    t0 = time.perf_counter()
    if wl.a_kind == "f32":
        oracle.gate(A, inp.W_bits, threads=threads)
    elif wl.w_kind in BLOCK_KINDS:
        qs, d = inp.W_bits
        oracle.mm(A, "f16", qs, wl.w_kind, w_scales=d, threads=threads)
    else:
        ref = oracle.mm(A, wl.a_kind, inp.W_bits, wl.w_kind, threads=threads)
        if wl.topk:
            oracle.topk(ref, wl.topk)
    dt = time.perf_counter() - t0
    return {"us_per_call": round(dt * 1e6 * m / rows, 1), "rows_timed": rows, "cores": threads,
            "kind": "oracle", "gpu_speedup": None}


def sweep(sk, torch, rounds, oracle_s=0.0, names=None):
    import dataclasses

    import workloads as WL

    rows = []
    for name, wl in WL.WORKLOADS.items():
        if names is not None and name not in names:
            continue
        inp = Inputs(wl, torch, max(wl.ms))
        rows += sweep_workload(sk, torch, name, wl, inp, rounds, oracle_s)
        if wl.w_kind in BLOCK_KINDS:
            # the f16 twin: the same shape on the library's own dequantisation of
            # each pool copy (the fused path's cost over a plain f16 weight)
            deq = block_dequant(sk, wl.w_kind)
            inp.W = [deq(qs, d) for qs, d in inp.W]
            twin = dataclasses.replace(wl, w_kind="f16")
            trows = sweep_workload(sk, torch, name + "_f16_twin", twin, inp, rounds, 0.0)
            by_m = {r["m"]: r for r in trows}
            for r in rows:
                if r["workload"] == name and r["m"] in by_m:
                    r["vs_f16_twin"] = round(r["us_per_call_min"] / by_m[r["m"]]["us_per_call_min"], 3)
            rows += trows
        del inp
        torch.cuda.empty_cache()
    return rows


def sweep_workload(sk, torch, name, wl, inp, rounds, oracle_s):
    """Sweep rows of one workload: each m captured as one HIP graph of L
    cold-weight calls, rounds interleaved across m, min and median kept."""
    rows = []
    a, w, c = dtype_codes(sk, wl)
    gate = wl.a_kind == "f32"  # the scalar gate: one GEMV, cast on load, sigmoid on store
    plan = sk.Plan(wl.n, wl.k, max(wl.ms), a, w, c, flags=sk.EPILOGUE_SIGMOID if gate else 0)
    ws = plan.workspace(inp.A.device)
    cdt = torch.float32 if wl.c_kind == "f32" else torch.float16
    graphs = {}
    keep = []  # every tensor a captured graph touches, alive until the graphs go
    for m in wl.ms:
        C = torch.empty((m, wl.n), dtype=cdt, device="cuda")
        keep.append(C)
        L = min(len(inp.W), 256)
        nA = len(inp.As)

        if wl.w_kind in BLOCK_KINDS:
            def fn(i, m=m, C=C):
                qs, d = inp.W[i % len(inp.W)]
                plan.run(m, inp.As[i % nA][:m], qs, C, scales=d, workspace=ws)
        elif wl.topk:
            lg = C
            idx = torch.empty((m, wl.topk), dtype=torch.int32, device="cuda")
            val = torch.empty((m, wl.topk), dtype=torch.float32, device="cuda")
            keep += [idx, val]

            def fn(i, m=m, lg=lg, idx=idx, val=val):
                plan.run_topk(m, inp.As[i % nA][:m], inp.W[i % len(inp.W)], lg, idx, val, wl.topk,
                              workspace=ws)
        else:
            def fn(i, m=m, C=C):
                plan.run(m, inp.As[i % nA][:m], inp.W[i % len(inp.W)], C, workspace=ws)
        keep.append(fn)
        graphs[m] = (capture(torch, fn, L), L)
    # interleave rounds across m (the min over interleaved rounds)
    per = {m: [] for m in wl.ms}
    for _ in range(rounds):
        for m in wl.ms:
            g, L = graphs[m]
            per[m].append(time_graph(torch, g, L, 1)[0])
    for m in wl.ms:
        ts = sorted(per[m])
        t_min, t_med = ts[0], ts[len(ts) // 2]
        nbytes = call_bytes(wl, m, bool(wl.topk))
        flops = 2.0 * m * wl.n * wl.k
        row = {
            "workload": name, "m": m, "path": plan.info(m).split()[0].split("=")[1],
            "plan": plan.info(m), "us_per_call_min": round(t_min, 3),
            "us_per_call_median": round(t_med, 3), "us_per_row": round(t_min / m, 4),
            "weight_GBps": round(wl.w_bytes / t_min / 1e3, 1),
            "hbm_frac": round(nbytes / t_min / 1e3 / HBM_PEAK_GBS, 4),
            "TFLOPs": round(flops / t_min / 1e6, 2),
            "mfma_frac": round(flops / t_min / 1e6 / MFMA_F16_PEAK_TFLOPS, 4),
        }
        if oracle_s > 0:
            row["oracle"] = oracle_call_time(wl, m, inp, oracle_s)
            row["oracle"]["gpu_speedup"] = round(row["oracle"]["us_per_call"] / t_min, 1)
        rows.append(row)
        log(f"  {name:12s} m={m:5d} {t_min:8.3f} us (med {t_med:8.3f})  us/row {t_min / m:8.4f}"
            f"  W {row['weight_GBps']:8.1f} GB/s  hbm {row['hbm_frac']:.3f}  "
            f"{row['TFLOPs']:8.1f} TF/s  mfma {row['mfma_frac']:.3f}  [{row['plan']}]")
    torch.cuda.synchronize()
    del graphs
    del keep
    return rows


def sweep_combine(sk, torch, rounds, oracle_s=0.0):
    """The MoE combine of the window: m tokens, each with its top-10 experts'
    fp32 output rows (d = 5120), fp32 routing weights, the shared expert's row
    and its gate; fp32 out.  Every call reads a different copy of the inputs
    (a pool of at least POOL_BYTES), so they come from HBM."""
    import workloads as WL

    cfg = WL.COMBINE
    topk, d, mmax = cfg["topk"], cfg["d"], max(cfg["ms"])
    y, w, sh, g = WL.gen_combine(mmax, topk, d, 1000 * cfg["index"])
    per_copy = (y.nbytes + w.nbytes + sh.nbytes + g.nbytes)
    copies = max(2, POOL_BYTES // per_copy)
    dev = [tuple(torch.from_numpy(a).cuda() for a in (y, w, sh, g)) for _ in range(copies)]
    rows, keep, graphs = [], [], {}
    for m in cfg["ms"]:
        out = torch.empty((m, d), dtype=torch.float32, device="cuda")
        keep.append(out)

        def fn(i, m=m, out=out):
            dy, dw, ds, dg = dev[i % copies]
            sk.moe_combine(dy[:m], dw[:m], ds[:m], dg[:m], out=out)
        keep.append(fn)
        L = min(copies, 256)
        graphs[m] = (capture(torch, fn, L), L)
    per = {m: [] for m in cfg["ms"]}
    for _ in range(rounds):
        for m in cfg["ms"]:
            gr, L = graphs[m]
            per[m].append(time_graph(torch, gr, L, 1)[0])
    for m in cfg["ms"]:
        ts = sorted(per[m])
        t_min, t_med = ts[0], ts[len(ts) // 2]
        nbytes = m * (topk + 1) * d * 4 + m * topk * 4 + m * 4 + m * d * 4  # rows, weights, gate, out
        row = {"workload": "moe_combine", "m": m, "path": "combine",
               "plan": f"combine topk={topk} d={d} rows=f32 out=f32 grid={(d + 511) // 512}x{m} x 1 wave",
               "us_per_call_min": round(t_min, 3), "us_per_call_median": round(t_med, 3),
               "us_per_row": round(t_min / m, 4), "GBps": round(nbytes / t_min / 1e3, 1),
               "hbm_frac": round(nbytes / t_min / 1e3 / HBM_PEAK_GBS, 4)}
        if oracle_s > 0:
            import oracle

            t0 = time.perf_counter()
            oracle.moe_combine(y[:m], w[:m], sh[:m], g[:m])
            dt = time.perf_counter() - t0
            row["oracle"] = {"us_per_call": round(dt * 1e6, 1), "rows_timed": m, "cores": 1, "kind": "oracle",
                             "gpu_speedup": round(dt * 1e6 / t_min, 1)}
        rows.append(row)
        log(f"  moe_combine  m={m:5d} {t_min:8.3f} us (med {t_med:8.3f})  {row['GBps']:8.1f} GB/s"
            f"  hbm {row['hbm_frac']:.3f}  [{row['plan']}]")
    torch.cuda.synchronize()
    del graphs, keep, dev
    torch.cuda.empty_cache()
    return rows


# ---------------------------------------------------------------------------
# CPU baseline (the oracle, as it stands) + parity on the same sample
# ---------------------------------------------------------------------------
COUNTERS = os.path.join(ROOT, "profiles", "router_gemv_topk_counters.txt")
KERNEL_SOURCES = [os.path.join(ROOT, "row_gemv_decode_amd", "csrc", f)
                  for f in ("gemv_kernel.h", "gemv_inst.hip", "device_common.h", "internal.h")]


def kernel_source_hash():
    import hashlib

    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch of the router kernel from the committed rocprofv3
    counter passes (FETCH_SIZE and WRITE_SIZE, each scaled by what it reads
    for a plain copy of known size); None when the kernel sources changed
    since the counters were taken, or when there is no measurement."""
    try:
        kv = {}
        with open(COUNTERS) as f:
            for line in f:
                if "=" in line and not line.startswith("#"):
                    k, v = line.split("=", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("kernel_source_sha256") != kernel_source_hash():
            return None
        return float(kv["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(torch, step, budget_s):
    import numpy as np

    import oracle

    wl = step.inp.wl
    A = step.inp.A_bits
    W = step.inp.W_bits
    threads = oracle.default_threads()
    # parity of the GPU's headline outputs on this sample (fresh call on copy 0)
    ok = True
    for m in HEADLINE_MS:
        step.call(m, 0)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    done_steps = 0
    while True:
        for m in HEADLINE_MS:
            ref = oracle.mm(A[:m], "bf16", W, "bf16", threads=threads)
            oi, _ = oracle.topk(ref, TOPK)
            if done_steps == 0:
                lg, idx, _ = step.out[m]
                got = lg.cpu().numpy().astype(np.float64)
                err = float(np.max(np.abs(got - ref)) / np.max(np.abs(ref)))
                gi, _ = oracle.topk(got, TOPK)
                if err > 2e-3 or not np.array_equal(idx.cpu().numpy(), gi):
                    ok = False
                    log(f"PARITY FAIL router m={m}: rel err {err:.3e}")
        done_steps += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    gbps = step.weight_bytes_per_step() * done_steps / dt / 1e9
    return {
        "value": round(gbps, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
        "cpu_model": cpu_model(),
        "sample": f"{done_steps} headline steps (router m=1,2,4,8,16 + top-10), fp64 oracle, "
                  f"{dt:.1f} s wall",
    }, ok


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.only:
        run_only(args.only, args.steps, args.warmup)
        return
    if args.tiles:
        run_tiles(args.tiles)
        return
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE={world}).", file=sys.stderr)
        sys.exit(2)

    import torch

    import row_gemv_decode_amd as sk
    import workloads as WL

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    props = torch.cuda.get_device_properties(0)
    log(f"device: {props.name}, {props.multi_processor_count} CUs")

    wl = WL.WORKLOADS[HEADLINE]
    inp = Inputs(wl, torch, max(HEADLINE_MS))
    step = RouterStep(sk, torch, inp)
    for m in HEADLINE_MS:
        log(f"  plan m={m}: {step.plan.info(m)}")

    # warmup: W untimed steps (eager), then the K-step graph
    for i in range(args.warmup):
        step.step(i)
    torch.cuda.synchronize()
    K = args.steps
    g = capture(torch, lambda i: step.step(i + args.warmup), K)

    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms_total = e0.elapsed_time(e1)
    ms_per_step = ms_total / K
    value = step.weight_bytes_per_step() / (ms_per_step / 1e3) / 1e9
    us_per_call = ms_total * 1e3 / (len(HEADLINE_MS) * K)
    log(f"headline: {ms_per_step * 1e3:.2f} us/step, {value:.1f} weight-GB/s, "
        f"{us_per_call:.3f} us/call")
    del g

    # the dominant kernel, the router GEMV, timed alone: the same K steps of
    # cold-weight calls with only the GEMV launch of each call
    gk = capture(torch, lambda i: step.step(i + args.warmup, step.gemv_call), K)
    torch.cuda.synchronize()
    e0.record()
    gk.replay()
    e1.record()
    torch.cuda.synchronize()
    us_per_launch = e0.elapsed_time(e1) * 1e3 / (len(HEADLINE_MS) * K)
    alg_bytes = step.gemv_bytes_per_step() / len(HEADLINE_MS)
    achieved = alg_bytes / us_per_launch / 1e3
    log(f"router GEMV launch alone: {us_per_launch:.3f} us, {achieved:.1f} GB/s algorithmic")
    del gk

    # per-m lines of the headline workload (same timing, one graph per m)
    per_m = []
    for m in HEADLINE_MS:
        L = min(len(inp.W), 256)
        gm = capture(torch, lambda i, m=m: step.call(m, i), L)
        t_min, t_med = time_graph(torch, gm, L, args.rounds)
        per_m.append({"m": m, "us_per_call": round(t_min, 3), "us_per_call_median": round(t_med, 3),
                      "us_per_row": round(t_min / m, 4),
                      "weight_GBps": round(wl.w_bytes / t_min / 1e3, 1)})
        del gm
    log("per m: " + ", ".join(f"m={r['m']}: {r['us_per_row']} us/row" for r in per_m))

    osec = 0.0 if args.no_cpu else args.oracle_seconds
    names = None if args.sweep_only is None else set(args.sweep_only.split(","))
    sweep_rows = []
    if not args.no_sweep:
        sweep_rows = sweep(sk, torch, args.rounds, osec, names)
        if names is None or "moe_combine" in names:
            sweep_rows += sweep_combine(sk, torch, args.rounds, osec)

    cpu = None
    parity_ok = True
    if not args.no_cpu:
        cpu, parity_ok = cpu_baseline(torch, step, args.cpu_seconds)
        log(f"cpu oracle: {cpu['value']} GB/s on {cpu['cores']} threads ({cpu['sample']})")

    derived = {}
    rows0 = [r for r in sweep_rows if r["workload"] == "gemv_k896"]
    if rows0:
        u = {r["m"]: r["us_per_row"] for r in rows0}
        if 1 in u and 8 in u:
            derived["gemv_k896_us_per_row_ratio_m1_over_m8"] = round(u[1] / u[8], 3)
    for r in sweep_rows:
        if "vs_f16_twin" in r and r["m"] > 16:
            derived[f"{r['workload']}_over_f16_twin_M{r['m']}"] = r["vs_f16_twin"]
    g2048 = [r for r in sweep_rows if r["workload"] == "wide_n7680" and r["m"] == 2048]
    if g2048:
        derived["f16_gemm_TFLOPs_M2048"] = g2048[0]["TFLOPs"]
        derived["f16_gemm_mfma_frac_M2048"] = g2048[0]["mfma_frac"]

    out = {
        "metric": "us_per_row & weight-GB/s vs m (1..16); f16 GEMM TFLOP/s at M=2048; % of peak",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "router GEMV + top-10: W bf16 [256 x 5120], A bf16 ~N(0,1), "
                        "fp32 logits; one step = m in (1,2,4,8,16), cold weight each call",
            "n": wl.n, "k": wl.k, "m_sweep": list(HEADLINE_MS), "topk": TOPK,
            "timing": "K steps captured as one HIP graph, replayed between events",
        },
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
            "kernel": "gemv_rows_kernel (the router GEMV launch of each call)",
            "alg_bytes_per_launch": round(alg_bytes, 1),
            "us_per_launch": round(us_per_launch, 4),
        },
        "cpu_baseline": cpu,
        "per_m": per_m,
        "derived": derived,
        "sweep": sweep_rows,
        "parity_ok": parity_ok,
    }
    print(json.dumps(out), flush=True)
    if not parity_ok:
        sys.exit(1)


if __name__ == "__main__":
    main()
