"""The benchmark's host-side contract, checked without a GPU: the one-GPU
refusal, the algorithmic byte counts its roofline divides by, the dtype codes
it hands the library, and the committed HBM counter file it reads `traffic`
from (taken only while the router kernel's sources still hash to the value
the file records)."""
import os
import subprocess
import sys

import numpy as np
import pytest

import workloads as WL

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _run_bench(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args,
                          capture_output=True, text=True, env=env, timeout=120)


@pytest.mark.parametrize("args,env", [(["--gpus", "2"], None), (["--gpus", "8", "--steps", "3"], None),
                                      ([], {"WORLD_SIZE": "4"})])
def test_more_than_one_gpu_is_refused_with_a_message(args, env):
    r = _run_bench(args, env)
    assert r.returncode == 2
    assert r.stdout == ""  # no JSON line
    assert "one GPU" in r.stderr


def test_call_bytes_count_each_operand_once():
    wl = WL.WORKLOADS["router_topk"]
    assert wl.w_bytes == 256 * 5120 * 2
    for m in (1, 16):
        assert bench.call_bytes(wl, m) == wl.w_bytes + m * 5120 * 2 + m * 256 * 4
        assert bench.call_bytes(wl, m, with_topk=True) == bench.call_bytes(wl, m) + m * 10 * 8
    gate = WL.WORKLOADS["scalar_gate"]  # fp32 rows: four bytes per A value
    assert bench.call_bytes(gate, 2) == 5120 * 2 + 2 * 5120 * 4 + 2 * 4
    q8 = WL.WORKLOADS["q8_0_n512"]  # one code byte per weight + one f16 scale per 32
    assert bench.call_bytes(q8, 4) == 512 * 2560 + 512 * 80 * 2 + 4 * 2560 * 2 + 4 * 512 * 2
    q4 = WL.WORKLOADS["q4_0_n512"]  # half a code byte per weight + one f16 scale per 32
    assert bench.call_bytes(q4, 4) == 512 * 2560 // 2 + 512 * 80 * 2 + 4 * 2560 * 2 + 4 * 512 * 2


def test_dtype_codes_follow_the_workload_kinds():
    class Codes:
        F16, BF16, F32, Q8_0, Q4_0, Q2_0 = "f16", "bf16", "f32", "q8_0", "q4_0", "q2_0"
    for wl in WL.WORKLOADS.values():
        a, w, c = bench.dtype_codes(Codes, wl)
        assert (a, w, c) == (wl.a_kind, wl.w_kind, wl.c_kind), wl.name


def test_traffic_is_read_only_while_the_kernel_sources_match(tmp_path, monkeypatch):
    # a counter file whose hash matches gives its figure; any other gives None
    f = tmp_path / "counters.txt"
    f.write_text(f"# comment = ignored\nkernel_source_sha256 = {bench.kernel_source_hash()}\n"
                 "traffic_bytes_per_launch = 12345\n")
    monkeypatch.setattr(bench, "COUNTERS", str(f))
    assert bench.measured_traffic() == 12345.0
    f.write_text("kernel_source_sha256 = 00\ntraffic_bytes_per_launch = 12345\n")
    assert bench.measured_traffic() is None
    monkeypatch.setattr(bench, "COUNTERS", str(tmp_path / "missing.txt"))
    assert bench.measured_traffic() is None


def test_committed_counters_match_the_router_kernel():
    # the committed figure must describe the kernel as it stands: at least the
    # algorithmic bytes of the mean launch over m = 1, 2, 4, 8, 16
    t = bench.measured_traffic()
    assert t is not None, "router kernel sources changed since the HBM counters were taken"
    wl = WL.WORKLOADS["router_topk"]
    alg = sum(bench.call_bytes(wl, m) for m in bench.HEADLINE_MS) / len(bench.HEADLINE_MS)
    assert alg <= t <= 1.6 * alg


def test_shard_workload_is_the_first_rows_of_the_full_weight():
    # one GPU's share of an 8-way column shard is the first n / 8 output rows
    # of the full weight, drawn from the same seed
    full, part = WL.WORKLOADS["gemv_k896"], WL.WORKLOADS["gemv_k896_shard8"]
    assert part.n * 8 == full.n and part.k == full.k
    assert np.array_equal(WL.gen_w(part), WL.gen_w(full)[:part.n])
    assert np.array_equal(WL.gen_a(part, 16), WL.gen_a(full, 16))
