"""Build libskinny.so (the HIP kernels + C ABI) in-tree for gfx950 with hipcc.

Every source is compiled on each call (one hipcc process per file, in
parallel) and linked into row_gemv_decode_amd/libskinny.so.  hipcc cross-
compiles for gfx950, so this runs on a machine without a GPU.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libskinny.so")
ARCH = "gfx950"
SOURCES = ["abi.cpp", "gemv.hip", "gemm.hip", "combine.hip", "static_scratch.hip"]
# sources compiled once per kernel family member: (source, object name, defines)
INSTANCES = [
    ("gemv_inst.hip", f"gemv_{w}{'_a32' if a == 'kAF32' else ''}_t{t}",
     [f"-DGEMV_WK={wk}", f"-DGEMV_AK={a}", f"-DGEMV_T={t}",
      f"-DGEMV_LAUNCHER=launch_gemv_{w}{'_a32' if a == 'kAF32' else ''}_t{t}"])
    for w, wk, a in (("f16", "WK_F16", "kA16"), ("bf16", "WK_BF16", "kA16"), ("q8", "WK_Q8", "kA16"),
                     ("q4", "WK_Q4", "kA16"), ("q2", "WK_Q2", "kA16"), ("bf16", "WK_BF16", "kAF32"))
    for t in (1, 2)
] + [
    ("gemm_inst.hip", f"gemm_{w}", [f"-DGEMM_WK={wk}", f"-DGEMM_LAUNCHER=launch_gemm_{w}"])
    for w, wk in (("f16", "WK_F16"), ("bf16", "WK_BF16"), ("q8", "WK_Q8"), ("q4", "WK_Q4"), ("q2", "WK_Q2"))
]


def jobs():
    """Every object of the library: (source, object name, extra defines)."""
    return list(INSTANCES) + [(src, os.path.splitext(src)[0], []) for src in SOURCES]


HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-fvisibility=hidden",
    # keep fp32 arithmetic off the packed-fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _compile(job, verbose: bool) -> str:
    src, name, defines = job
    obj = os.path.join(OUT_DIR, name + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [HIPCC, *COMMON, *defines, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    todo = jobs()
    with cf.ThreadPoolExecutor(max_workers=len(todo)) as ex:
        objs = list(ex.map(lambda j: _compile(j, verbose), todo))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
