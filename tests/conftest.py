import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs through the C ABI on the GPU)")


GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden_lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line


# --- helpers for the GPU tests ---------------------------------------------
def gpu_available():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False


def to_dev(bits, kind):
    """numpy f16/bf16 bit patterns (uint16), int8 codes ("i8") or packed 4-bit
    codes ("u8") -> a device tensor."""
    import numpy as np
    import torch

    if kind == "i8":
        return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.int8)).cuda()
    if kind == "u8":
        return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint8)).cuda()
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16 if kind == "bf16" else torch.float16).cuda()


def bits_of(t):
    """A device f16/bf16 tensor -> numpy uint16 bit patterns."""
    import numpy as np
    import torch

    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def rel_err(got, ref):
    """max|got - ref| / max|ref| -- the acceptance measure for floating outputs."""
    import numpy as np

    denom = float(np.max(np.abs(ref)))
    return float(np.max(np.abs(np.asarray(got, np.float64) - ref))) / (denom if denom > 0 else 1.0)


# max|C_gpu - C_ref| / max|C_ref| bar for every floating output
REL_TOL = 2e-3
