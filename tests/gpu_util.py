"""Shared helpers of the GPU parity tests (inputs to the device, comparison
against the oracle, tolerance from the bf16 output contract)."""
import sys

import numpy as np

# Output tolerance of the bf16 path against the fp64 oracle, over real rows.
MAX_ABS = 2e-2
MEAN_ABS = 2e-3


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_gpu(arr):
    import torch
    return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to("cuda:0")


def case_to_gpu(case):
    return to_gpu(case.q), to_gpu(case.k), to_gpu(case.v)


def out_to_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def assert_close(got, ref, rows_mask=None, what="output"):
    """got, ref [..., D]; rows_mask selects the real rows (others must be 0)."""
    err = np.abs(got - ref)
    if rows_mask is not None:
        err = err[rows_mask]
    mx, mean = float(err.max()) if err.size else 0.0, float(err.mean()) if err.size else 0.0
    assert mx <= MAX_ABS and mean <= MEAN_ABS, f"{what}: max-abs {mx:.3g}, mean-abs {mean:.3g}"
    return mx, mean
