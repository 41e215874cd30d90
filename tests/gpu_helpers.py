"""Shared helpers of the GPU parity tests: device upload of the seeded inputs,
error statistics and the tolerances the results are held to."""
import sys

import numpy as np
import torch

import gqa_inputs as gi

# bf16 I/O: max |err| <= 2e-2 and mean |err| <= 2e-3; fp32 I/O: max |err| <= 1e-4
BF16_MAX, BF16_MEAN = 2e-2, 2e-3
FP32_MAX = 1e-4
# the log-sum-exp output is held to the same bar as the attention output of its
# path: the bf16 kernels form the normaliser from the bf16-rounded weights they
# feed to the matrix cores (relative error up to 2^-9 per weight)


def say(msg: str):
    """Name the case before any GPU step, so a fault names it."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def dev_tensor(t: gi.Tensor, device):
    return gi.to_torch(t, device)


def dev_i32(a, device):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


def dev_f32(a, device):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def to_f64(x: torch.Tensor) -> np.ndarray:
    return x.detach().float().cpu().numpy().astype(np.float64)


def err_stats(got: np.ndarray, ref: np.ndarray):
    e = np.abs(got - ref)
    return float(e.max()) if e.size else 0.0, float(e.mean()) if e.size else 0.0


def assert_bf16_close(got, ref, what=""):
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    mx, mean = err_stats(got, ref)
    assert mx <= BF16_MAX and mean <= BF16_MEAN, f"{what}: max {mx:.3e} mean {mean:.3e}"
    return mx, mean


def assert_fp32_close(got, ref, what=""):
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    mx, mean = err_stats(got, ref)
    assert mx <= FP32_MAX, f"{what}: max {mx:.3e}"
    return mx, mean


def assert_lse_close(got, ref, what="", fp32=False):
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin), f"{what}: lse finiteness differs"
    assert (got[~fin] == ref[~fin]).all(), f"{what}: infinite lse differs"
    if fin.any():
        e = np.abs(got[fin] - ref[fin])
        if fp32:
            assert e.max() <= FP32_MAX, f"{what}: lse max err {e.max():.3e}"
        else:
            assert e.max() <= BF16_MAX and e.mean() <= BF16_MEAN, f"{what}: lse max {e.max():.3e} mean {e.mean():.3e}"
