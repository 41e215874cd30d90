"""Shared helpers of the GPU parity tests: device upload of the seeded inputs,
error statistics and the tolerances the results are held to."""
import sys

import numpy as np
import torch

import gqa_inputs as gi

# bf16 I/O: max |err| <= 2e-2 and mean |err| <= 2e-3; fp32 I/O: max |err| <= 1e-4
BF16_MAX, BF16_MEAN = 2e-2, 2e-3
FP32_MAX = 1e-4
# log-sum-exp is fp32 in both paths; bf16 inputs are exact in fp32, so only fp32
# rounding of the sums (and the bf16 rounding of P in the sum's companion) remain
LSE_TOL = 2e-3


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


def assert_lse_close(got, ref, what=""):
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin), f"{what}: lse finiteness differs"
    assert (got[~fin] == ref[~fin]).all(), f"{what}: infinite lse differs"
    if fin.any():
        mx = float(np.abs(got[fin] - ref[fin]).max())
        assert mx <= LSE_TOL, f"{what}: lse max err {mx:.3e}"
