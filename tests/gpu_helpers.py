"""Shared helpers of the GPU parity tests: device upload of the seeded inputs,
error statistics and the tolerances the results are held to."""
import sys

import numpy as np
import torch

import gqa_inputs as gi

# bf16 I/O: max |err| <= 2e-2 and mean |err| <= 2e-3; fp32 I/O: max |err| <= 1e-4
BF16_MAX, BF16_MEAN = 2e-2, 2e-3
FP32_MAX = 1e-4
# Log-sum-exp of the bf16 paths.  The kernels form lse = m + ln Z from the same
# fp32 scores the weights come from (bf16 products are exact in fp32, 64-term
# fp32 sums: <= 64 u |x| with u = 2^-24, about 3e-5 for these inputs), weights
# exp2(x c - m) of unrounded fp32 arguments (<= 4 u relative each, argument
# rounding plus the exp2 instruction), a normaliser Z summed in fp32 from those
# unrounded weights, and an fp32 log2.  No normaliser is one long chain of adds:
# the prefill sums 16 keys per lane per tile in chunks of 4 and adds a running
# sum once per 32-key half tile; the decode sums a tile per lane, adds a running
# sum once per tile and merges at most 64 split partials.  So the longest chain
# in a row with n visible keys is below n/16 + 40 adds, and for positive terms
# the relative error of Z is at most that many u.  With the log2 and the final
# multiply (2^-22 (1 + |lse|)), a row of n = 131072 keys (the longest decode
# here) and |lse| <= 30: |err| <= (8192 + 40 + 4) u + 64 u |x| + 2^-22 * 31
# ~= 5.2e-4.  Held to max 1e-3; the mean, a sum of independent roundings, far
# below that, to 1e-4.
LSE_BF16_MAX, LSE_BF16_MEAN = 1e-3, 1e-4


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
        print(f"[gpu]   {what}: lse max err {e.max():.3e} mean err {e.mean():.3e}", flush=True)
        if fp32:
            assert e.max() <= FP32_MAX, f"{what}: lse max err {e.max():.3e}"
        else:
            assert e.max() <= LSE_BF16_MAX and e.mean() <= LSE_BF16_MEAN, \
                f"{what}: lse max {e.max():.3e} mean {e.mean():.3e}"


# Gradients (backward of the prefill) are compared relative to the largest
# reference magnitude of the tensor: the bf16 kernels round the weights P and
# the logit gradients dS to bf16 before the matrix products (relative 2^-9
# each, independent signs, fp32 sums) and round the result to bf16 (2^-9),
# and D = <dO, o> comes from the bf16 forward output; max |err| <= 1e-2 and
# mean |err| <= 1e-3 of max |ref| hold that with room.  fp32 path: 1e-4.
GRAD_BF16_MAX, GRAD_BF16_MEAN = 1e-2, 1e-3
GRAD_FP32_MAX = 1e-4


def assert_grad_close(got, ref, what="", fp32=False):
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    scale = max(float(np.abs(ref).max()) if ref.size else 0.0, 1e-30)
    mx, mean = err_stats(got, ref)
    print(f"[gpu]   {what}: max|ref| {scale:.3e}  max err {mx / scale:.2e}  mean err {mean / scale:.2e} (relative)",
          flush=True)
    if fp32:
        assert mx <= GRAD_FP32_MAX * max(scale, 1.0), f"{what}: max {mx:.3e} (scale {scale:.3e})"
    else:
        assert mx <= GRAD_BF16_MAX * scale and mean <= GRAD_BF16_MEAN * scale, \
            f"{what}: max {mx:.3e} mean {mean:.3e} (scale {scale:.3e})"
    return mx, mean


def assert_dsinks_close(got, ref, ref_abs, what="", fp32=False):
    """dsinks[h] sums -exp(s_h - lse) D over every row; D = <dO, o> carries the
    rounding of the bf16 forward output (about 2^-9 of sum |dO o| per row), so
    the error is held against ref_abs[h], the sum of the terms' magnitudes."""
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    bound = (GRAD_FP32_MAX * np.maximum(ref_abs, 1.0)) if fp32 else GRAD_BF16_MAX * ref_abs
    worst = float((err / np.maximum(ref_abs, 1e-30)).max())
    print(f"[gpu]   {what}: max err / sum|terms| {worst:.2e}", flush=True)
    assert (err <= bound).all(), f"{what}: err {err.max():.3e}, sum|terms| {ref_abs.min():.3e}..{ref_abs.max():.3e}"
