"""Helpers for the GPU parity tests: device upload of the seeded inputs, the
library calls, and the error metrics with their bounds.

Tolerances (the attention library's stated parity bounds):
  float32 inputs:      O max-abs <= 1e-5, LSE max-abs <= 1e-5
  bf16 / fp16 inputs:  O max-abs <= 1e-2 and mean-abs <= 1e-3, LSE max-abs <= 1e-3
  backward:            dQ, dK, dV relative L2 (||gpu - oracle|| / ||oracle||) <= 1e-2
Inputs whose outputs are not small averages (peaked softmax rows with O
close to a single value row, so |O| reaches 4 and more; a single key; 8-bit
values times float scales, which are no 16-bit values) apply the O bounds to
what exceeds the rounding of O to its output type (half a unit in the last
place at the oracle's value, element by element): the result is exact "up to
the usual rounding", and rounding O to bf16 alone moves an element in [4, 8)
by up to 2^-6 = 0.0156, more than 1e-2.
"""

from __future__ import annotations

import sys

import numpy as np

TOL = {
    "f32": dict(o_max=1e-5, o_mean=1e-5, lse_max=1e-5),
    "bf16": dict(o_max=1e-2, o_mean=1e-3, lse_max=1e-3),
    "f16": dict(o_max=1e-2, o_mean=1e-3, lse_max=1e-3),
}
BWD_REL_L2 = 1e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_device(store: np.ndarray, dtype: str):
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(store).view(np.int16)).view(torch.bfloat16)
    elif dtype == "f16":
        t = torch.from_numpy(np.ascontiguousarray(store))
    else:
        t = torch.from_numpy(np.ascontiguousarray(store, dtype=np.float32))
    return t.cuda()


def lib():
    import exact_io_aware_fa2_amd as fa
    fa.load_library()
    return fa


def gpu_fwd(inputs: dict, dtype: str, causal: bool, scale: float):
    """Upload q, k, v, run the library forward, return device tensors (q, k, v, o, lse)."""
    import torch
    fa = lib()
    q, k, v = (to_device(inputs[n][1], dtype) for n in ("q", "k", "v"))
    o, lse = fa.fwd(q, k, v, causal, scale)
    torch.cuda.synchronize()
    return q, k, v, o, lse


def fwd_errors(o_gpu: np.ndarray, lse_gpu: np.ndarray, o_ref: np.ndarray, lse_ref: np.ndarray):
    do = np.abs(o_gpu.astype(np.float64) - o_ref)
    dl = np.abs(lse_gpu.astype(np.float64) - lse_ref)
    return dict(o_max=float(do.max()), o_mean=float(do.mean()), lse_max=float(dl.max()))


def assert_fwd_ok(err: dict, dtype: str, label: str):
    tol = TOL[dtype]
    say(f"  {label}: O max {err['o_max']:.3e} mean {err['o_mean']:.3e}  LSE max {err['lse_max']:.3e}")
    assert np.isfinite(err["o_max"]) and np.isfinite(err["lse_max"]), label
    assert err["o_max"] <= tol["o_max"], (label, err)
    assert err["o_mean"] <= tol["o_mean"], (label, err)
    assert err["lse_max"] <= tol["lse_max"], (label, err)


def rel_l2(x: np.ndarray, ref: np.ndarray) -> float:
    return float(np.linalg.norm(x.astype(np.float64) - ref) / np.linalg.norm(ref))


def half_ulp(x: np.ndarray, dtype: str) -> np.ndarray:
    """Half a unit in the last place of the 16-bit output type at |x| (float64)."""
    mant = {"bf16": 7, "f16": 10}[dtype]
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -14)))
    return 0.5 * 2.0 ** (e - mant)


def assert_fwd_ok_peaked(o_gpu, lse_gpu, o_ref, lse_ref, dtype: str, label: str):
    """The forward bounds for inputs whose outputs are not small averages
    (peaked softmax rows, a single key, dequantised 8-bit values that are no
    16-bit values): the O bounds apply to what exceeds the rounding of O to
    its output type, element by element (|O - O_ref| less half a unit in the
    last place at O_ref): max <= 1e-2 and mean of the positive part <= 1e-3;
    LSE as usual."""
    tol = TOL[dtype]
    do = np.abs(np.asarray(o_gpu, dtype=np.float64) - o_ref)
    dl = np.abs(np.asarray(lse_gpu, dtype=np.float64) - lse_ref)
    excess = do - half_ulp(o_ref, dtype)
    pos_mean = float(np.maximum(excess, 0.0).mean())
    say(f"  {label}: O max {do.max():.3e} mean {do.mean():.3e} (less the output rounding: max {excess.max():.3e}, "
        f"mean {pos_mean:.3e})  LSE max {dl.max():.3e}")
    assert np.isfinite(do).all() and np.isfinite(dl).all(), label
    assert excess.max() <= tol["o_max"], (label, float(excess.max()))
    assert pos_mean <= tol["o_mean"], (label, pos_mean)
    assert dl.max() <= tol["lse_max"], (label, float(dl.max()))
