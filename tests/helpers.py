"""Shared test utilities: device transfer and the error metric.

Error metric (applies to every parity test): for each (batch, head) slice --
or each (sequence, head, level) state -- the largest absolute difference
divided by the largest absolute reference value in that slice; the test
reports the maximum over slices.
"""
import numpy as np
import torch

TOL_F32 = 1e-4   # fp32 inputs, fp32 matrix cores, fp32 accumulation
TOL_BF16 = 2e-2  # bf16 inputs, bf16 matrix cores, fp32 accumulation


def to_dev(x: np.ndarray, dtype=torch.float32) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(dtype).contiguous()


def in_dtype(cfg_dtype: str):
    return torch.bfloat16 if cfg_dtype == "bf16" else torch.float32


def slice_rel_err(got, ref, lead: int) -> float:
    """max over the first `lead` dims of max|got-ref| / max|ref|."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if got.size == 0:
        return 0.0
    n = int(np.prod(got.shape[:lead])) if lead else 1
    g = got.reshape(n, -1)
    r = ref.reshape(n, -1)
    den = np.max(np.abs(r), axis=1)
    num = np.max(np.abs(g - r), axis=1)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(num / den))


def state_rel_err(got, ref) -> float:
    """Error of level states [P, L, dk, dv]: per (pair, level) slice, the largest
    absolute difference over max(largest |ref| in the slice, 1e-6 x the largest
    |ref| over all levels of that pair).  The floor keeps levels that decay has
    driven far below fp32 range relative to their siblings (the fp64 oracle
    keeps 1e-80 where fp32 holds 0) from reading as a 100% error; such a level
    contributes nothing measurable to any output."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape and got.ndim == 4, (got.shape, ref.shape)
    P, L = ref.shape[:2]
    r = np.abs(ref).reshape(P, L, -1).max(axis=2)
    d = np.abs(got - ref).reshape(P, L, -1).max(axis=2)
    floor = 1e-6 * r.max(axis=1, keepdims=True)
    den = np.maximum(np.maximum(r, floor), 1e-300)
    return float(np.max(d / den))


def banner(msg: str) -> None:
    print(f"[gpu-case] {msg}", flush=True)
