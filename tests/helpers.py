"""Shared test utilities: device transfer and the error metric.

Error metric (applies to every parity test): for each (batch, head) slice --
or each (sequence, head, level) state -- the largest absolute difference
divided by the largest absolute reference value in that slice; the test
reports the maximum over slices.
"""
import os

import numpy as np
import torch

_ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
# Every error a GPU parity test computes is appended here, with the test's id,
# so that a run leaves its per-case margins behind (LOGLIN_PARITY_LOG=0 turns
# this off).
PARITY_LOG = os.environ.get("LOGLIN_PARITY_LOG",
                            os.path.join(_ROOT, "test_logs", "parity_errors.tsv"))


def record(kind: str, err: float) -> None:
    """Append (test id, kind, error) to the parity log when a GPU is present."""
    if PARITY_LOG == "0" or not torch.cuda.is_available():
        return
    test = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]
    try:
        os.makedirs(os.path.dirname(PARITY_LOG), exist_ok=True)
        with open(PARITY_LOG, "a") as f:
            f.write(f"{test}\t{kind}\t{err:.3e}\n")
    except OSError:
        pass

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
    err = float(np.max(num / den))
    record("out", err)
    return err


STATE_FLOOR = 1e-30  # relative to the largest level of the pair


def state_rel_err(got, ref) -> float:
    """Error of level states [P, L, dk, dv]: per (pair, level) slice, the largest
    absolute difference over max(largest |ref| in the slice, STATE_FLOOR x the
    largest |ref| over all levels of that pair).  The floor only covers levels
    that decay has driven below what fp32 can hold next to their siblings (the
    fp64 oracle keeps ~1e-80 where fp32 holds 0, and fp32's normal range ends
    near 1e-38); every level above 1e-30 of its pair's largest is held to the
    full relative tolerance."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape and got.ndim == 4, (got.shape, ref.shape)
    P, L = ref.shape[:2]
    r = np.abs(ref).reshape(P, L, -1).max(axis=2)
    d = np.abs(got - ref).reshape(P, L, -1).max(axis=2)
    floor = STATE_FLOOR * r.max(axis=1, keepdims=True)
    den = np.maximum(np.maximum(r, floor), 1e-300)
    err = float(np.max(d / den))
    record("state", err)
    return err


def banner(msg: str) -> None:
    print(f"[gpu-case] {msg}", flush=True)
