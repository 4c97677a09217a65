"""Seeded sweep of sequence lengths, batch and head counts, lambda row lengths
and decay strengths, on the (dtype, chunk size, head dims) combinations the
other GPU tests name, against the oracle: the forward against the
materialised mask (Form A), the backward against its chain-rule gradients.
The cases are drawn once, from a fixed seed, when the module is collected,
so every run checks the same ones."""
import numpy as np
import pytest
import torch

from log_linear_token_amd import inputs as I
from log_linear_token_amd import loglin as LL
from oracle import reference as ref
from tests.helpers import TOL_BF16, TOL_F32, banner, in_dtype, slice_rel_err, to_dev

pytestmark = pytest.mark.gpu

# (dtype, C, dk, dv) of the forward and backward tests
FWD_KINDS = [("f32", 16, 16, 16), ("f32", 16, 32, 16), ("f32", 32, 16, 64), ("f32", 64, 64, 32),
             ("f32", 128, 128, 128), ("bf16", 16, 16, 32), ("bf16", 32, 32, 32),
             ("bf16", 64, 128, 64), ("bf16", 64, 64, 128), ("bf16", 128, 128, 128),
             ("bf16", 128, 64, 16), ("bf16", 64, 64, 64), ("bf16", 64, 32, 16)]
BWD_KINDS = [("f32", 16, 16, 16), ("f32", 16, 16, 32), ("f32", 32, 64, 64), ("f32", 64, 32, 64),
             ("bf16", 64, 64, 64), ("bf16", 64, 128, 64), ("bf16", 16, 16, 16),
             ("bf16", 32, 64, 128), ("bf16", 128, 128, 128), ("bf16", 16, 32, 32),
             ("bf16", 32, 128, 64), ("bf16", 128, 64, 64)]


def _draw(kinds, n, tmax, bhmax, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dtype, C, dk, dv = kinds[int(rng.integers(len(kinds)))]
        T = int(rng.integers(1, tmax + 1))
        B = int(rng.integers(1, 3))
        H = int(rng.integers(1, bhmax // B + 1))
        extra = int(rng.integers(0, 4))
        mu = float(rng.choice([-1.0, -3.0, -8.0]))
        cases.append((i, dtype, C, dk, dv, T, B, H, extra, mu))
    return cases


FWD_CASES = _draw(FWD_KINDS, 16, 2500, 6, 20261203)
BWD_CASES = _draw(BWD_KINDS, 12, 1500, 4, 20261204)


def _id(c):
    i, dtype, C, dk, dv, T, B, H, extra, mu = c
    return f"{i}-{dtype}-C{C}-d{dk}x{dv}-T{T}-B{B}H{H}-L+{extra}-mu{mu:g}"


def _inputs(B, H, T, dk, dv, L, mu, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, T, dk)) / np.sqrt(dk)
    k = rng.standard_normal((B, H, T, dk)) / np.sqrt(dk)
    v = rng.standard_normal((B, H, T, dv))
    g = rng.standard_normal((B, H, T, dv))
    a = (-np.logaddexp(0, rng.normal(mu, 0.5, (B, H, T)))).astype(np.float32).astype(np.float64)
    lam = rng.random((B, H, T, L)).astype(np.float32).astype(np.float64)
    return q, k, v, a, lam, g


def _round(x, dt):
    return to_dev(x, dt).float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("case", FWD_CASES, ids=_id)
def test_forward_shape_sweep(case):
    i, dtype, C, dk, dv, T, B, H, extra, mu = case
    L = (T - 1).bit_length() + 1 + extra
    banner(f"sweep fwd {_id(case)}")
    q, k, v, a, lam, _ = _inputs(B, H, T, dk, dv, L, mu, seed=500 + i)
    dt = in_dtype(dtype)
    out = LL.loglin_fwd_chunked(to_dev(q, dt), to_dev(k, dt), to_dev(v, dt), to_dev(a), to_dev(lam), C)
    torch.cuda.synchronize()
    want = ref.form_a(*(_round(x, dt) for x in (q, k, v)), a, lam)
    err = slice_rel_err(out.cpu().numpy(), want, 2)
    print(f"  out {err:.2e}", flush=True)
    assert err <= (TOL_BF16 if dtype == "bf16" else TOL_F32), err


@pytest.mark.parametrize("case", BWD_CASES, ids=_id)
def test_backward_shape_sweep(case):
    i, dtype, C, dk, dv, T, B, H, extra, mu = case
    L = (T - 1).bit_length() + 1 + extra
    banner(f"sweep bwd {_id(case)}")
    q, k, v, a, lam, g = _inputs(B, H, T, dk, dv, L, mu, seed=700 + i)
    dt = in_dtype(dtype)
    got = LL.loglin_bwd_chunked(to_dev(q, dt), to_dev(k, dt), to_dev(v, dt), to_dev(a), to_dev(lam),
                                to_dev(g, dt), C)
    torch.cuda.synchronize()
    want = ref.form_a_grads(*(_round(x, dt) for x in (q, k, v)), a, lam, _round(g, dt))
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    errs = {n: slice_rel_err(x.cpu().numpy(), y, 2)
            for n, x, y in zip(["dq", "dk", "dv", "dlog_decay", "dlam"], got, want)}
    print("  " + " ".join(f"{n} {e:.2e}" for n, e in errs.items()), flush=True)
    for n, e in errs.items():
        assert e <= tol, (n, e)
