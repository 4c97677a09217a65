"""Seeded sweep of sequence lengths, batch and head counts, lambda row lengths
and decay strengths, on the (dtype, chunk size, head dims) combinations the
other GPU tests name, against the oracle: the forward against the
materialised mask (Form A), the backward against its chain-rule gradients,
the log-linear Gated DeltaNet forward against its masked form, the prefill
hand-over against the recurrence's level states (slots that are not live
exactly zero), and decode steps from pre-filled states against the
recurrence.  The cases are drawn once, from fixed seeds, when the
module is collected, so every run checks the same ones."""
import numpy as np
import pytest
import torch

from log_linear_token_amd import inputs as I
from log_linear_token_amd import loglin as LL
from oracle import reference as ref
from tests.helpers import TOL_BF16, TOL_F32, banner, in_dtype, slice_rel_err, state_rel_err, to_dev

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


# the log-linear Gated DeltaNet forward: (dtype, dk, dv) of its other tests
GDN_KINDS = [("f32", 64, 64), ("f32", 64, 16), ("f32", 128, 32), ("f32", 128, 64), ("f32", 64, 32),
             ("bf16", 128, 64), ("bf16", 64, 64), ("bf16", 128, 16), ("bf16", 64, 32)]


def _draw_gdn(n, tmax, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dtype, dk, dv = GDN_KINDS[int(rng.integers(len(GDN_KINDS)))]
        out.append((i, dtype, dk, dv, int(rng.integers(1, tmax + 1)), int(rng.integers(1, 3)),
                    int(rng.integers(1, 3)), int(rng.integers(0, 3)),
                    str(rng.choice(["base", "unit", "weak"]))))
    return out


GDN_CASES = _draw_gdn(8, 1800, 20261205)


@pytest.mark.parametrize("case", GDN_CASES,
                         ids=lambda c: f"{c[0]}-{c[1]}-d{c[2]}x{c[3]}-T{c[4]}-B{c[5]}H{c[6]}-L+{c[7]}-{c[8]}")
def test_gdn_forward_shape_sweep(case):
    i, dtype, dk, dv, T, B, H, extra, variant = case
    banner(f"sweep gdn {case}")
    L = (T - 1).bit_length() + 1 + extra
    cfg = I.CONFIGS["gdn2k"].scaled(B=B, H=H, T=T, dk=dk, dv=dv, C=64, L=L, dtype=dtype)
    d = I.make_gdn(cfg, variant, seed=900 + i)
    dt = in_dtype(dtype)
    out = LL.loglin_gdn_fwd_chunked(to_dev(d["q"], dt), to_dev(d["k"], dt), to_dev(d["v"], dt),
                                    to_dev(d["a"]), to_dev(d["beta"]), to_dev(d["lam"]), 64)
    torch.cuda.synchronize()
    want = ref.gdn_form_a(d["q"], d["k"], d["v"], d["a"], d["beta"], d["lam"])
    err = slice_rel_err(out.cpu().numpy(), want, 2)
    print(f"  out {err:.2e}", flush=True)
    assert err <= (TOL_BF16 if dtype == "bf16" else TOL_F32), err


# the prefill -> decode hand-over: (dtype, dk, dv) of its other tests
PF_KINDS = [("f32", 16, 16), ("f32", 16, 32), ("f32", 32, 16), ("f32", 64, 64), ("bf16", 64, 64),
            ("bf16", 128, 64), ("f32", 32, 32), ("bf16", 32, 32), ("bf16", 128, 128)]


def _draw_pf(n, tmax, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dtype, dk, dv = PF_KINDS[int(rng.integers(len(PF_KINDS)))]
        out.append((i, dtype, dk, dv, int(rng.integers(1, tmax + 1)), int(rng.integers(1, 3)),
                    int(rng.integers(1, 3)), float(rng.choice([-1.0, -8.0]))))
    return out


PF_CASES = _draw_pf(8, 3000, 20261206)


@pytest.mark.parametrize("case", PF_CASES,
                         ids=lambda c: f"{c[0]}-{c[1]}-d{c[2]}x{c[3]}-T{c[4]}-B{c[5]}H{c[6]}-mu{c[7]:g}")
def test_prefill_shape_sweep(case):
    i, dtype, dk, dv, T, B, H, mu = case
    banner(f"sweep prefill {case}")
    L = (T - 1).bit_length() + 1
    q, k, v, a, lam, _ = _inputs(B, H, T, dk, dv, L, mu, seed=1100 + i)
    dt = in_dtype(dtype)
    got = LL.loglin_prefill_states(to_dev(k, dt), to_dev(v, dt), to_dev(a), L).cpu().numpy()
    _, want = ref.form_b(q, _round(k, dt), _round(v, dt), a, lam, return_states=True)
    err = state_rel_err(got.reshape(B * H, L, dk, dv), want.reshape(B * H, L, dk, dv))
    print(f"  states {err:.2e}", flush=True)
    assert err <= (TOL_BF16 if dtype == "bf16" else TOL_F32), err
    live = set(ref.live_slots(T))
    for lv in range(L):
        if lv not in live:
            assert not np.any(got[:, :, lv]), lv


# decode steps from synthetic pre-filled states: (dk, dv) of its other tests
DEC_KINDS = [(16, 16), (32, 64), (128, 128), (64, 16), (32, 16)]


def _draw_dec(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dk, dv = DEC_KINDS[int(rng.integers(len(DEC_KINDS)))]
        nseq, H, Lmax = int(rng.integers(1, 7)), int(rng.integers(1, 4)), int(rng.integers(10, 17))
        steps, max_prefill = int(rng.integers(20, 131)), int(rng.integers(1, 2000))
        # every position reached must fit the levels (t < 2^(Lmax - 1))
        Lmax = max(Lmax, (max_prefill + steps).bit_length() + 1)
        out.append((i, dk, dv, nseq, H, Lmax, steps, max_prefill, str(rng.choice(["base", "unit"]))))
    return out


DEC_CASES = _draw_dec(6, 20261207)


@pytest.mark.parametrize("case", DEC_CASES,
                         ids=lambda c: f"{c[0]}-d{c[1]}x{c[2]}-n{c[3]}H{c[4]}-L{c[5]}-s{c[6]}-p{c[7]}-{c[8]}")
def test_decode_shape_sweep(case):
    """Steps from pre-filled states (prefill lengths up to the drawn bound,
    steps crossing 64-token window ends): outputs, positions and level
    states against the oracle recurrence, dead slots empty."""
    from tests.test_gpu_decode import _decode_gpu, _live_mask_ok, _oracle
    i, dk, dv, nseq, H, Lmax, steps, max_prefill, variant = case
    banner(f"sweep decode {case}")
    cfg = I.CONFIGS["decode"].scaled(nseq=nseq, H=H, dk=dk, dv=dv, Lmax=Lmax, steps=steps,
                                     max_prefill=max_prefill)
    d = I.make_decode(cfg, variant, seed=1300 + i, live_slots=ref.live_slots)
    out, pos, lv = _decode_gpu(d, d["states"])
    pairs = [(s, h) for s in range(nseq) for h in range(H)]
    o_ref, st_ref, pos_ref = _oracle(d, d["states"], pairs, steps)
    got = out.reshape(steps, -1, dv).transpose(1, 0, 2)
    err = slice_rel_err(got, o_ref.transpose(1, 0, 2), 1)
    serr = state_rel_err(lv.reshape(-1, Lmax, dk, dv), st_ref)
    print(f"  out {err:.2e} states {serr:.2e}", flush=True)
    assert err <= TOL_BF16, err
    assert np.array_equal(pos, pos_ref.reshape(nseq, H)[:, 0])
    assert serr <= TOL_BF16, serr
    ok, where = _live_mask_ok(lv, pos, Lmax)
    assert ok, where
