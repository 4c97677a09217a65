"""GPU parity of the prefill -> decode hand-over against the fp64 oracle.

Page: "Log-linear attention, and what a logarithm buys", section 2 (the
Fenwick states after a prefix and the decode recurrence that continues it).
The states after T tokens are compared with the oracle recurrence's final
states; a decode continued from them is compared with the oracle recurrence
run over the whole sequence.
"""
import numpy as np
import pytest
import torch

from log_linear_token_amd import inputs as I
from log_linear_token_amd import loglin as LL
from oracle import reference as ref
from tests.helpers import TOL_BF16, TOL_F32, banner, slice_rel_err, state_rel_err, to_dev

pytestmark = pytest.mark.gpu


def _inputs(B, H, T, dk, dv, L, seed, weak=False):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, T, dk)) / np.sqrt(dk)
    k = rng.standard_normal((B, H, T, dk)) / np.sqrt(dk)
    v = rng.standard_normal((B, H, T, dv))
    mu = -8.0 if weak else -1.0
    # a and lambda are fp32 on the device: the oracle gets the same values
    a = (-np.logaddexp(0, rng.normal(mu, 0.5, (B, H, T)))).astype(np.float32).astype(np.float64)
    lam = rng.random((B, H, T, L)).astype(np.float32).astype(np.float64)
    return q, k, v, a, lam


def _round(x, dtype):
    """The values the GPU sees: bf16 inputs are rounded once, here."""
    return to_dev(x, dtype).float().cpu().numpy().astype(np.float64)


CASES = [
    # B, H, T, dk, dv, dtype: empty prefix aside, every ragged and power-of-two
    # corner of the bucket decomposition, whole 512-token pieces and the tail
    (1, 2, 1, 16, 16, torch.float32), (1, 2, 2, 16, 32, torch.float32),
    (1, 2, 63, 32, 16, torch.float32), (1, 2, 64, 16, 16, torch.float32),
    (1, 2, 65, 64, 64, torch.float32), (1, 2, 512, 64, 64, torch.bfloat16),
    (1, 2, 513, 128, 64, torch.bfloat16), (1, 2, 514, 32, 32, torch.float32),
    (2, 2, 1000, 64, 64, torch.bfloat16),
    (1, 2, 1024, 32, 32, torch.bfloat16), (1, 2, 1025, 128, 64, torch.bfloat16),
    (1, 1, 3000, 128, 128, torch.bfloat16), (1, 2, 5000, 16, 32, torch.float32),
]


@pytest.mark.parametrize("weak", [False, True])
@pytest.mark.parametrize("B,H,T,dk,dv,dtype", CASES)
def test_prefill_states_vs_recurrence(B, H, T, dk, dv, dtype, weak):
    banner(f"prefill states B={B} H={H} T={T} dk={dk} dv={dv} {dtype} weak={weak}")
    L = max(1, (T - 1).bit_length() + 1)
    q, k, v, a, lam = _inputs(B, H, T, dk, dv, L, seed=T + dk + dv + weak)
    kd, vd = to_dev(k, dtype), to_dev(v, dtype)
    got = LL.loglin_prefill_states(kd, vd, to_dev(a), L).cpu().numpy()
    _, want = ref.form_b(q, _round(k, dtype), _round(v, dtype), a, lam, return_states=True)
    err = state_rel_err(got.reshape(B * H, L, dk, dv), want.reshape(B * H, L, dk, dv))
    tol = TOL_F32 if dtype == torch.float32 else TOL_BF16
    print(f"  max state rel err {err:.2e}", flush=True)
    assert err <= tol, err
    # slots that are not live after T tokens are exactly zero
    live = set(ref.live_slots(T))
    for lv in range(L):
        if lv not in live:
            assert not np.any(got[:, :, lv]), lv


def test_prefill_of_nothing_is_zero():
    banner("prefill T=0")
    k = torch.empty((1, 2, 0, 16), device="cuda")
    st = LL.loglin_prefill_states(k, torch.empty((1, 2, 0, 16), device="cuda"),
                                  torch.empty((1, 2, 0), device="cuda"), 4,
                                  out=torch.full((1, 2, 4, 16, 16), 7.0, device="cuda"))
    assert not torch.any(st).item()


@pytest.mark.parametrize("T,dk,dv,dtype", [(777, 64, 32, torch.bfloat16), (64, 16, 16, torch.float32),
                                           (2048, 128, 128, torch.bfloat16)])
def test_decode_continues_a_prefill(T, dk, dv, dtype):
    """Prefill T tokens on the GPU, load the states, decode 40 more tokens: the
    outputs match the oracle recurrence over all T + 40 tokens."""
    banner(f"prefill then decode T={T} dk={dk} dv={dv} {dtype}")
    B, H, steps = 2, 2, 40
    Lmax = (T + steps - 1).bit_length() + 1
    q, k, v, a, lam = _inputs(B, H, T + steps, dk, dv, Lmax, seed=T * 3 + dk)
    kd, vd = to_dev(k[:, :, :T], dtype), to_dev(v[:, :, :T], dtype)
    states = LL.loglin_prefill_states(kd, vd, to_dev(a[:, :, :T]), Lmax)
    st = LL.loglin_state_init(B, H, dk, dv, Lmax)
    LL.loglin_state_load(st, np.full(B, T, np.int64), states)
    outs = torch.empty((steps, B, H, dv), device="cuda")
    tok = lambda x, s: to_dev(np.ascontiguousarray(x[:, :, T + s]), dtype)  # noqa: E731
    for s in range(steps):
        LL.loglin_decode_step(st, tok(q, s), tok(k, s), tok(v, s),
                              to_dev(np.ascontiguousarray(a[:, :, T + s])),
                              to_dev(np.ascontiguousarray(lam[:, :, T + s])), out=outs[s])
    got = outs.cpu().numpy()
    LL.loglin_state_free(st)
    want = ref.form_b(_round(q, dtype), _round(k, dtype), _round(v, dtype), a, lam)[:, :, T:]
    got = np.transpose(got, (1, 2, 0, 3))  # [B, H, steps, dv]
    err = slice_rel_err(got, want, 2)
    tol = TOL_F32 if dtype == torch.float32 else TOL_BF16
    print(f"  max output rel err {err:.2e}", flush=True)
    assert err <= tol, err


@pytest.mark.parametrize("T,dtype", [(1000, torch.bfloat16), (5000, torch.float32),
                                     (2049, torch.bfloat16)])
def test_prefill_with_many_slots_zeroes_dead_ones(T, dtype):
    """Lmax = 40 (slots far above the levels T uses, where a level index past
    31 must not be taken for a live bucket) with the output buffer filled
    with NaN first: live slots match the recurrence, every other slot is
    exactly zero."""
    banner(f"prefill Lmax=40 T={T} {dtype}")
    B, H, dk, dv, Lmax = 1, 2, 32, 32, 40
    q, k, v, a, lam = _inputs(B, H, T, dk, dv, Lmax, seed=T + 40, weak=True)
    out = torch.full((B, H, Lmax, dk, dv), float("nan"), device="cuda")
    got = LL.loglin_prefill_states(to_dev(k, dtype), to_dev(v, dtype), to_dev(a), Lmax,
                                   out=out).cpu().numpy()
    _, want = ref.form_b(q, _round(k, dtype), _round(v, dtype), a, lam, return_states=True)
    live = set(ref.live_slots(T))
    for lv in range(Lmax):
        if lv not in live:
            assert np.all(got[:, :, lv] == 0), lv
    err = state_rel_err(got.reshape(B * H, Lmax, dk, dv), want.reshape(B * H, Lmax, dk, dv))
    tol = TOL_F32 if dtype == torch.float32 else TOL_BF16
    assert err <= tol, err


def test_prefill_deterministic():
    """Two prefills of the same tokens give bit-identical states."""
    banner("determinism prefill T=3000")
    B, H, T, dk, dv = 1, 2, 3000, 128, 64
    L = (T - 1).bit_length() + 1
    _, k, v, a, _ = _inputs(B, H, T, dk, dv, L, seed=5)
    kd, vd, ad = to_dev(k, torch.bfloat16), to_dev(v, torch.bfloat16), to_dev(a)
    s1 = LL.loglin_prefill_states(kd, vd, ad, L).cpu().numpy()
    s2 = LL.loglin_prefill_states(kd, vd, ad, L).cpu().numpy()
    assert np.array_equal(s1, s2)
