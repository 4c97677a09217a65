"""Pins of the oracle's gradients (the backward pass) on the CPU.

The gradients of sum(O * dO) that oracle.reference.form_a_grads writes out by
the chain rule are checked against central finite differences of Form A
itself (whose values are pinned elsewhere by the worked examples, brute force
and the textbook special cases), element by element, on tiny inputs that
cover an empty-ish sequence, ragged lengths, several Fenwick levels and a
level of lambda that the sequence never uses.  Planted mistakes in the
gradient formulas must fail the same check.
"""
import numpy as np
import pytest

from oracle import reference as ref


def _case(T, dk, dv, L, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, dk))
    k = rng.standard_normal((T, dk))
    v = rng.standard_normal((T, dv))
    a = -np.logaddexp(0, rng.standard_normal(T))
    lam = rng.random((T, L))
    g = rng.standard_normal((T, dv))
    return q, k, v, a, lam, g


def _numeric(args, g, h=1e-6):
    """Central differences of sum(form_a(...) * g) in every input element."""
    def f(xs):
        return float(np.sum(ref.form_a(*xs) * g))
    out = []
    for ai, x in enumerate(args):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xs = list(args)
            xp = x.copy(); xp[idx] += h
            xm = x.copy(); xm[idx] -= h
            xs[ai] = xp
            fp = f(xs)
            xs[ai] = xm
            num[idx] = (fp - f(xs)) / (2 * h)
        out.append(num)
    return out


def _max_err(grads, nums):
    return max(float(np.max(np.abs(d - n), initial=0.0)) / max(1.0, float(np.max(np.abs(n), initial=0.0)))
               for d, n in zip(grads, nums))


@pytest.mark.parametrize("T,dk,dv,extra", [(1, 2, 3, 0), (2, 1, 1, 1), (5, 3, 2, 0), (16, 2, 2, 1),
                                           (19, 3, 2, 2)])
def test_grads_match_finite_differences(T, dk, dv, extra):
    L = (T - 1).bit_length() + 1 + extra if T > 1 else 1 + extra
    q, k, v, a, lam, g = _case(T, dk, dv, L, seed=T * 7 + dk)
    grads = ref.form_a_grads(q, k, v, a, lam, g)
    nums = _numeric([q, k, v, a, lam], g)
    assert _max_err(grads, nums) < 1e-7
    # levels the sequence never reaches get no gradient at all
    used = (T - 1).bit_length() + 1 if T > 1 else 1
    assert not np.any(grads[4][:, used:])


def test_grads_batched_shapes():
    """Leading (batch, head) dimensions are independent slices."""
    rng = np.random.default_rng(3)
    B, H, T, dk, dv, L = 2, 3, 9, 2, 3, 5
    q, k = rng.standard_normal((2, B, H, T, dk))
    v, g = rng.standard_normal((2, B, H, T, dv))
    a = -np.logaddexp(0, rng.standard_normal((B, H, T)))
    lam = rng.random((B, H, T, L))
    full = ref.form_a_grads(q, k, v, a, lam, g)
    for b in range(B):
        for h in range(H):
            one = ref.form_a_grads(q[b, h], k[b, h], v[b, h], a[b, h], lam[b, h], g[b, h])
            for x, y in zip(full, one):
                np.testing.assert_array_equal(x[b, h], y)


# ---- planted mistakes: each must be caught by the finite-difference pin

def _planted(monkeypatch, name, wrong):
    T, dk, dv = 9, 2, 2
    L = (T - 1).bit_length() + 1
    q, k, v, a, lam, g = _case(T, dk, dv, L, seed=11)
    nums = _numeric([q, k, v, a, lam], g)
    monkeypatch.setattr(ref, name, wrong)
    return _max_err(ref.form_a_grads(q, k, v, a, lam, g), nums)


def test_prefix_instead_of_suffix_sum_for_da_is_caught(monkeypatch):
    assert _planted(monkeypatch, "_suffix_sum", np.cumsum) > 1e-3


def test_dropped_column_term_of_da_is_caught(monkeypatch):
    assert _planted(monkeypatch, "_running_sum_grad", lambda W: W.sum(axis=1)) > 1e-3


def test_wrong_level_assignment_is_caught(monkeypatch):
    orig = ref.level_map
    assert _planted(monkeypatch, "level_map",
                    lambda T: np.where(orig(T) > 1, orig(T) - 1, orig(T)).astype(np.int8)) > 1e-3
