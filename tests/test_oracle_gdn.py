"""Pins of the log-linear Gated DeltaNet oracle (CPU only).

Page: "Log-linear attention, and what a logarithm buys" -- section 1 (Gated
DeltaNet changes the query-key interaction, not the mask), section 2 (Fenwick
buckets and the level-weighted read-out), section 3 (the lift composes the
temporal mask with the level mask); the gated delta rule is that of the Gated
DeltaNet paper, the page's source 3.

What pins the two oracle forms to something other than themselves:
  * the hand-derived outputs of tests/golden/gdn_worked_examples.json;
  * lambda equal over the levels -> that constant times the textbook gated
    delta-rule recurrence, written out here token by token;
  * mutually orthogonal keys (no key is changed by another's transition) ->
    the log-linear Mamba-2 mixer (pinned in test_oracle_pins.py) with each
    value scaled by its writing strength;
  * beta = 0 -> zero output;
  * lambda one-hot on a level -> the sum over that bucket with the transition
    products formed as explicit d_k x d_k matrices (brute force, tiny T);
  * the two forms agree with each other, and decode continues a forward;
  * planted mistakes in a copy of the masked form are caught by the fixture.
"""
import json
import os

import numpy as np
import pytest
from scipy.linalg import solve_triangular

from oracle import reference as ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "gdn_worked_examples.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


def _case_arrays(c):
    return (np.array(c["q"], float), np.array(c["k"], float), np.array(c["v"], float),
            np.array(c["a"], float), np.array(c["beta"], float), np.array(c["lam"], float))


def _rand(rng, T, dk, dv, L, normalise=True, lead=()):
    q = rng.standard_normal(lead + (T, dk)) / np.sqrt(dk)
    k = rng.standard_normal(lead + (T, dk))
    if normalise:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    else:
        k /= np.sqrt(dk)
    v = rng.standard_normal(lead + (T, dv))
    a = -np.logaddexp(0.0, rng.standard_normal(lead + (T,)) - 1.0)
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal(lead + (T,))))
    lam = rng.random(lead + (T, L))
    return q, k, v, a, beta, lam


def _levels_needed(T):
    return 1 if T <= 1 else (T - 1).bit_length() + 1


# ------------------------------------------------------------------ fixture

@pytest.mark.parametrize("form", ["a", "b"])
def test_hand_derived_outputs(form):
    for c in _golden():
        q, k, v, a, beta, lam = _case_arrays(c)
        f = ref.gdn_form_a if form == "a" else ref.gdn_form_b
        got = f(q, k, v, a, beta, lam)
        np.testing.assert_allclose(got, np.array(c["out"], float), rtol=1e-13, atol=1e-13,
                                   err_msg=c["name"])


# ------------------------------------------------------------------ special cases

def _textbook_gated_delta_rule(q, k, v, a, beta):
    """S_t = exp(a_t) (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T, o_t = S_t^T q_t."""
    T, dk = q.shape
    S = np.zeros((dk, v.shape[1]))
    out = np.zeros((T, v.shape[1]))
    for t in range(T):
        G = np.exp(a[t]) * (np.eye(dk) - beta[t] * np.outer(k[t], k[t]))
        S = G @ S + beta[t] * np.outer(k[t], v[t])
        out[t] = S.T @ q[t]
    return out


@pytest.mark.parametrize("T", [1, 5, 16, 33, 100])
def test_equal_lambda_is_the_gated_delta_rule(T):
    rng = np.random.default_rng(T)
    dk, dv = 6, 4
    L = _levels_needed(T) + 1
    q, k, v, a, beta, _ = _rand(rng, T, dk, dv, L)
    c = rng.random(T) + 0.5
    lam = np.repeat(c[:, None], L, axis=1)
    want = c[:, None] * _textbook_gated_delta_rule(q, k, v, a, beta)
    np.testing.assert_allclose(ref.gdn_form_a(q, k, v, a, beta, lam), want, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(ref.gdn_form_b(q, k, v, a, beta, lam), want, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("T", [3, 8, 13])
def test_orthogonal_keys_reduce_to_the_scalar_gated_mixer(T):
    """With k_r . k_s = 0 for r != s no transition changes an earlier key,
    so Phi(t, s) k_s = exp(A_t - A_s) k_s and the lift is the log-linear
    Mamba-2 mixer with v_s scaled by beta_s."""
    rng = np.random.default_rng(100 + T)
    dk, dv = 16, 3
    L = _levels_needed(T)
    q, _, v, a, beta, lam = _rand(rng, T, dk, dv, L)
    basis, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = basis[:T] * rng.uniform(0.5, 1.5, (T, 1))  # orthogonal rows, various norms
    want = ref.form_a(q, k, beta[:, None] * v, a, lam)
    np.testing.assert_allclose(ref.gdn_form_a(q, k, v, a, beta, lam), want, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(ref.gdn_form_b(q, k, v, a, beta, lam), want, rtol=1e-11, atol=1e-12)


def test_zero_writing_strength_gives_zero():
    rng = np.random.default_rng(7)
    q, k, v, a, beta, lam = _rand(rng, 20, 4, 4, 6)
    beta[:] = 0.0
    assert np.all(ref.gdn_form_a(q, k, v, a, beta, lam) == 0.0)
    assert np.all(ref.gdn_form_b(q, k, v, a, beta, lam) == 0.0)


@pytest.mark.parametrize("level", [0, 1, 2, 3])
def test_one_hot_level_is_the_bucket_sum(level):
    """lambda one-hot at `level`: o_t sums the keys of that bucket only, each
    through the explicit product of the transition matrices after it."""
    rng = np.random.default_rng(200 + level)
    T, dk, dv = 12, 3, 2
    L = _levels_needed(T)
    q, k, v, a, beta, _ = _rand(rng, T, dk, dv, L)
    lam = np.zeros((T, L))
    lam[:, level] = 1.0
    G = [np.exp(a[r]) * (np.eye(dk) - beta[r] * np.outer(k[r], k[r])) for r in range(T)]
    want = np.zeros((T, dv))
    for t in range(T):
        for lev, s0, s1 in ref.fenwick_buckets(t):
            if lev != level:
                continue
            for s in range(s0, s1):
                phi = np.eye(dk)
                for r in range(s + 1, t + 1):
                    phi = G[r] @ phi
                want[t] += beta[s] * (q[t] @ phi @ k[s]) * v[s]
    np.testing.assert_allclose(ref.gdn_form_a(q, k, v, a, beta, lam), want, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(ref.gdn_form_b(q, k, v, a, beta, lam), want, rtol=1e-11, atol=1e-13)


# ------------------------------------------------------------------ the two forms

@pytest.mark.parametrize("T,dk,dv,extra,normalise", [(1, 2, 2, 0, True), (7, 3, 5, 1, True),
                                                    (64, 8, 4, 0, True), (129, 5, 7, 2, False),
                                                    (300, 16, 16, 0, True)])
def test_forms_agree(T, dk, dv, extra, normalise):
    rng = np.random.default_rng(T * 31 + dk)
    L = _levels_needed(T) + extra
    q, k, v, a, beta, lam = _rand(rng, T, dk, dv, L, normalise=normalise, lead=(2,))
    fa = ref.gdn_form_a(q, k, v, a, beta, lam)
    fb = ref.gdn_form_b(q, k, v, a, beta, lam)
    np.testing.assert_allclose(fb, fa, rtol=1e-10, atol=1e-11 * np.max(np.abs(fa)))


def test_recurrence_live_slots_and_states():
    """After n tokens the recurrence holds exactly the slots of the buckets
    query n-1 sees, and the level states sum to the textbook state."""
    rng = np.random.default_rng(9)
    for T in (1, 2, 3, 8, 13, 64, 100):
        L = _levels_needed(T) + 2
        q, k, v, a, beta, lam = _rand(rng, T, 3, 2, L)
        _, st = ref.gdn_form_b(q, k, v, a, beta, lam, return_states=True)
        nz = [lv for lv in range(L) if np.any(st[lv] != 0)]
        assert nz == ref.live_slots(T), (T, nz)
        S = np.zeros((3, 2))
        for t in range(T):
            S = np.exp(a[t]) * (np.eye(3) - beta[t] * np.outer(k[t], k[t])) @ S \
                + beta[t] * np.outer(k[t], v[t])
        np.testing.assert_allclose(st.sum(axis=0), S, rtol=1e-11, atol=1e-13)


def test_decode_continues_the_forward():
    rng = np.random.default_rng(10)
    T0, T, dk, dv = 37, 70, 4, 3
    L = _levels_needed(T)
    q, k, v, a, beta, lam = _rand(rng, T, dk, dv, L)
    _, st0 = ref.gdn_form_b(q[:T0], k[:T0], v[:T0], a[:T0], beta[:T0], lam[:T0],
                            return_states=True)
    _, st_full = ref.gdn_form_b(q, k, v, a, beta, lam, return_states=True)
    sl = slice(T0, T)
    out, st, pos = ref.gdn_decode(st0[None], [T0], q[sl, None], k[sl, None], v[sl, None],
                                  a[sl, None], beta[sl, None], lam[sl, None])
    np.testing.assert_allclose(st[0], st_full, rtol=1e-12, atol=1e-12)
    assert pos[0] == T
    np.testing.assert_allclose(out[:, 0], ref.gdn_form_a(q, k, v, a, beta, lam)[T0:], rtol=1e-10,
                               atol=1e-11)


def test_decode_from_empty_state():
    rng = np.random.default_rng(11)
    T, dk, dv = 20, 3, 3
    L = _levels_needed(T)
    q, k, v, a, beta, lam = _rand(rng, T, dk, dv, L)
    out, _, _ = ref.gdn_decode(np.zeros((1, L, dk, dv)), [0], q[:, None], k[:, None],
                               v[:, None], a[:, None], beta[:, None], lam[:, None])
    np.testing.assert_allclose(out[:, 0], ref.gdn_form_a(q, k, v, a, beta, lam), rtol=1e-11,
                               atol=1e-12)


def test_capacity_error():
    rng = np.random.default_rng(12)
    q, k, v, a, beta, lam = _rand(rng, 9, 2, 2, 4)  # position 8 needs level 4
    with pytest.raises(RuntimeError):
        ref.gdn_form_b(q, k, v, a, beta, lam)


# ------------------------------------------------------------------ planted mistakes

def _masked_form(q, k, v, a, beta, lam, mistake):
    """A copy of the masked form with one planted mistake."""
    T = q.shape[0]
    lev = ref.level_map(T).astype(np.int64)
    tri = lev >= 0
    strict = np.tril(np.ones((T, T), bool), -1)
    A = np.cumsum(a)
    KK = k @ k.T
    sign = -1.0 if mistake == "plus_sign" else 1.0
    system = np.eye(T) + sign * beta[:, None] * np.where(strict, KK, 0.0)
    rhs = np.eye(T) if mistake == "no_write_strength" else np.diag(beta)
    inv_beta = solve_triangular(system, rhs, lower=True, unit_diagonal=True)
    if mistake == "no_delta":
        inv_beta = np.diag(beta)
    inter = np.where(tri, q @ k.T, 0.0) @ inv_beta
    decay = np.where(tri, np.exp(np.where(tri, A[:, None] - A[None, :], 0.0)), 0.0)
    if mistake == "key_gate_included":
        decay = np.where(tri, np.exp(np.where(tri, A[:, None] - A[None, :] + a[None, :], 0.0)), 0.0)
    rows = np.arange(T)[:, None]
    lvl_idx = np.maximum(lev, 0)
    lvl = lam[rows, lvl_idx] if mistake != "lambda_by_key" else lam.T[lvl_idx, np.arange(T)[None, :]]
    return (inter * decay * np.where(tri, lvl, 0.0)) @ v


def _fixture_matches(mistake):
    for c in _golden():
        q, k, v, a, beta, lam = _case_arrays(c)
        if not np.allclose(_masked_form(q, k, v, a, beta, lam, mistake), c["out"], rtol=1e-12,
                           atol=1e-12):
            return False
    return True


def test_unmutated_copy_matches_the_fixture():
    assert _fixture_matches(None)


@pytest.mark.parametrize("mistake", ["plus_sign", "no_write_strength", "no_delta",
                                     "key_gate_included", "lambda_by_key"])
def test_planted_mistake_is_caught(mistake):
    assert not _fixture_matches(mistake)
