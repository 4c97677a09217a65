"""Pins for the fp64 oracle, against facts the page and plain mathematics fix.

Page: "Log-linear attention, and what a logarithm buys".  Each test names what
it pins.  None of these retypes the oracle's formula: they compare it with
hand-derived values, with textbook recurrences that are special cases of the
mixer, with brute-force properties of the bucket partition, and the two oracle
forms with each other.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import reference as ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "fenwick_worked_examples.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _rand_case(rng, T, dk, dv, L, decay=True, lam_kind="uniform"):
    q = rng.standard_normal((T, dk))
    k = rng.standard_normal((T, dk))
    v = rng.standard_normal((T, dv))
    a = -np.logaddexp(0.0, rng.standard_normal(T)) if decay else np.zeros(T)
    lam = rng.random((T, L)) if lam_kind == "uniform" else np.ones((T, L))
    return q, k, v, a, lam


def _levels_needed(T):
    return 1 if T <= 1 else (T - 1).bit_length() + 1


# ---------------------------------------------------------------- buckets

def test_buckets_match_hand_derived_table():
    """Section 2 rule (greedy largest power of two, oldest first), by hand for small t."""
    g = _golden()["buckets"]
    for t, expect in g.items():
        if t == "comment":
            continue
        got = [list(b) for b in ref.fenwick_buckets(int(t))]
        assert got == expect, (t, got, expect)


def test_bucket_partition_properties_bruteforce():
    """Disjoint, covering [0, t], bucket l >= 1 of size 2^(l-1), sentinel of size one,
    at most ceil(log2 t + 1) + 1 buckets (section 2), sizes decreasing with recency."""
    for t in range(0, 4097):
        bk = ref.fenwick_buckets(t)
        cover = np.zeros(t + 1, dtype=np.int64)
        for lev, a, b in bk:
            cover[a:b] += 1
            if lev == 0:
                assert (a, b) == (t, t + 1)
            else:
                assert b - a == 2 ** (lev - 1)
        assert np.all(cover == 1), t
        sizes = [b - a for lev, a, b in bk if lev > 0]
        assert sizes == sorted(sizes, reverse=True)
        assert len(set(lev for lev, _, _ in bk)) == len(bk)
        if t >= 1:
            assert len(bk) <= ref.bucket_bound(t)


def test_bucket_bound_at_128k_is_19():
    """Section 5: at 128K context the page's bucket formula gives 19."""
    assert ref.bucket_bound(128 * 1024) == 19
    worst = max(len(ref.fenwick_buckets(t)) for t in range(1, 128 * 1024 + 1, 7))
    worst = max(worst, len(ref.fenwick_buckets(128 * 1024 - 1)))
    assert worst <= 19


def test_level_map_rows():
    m = ref.level_map(12)
    assert list(m[7, :8]) == [3, 3, 3, 3, 2, 2, 1, 0]
    assert list(m[11, :12]) == [4] * 8 + [2, 2, 1, 0]
    assert np.all(m[np.triu_indices(12, 1)] == -1)


# ---------------------------------------------------------------- worked outputs

@pytest.mark.parametrize("case", range(4))
def test_worked_examples_both_forms(case):
    """Hand-computed outputs (golden fixture) reproduced by Form A and Form B."""
    c = _golden()["outputs"][case]
    T = len(c["q"])
    q = np.array(c["q"], float).reshape(T, 1)
    k = np.array(c["k"], float).reshape(T, 1)
    v = np.array(c["v"], float).reshape(T, 1)
    a = np.array(c["a"], float)
    L = 4
    if c["lam_rows"] == "row_scaled":
        lam = np.array([[(t + 1) * 10.0 ** l for l in range(L)] for t in range(T)])
    else:
        lam = np.tile(np.array(c["lam_rows"], float), (T, 1))
    want = np.array(c["out"], float)
    oa = ref.form_a(q, k, v, a, lam)[:, 0]
    ob = ref.form_b(q, k, v, a, lam)[:, 0]
    np.testing.assert_allclose(oa, want, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(ob, want, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------- the two forms agree

@pytest.mark.parametrize("T,dk,dv,extraL", [(1, 3, 2, 0), (2, 4, 4, 1), (5, 3, 7, 0), (16, 8, 8, 2),
                                            (37, 5, 3, 0), (64, 16, 16, 1), (100, 6, 9, 0),
                                            (257, 4, 4, 0)])
def test_form_a_equals_form_b(T, dk, dv, extraL):
    rng = np.random.default_rng(T * 1000 + dk)
    L = _levels_needed(T) + extraL
    q, k, v, a, lam = _rand_case(rng, T, dk, dv, L)
    oa = ref.form_a(q, k, v, a, lam)
    ob = ref.form_b(q, k, v, a, lam)
    err = np.max(np.abs(oa - ob)) / max(np.max(np.abs(oa)), 1e-300)
    assert err < 1e-12, err


def test_form_a_rows_equals_form_a():
    rng = np.random.default_rng(7)
    T, L = 300, 11
    q, k, v, a, lam = _rand_case(rng, T, 8, 5, L)
    full = ref.form_a(q, k, v, a, lam)
    rows = [0, 1, 63, 64, 127, 128, 255, 256, 299]
    np.testing.assert_allclose(ref.form_a_rows(q, k, v, a, lam, rows), full[rows], rtol=1e-12,
                               atol=1e-12)


def test_batched_slices_are_independent():
    rng = np.random.default_rng(3)
    B, H, T, dk, dv, L = 2, 3, 40, 4, 6, 8
    q = rng.standard_normal((B, H, T, dk))
    k = rng.standard_normal((B, H, T, dk))
    v = rng.standard_normal((B, H, T, dv))
    a = -np.abs(rng.standard_normal((B, H, T)))
    lam = rng.random((B, H, T, L))
    ob = ref.form_b(q, k, v, a, lam, nthreads=3)
    for b in range(B):
        for h in range(H):
            one = ref.form_a(q[b, h], k[b, h], v[b, h], a[b, h], lam[b, h])
            np.testing.assert_allclose(ob[b, h], one, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- special cases

def _gated_linear_attention(q, k, v, a):
    """Textbook Mamba-2 / gated linear attention: S_t = alpha_t S_{t-1} + k_t v_t^T."""
    S = np.zeros((q.shape[1], v.shape[1]))
    out = np.zeros((q.shape[0], v.shape[1]))
    for t in range(q.shape[0]):
        S = math.exp(a[t]) * S + np.outer(k[t], v[t])
        out[t] = q[t] @ S
    return out


@pytest.mark.parametrize("T", [1, 9, 64, 130])
def test_equal_lambda_collapses_to_gated_linear_attention(T):
    """Section 5: with all lambda_t^(l) equal across levels the mixer is linear
    attention with the base model's gate (here a per-row factor c_t)."""
    rng = np.random.default_rng(11 + T)
    L = _levels_needed(T) + 1
    q, k, v, a, _ = _rand_case(rng, T, 6, 4, L)
    c = rng.random(T) + 0.5
    lam = np.repeat(c[:, None], L, axis=1)
    want = c[:, None] * _gated_linear_attention(q, k, v, a)
    for got in (ref.form_a(q, k, v, a, lam), ref.form_b(q, k, v, a, lam)):
        np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-11)


def test_unit_decay_single_bucket_is_linear_attention():
    """Section 1: linear attention is the all-ones lower-triangular mask."""
    rng = np.random.default_rng(5)
    T, L = 90, 9
    q, k, v, _, _ = _rand_case(rng, T, 5, 7, L)
    a = np.zeros(T)
    lam = np.ones((T, L))
    kv = np.cumsum(k[:, :, None] * v[:, None, :], axis=0)
    want = np.einsum("td,tde->te", q, kv)
    for got in (ref.form_a(q, k, v, a, lam), ref.form_b(q, k, v, a, lam)):
        np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-11)


def test_level_zero_only_is_diagonal():
    """Only the sentinel bucket weighted: o_t = lambda_t^(0) (q_t . k_t) v_t."""
    rng = np.random.default_rng(8)
    T, L = 50, 8
    q, k, v, a, lam = _rand_case(rng, T, 4, 3, L)
    lam[:, 1:] = 0.0
    want = (lam[:, 0] * np.sum(q * k, axis=1))[:, None] * v
    np.testing.assert_allclose(ref.form_b(q, k, v, a, lam), want, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ref.form_a(q, k, v, a, lam), want, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("level", range(1, 5))
def test_one_hot_level_is_that_bucket_sum(level):
    """lambda one-hot at one level: o_t sums exactly the tokens of that bucket
    (bucket found by brute force over aligned power-of-two blocks, T <= 16)."""
    rng = np.random.default_rng(20 + level)
    T, L = 16, 6
    q, k, v, a, lam = _rand_case(rng, T, 3, 2, L)
    lam[:] = 0.0
    lam[:, level] = 1.0
    A = np.cumsum(a)
    want = np.zeros((T, 2))
    size = 2 ** (level - 1)
    for t in range(T):
        # brute force: among all aligned blocks of this size inside [0, t), the
        # one the greedy cut produces is the block that, together with the
        # larger buckets before it, starts right where the larger ones end.
        larger = sum(2 ** p for p in range(level, 8) if (t >> p) & 1)
        if (t >> (level - 1)) & 1:
            members = range(larger, larger + size)
            for s in members:
                want[t] += math.exp(A[t] - A[s]) * (q[t] @ k[s]) * v[s]
    np.testing.assert_allclose(ref.form_b(q, k, v, a, lam), want, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ref.form_a(q, k, v, a, lam), want, rtol=1e-12, atol=1e-12)


def test_exact_arithmetic_case_is_exact():
    """No decay, entries in {-1, 0, 1}, lambda in {0, 1/2, 1}: every product and
    sum is an exact binary fraction, so both forms agree to the last bit."""
    rng = np.random.default_rng(9)
    T, dk, dv, L = 64, 16, 16, 8
    q = rng.integers(-1, 2, (T, dk)).astype(float)
    k = rng.integers(-1, 2, (T, dk)).astype(float)
    v = rng.integers(-1, 2, (T, dv)).astype(float)
    lam = rng.integers(0, 3, (T, L)).astype(float) / 2.0
    a = np.zeros(T)
    oa = ref.form_a(q, k, v, a, lam)
    ob = ref.form_b(q, k, v, a, lam)
    assert np.array_equal(oa, ob)
    assert np.array_equal(oa * 2, np.round(oa * 2))


# ---------------------------------------------------------------- decode

def test_decode_continues_forward():
    """Section 2 decode: nothing is recomputed -- the state after T0 tokens,
    continued by decode, gives the same outputs and states as one pass."""
    rng = np.random.default_rng(12)
    T, T0, dk, dv = 77, 30, 5, 4
    L = _levels_needed(T) + 1
    q, k, v, a, lam = _rand_case(rng, T, dk, dv, L)
    full, st_full = ref.form_b(q, k, v, a, lam, return_states=True)
    _, st0 = ref.form_b(q[:T0], k[:T0], v[:T0], a[:T0], lam[:T0], return_states=True)
    steps = T - T0
    out, st, pos = ref.decode(st0[None], [T0], q[T0:, None], k[T0:, None], v[T0:, None],
                              a[T0:, None], lam[T0:, None])
    np.testing.assert_allclose(out[:, 0], full[T0:], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(st[0], st_full, rtol=1e-12, atol=1e-12)
    assert pos[0] == T
    fa = ref.form_a(q, k, v, a, lam)
    np.testing.assert_allclose(out[:, 0], fa[T0:], rtol=1e-11, atol=1e-11)


def test_decode_from_empty_state():
    rng = np.random.default_rng(13)
    T, dk, dv, L = 20, 3, 3, 6
    q, k, v, a, lam = _rand_case(rng, T, dk, dv, L)
    out, st, pos = ref.decode(np.zeros((1, L, dk, dv)), [0], q[:, None], k[:, None], v[:, None],
                              a[:, None], lam[:, None])
    np.testing.assert_allclose(out[:, 0], ref.form_a(q, k, v, a, lam), rtol=1e-12, atol=1e-12)


def test_live_levels_of_states():
    """After t tokens only slot 0 and slots p+1 for the set bits p of t-1 hold
    a bucket; the others are zero (the recurrence zeroes merged levels)."""
    rng = np.random.default_rng(14)
    for T in (1, 2, 3, 8, 13, 64, 100):
        L = _levels_needed(T) + 2
        q, k, v, a, lam = _rand_case(rng, T, 2, 2, L)
        _, st = ref.form_b(q, k, v, a, lam, return_states=True)
        nz = [lv for lv in range(L) if np.any(st[lv] != 0)]
        want = [0] + [p + 1 for p in range((T - 1).bit_length()) if ((T - 1) >> p) & 1]
        assert nz == want, (T, nz, want)
        # the live-slot list the parity tests use, read off the greedy buckets
        assert ref.live_slots(T) == nz, (T, ref.live_slots(T), nz)
    assert ref.live_slots(0) == []


def test_capacity_error():
    rng = np.random.default_rng(15)
    T = 9
    q, k, v, a, lam = _rand_case(rng, T, 2, 2, 4)  # position 8 needs level 4 -> L >= 5
    with pytest.raises(RuntimeError):
        ref.form_b(q, k, v, a, lam)
    lam5 = np.concatenate([lam, lam[:, :1]], axis=1)
    ref.form_b(q, k, v, a, lam5)


def test_long_sequence_invariants_hold():
    """The recurrence checks its live set and the bucket bound at every step."""
    rng = np.random.default_rng(16)
    T = 5000
    q, k, v, a, lam = _rand_case(rng, T, 1, 1, _levels_needed(T))
    out = ref.form_b(q, k, v, a, lam)
    rows = [0, 1, 1023, 1024, 4095, 4096, 4999]
    np.testing.assert_allclose(out[rows], ref.form_a_rows(q, k, v, a, lam, rows), rtol=1e-11,
                               atol=1e-11)
