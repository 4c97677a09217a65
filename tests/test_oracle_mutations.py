"""Planted mistakes in the oracle must be caught by the pins.

Each case swaps one plausible wrong reading into the Python oracle (on the CPU,
through monkeypatch) and checks that the hand-derived fixture or the textbook
special cases no longer match.  This guards the pins themselves.
"""
import json
import os

import numpy as np

from oracle import reference as ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "fenwick_worked_examples.json")


def _fixture_outputs_match():
    with open(GOLDEN) as f:
        g = json.load(f)
    for c in g["outputs"]:
        T = len(c["q"])
        q = np.array(c["q"], float).reshape(T, 1)
        k = np.array(c["k"], float).reshape(T, 1)
        v = np.array(c["v"], float).reshape(T, 1)
        a = np.array(c["a"], float)
        if c["lam_rows"] == "row_scaled":
            lam = np.array([[(t + 1) * 10.0 ** l for l in range(4)] for t in range(T)])
        else:
            lam = np.tile(np.array(c["lam_rows"], float), (T, 1))
        if not np.allclose(ref.form_a(q, k, v, a, lam)[:, 0], c["out"], rtol=1e-12, atol=1e-12):
            return False
    return True


def test_unmutated_oracle_matches():
    assert _fixture_outputs_match()


def test_newest_first_greedy_is_caught(monkeypatch):
    orig = ref.fenwick_buckets

    def newest_first(t):
        bk = orig(t)
        body = [b for b in bk if b[0] > 0]
        sizes = [b[2] - b[1] for b in body][::-1]
        levels = [b[0] for b in body][::-1]
        out, start = [], 0
        for lev, sz in zip(levels, sizes):
            out.append((lev, start, start + sz))
            start += sz
        return out + [bk[-1]]

    monkeypatch.setattr(ref, "fenwick_buckets", newest_first)
    assert not _fixture_outputs_match()


def test_level_off_by_one_is_caught(monkeypatch):
    orig = ref.fenwick_buckets
    monkeypatch.setattr(ref, "fenwick_buckets",
                        lambda t: [(lev + 1 if lev > 0 else 0, a, b) for lev, a, b in orig(t)])
    assert not _fixture_outputs_match()


def test_decay_including_key_gate_is_caught(monkeypatch):
    # wrong convention: M[t,s] = prod_{r=s..t} alpha_r (the key's own gate included)
    real_cumsum = np.cumsum
    monkeypatch.setattr(ref.np, "cumsum", lambda x, *a, **k: real_cumsum(x, *a, **k) - x)
    try:
        assert not _fixture_outputs_match()
    finally:
        monkeypatch.undo()


def test_lambda_by_key_is_caught(monkeypatch):
    orig = ref.form_a

    def by_key(q, k, v, a, lam):
        lam = np.asarray(lam, float)
        T = lam.shape[-2]
        lev = ref.level_map(T).astype(np.int64)
        A = np.cumsum(np.asarray(a, float))
        out = np.zeros((T, np.asarray(v).shape[-1]))
        for t in range(T):
            for s in range(t + 1):
                out[t] += lam[s, lev[t, s]] * np.exp(A[t] - A[s]) * (q[t] @ k[s]) * v[s]
        return out

    monkeypatch.setattr(ref, "form_a", by_key)
    assert not _fixture_outputs_match()
    monkeypatch.setattr(ref, "form_a", orig)
