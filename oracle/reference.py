"""CPU oracle for the log-linear (Fenwick-tree) token mixer, in fp64.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
CPU-baseline leg of the benchmark may import this module; the product path
never does, and this module imports nothing from the product package.

Two independent forms of the same output are provided:

* Form A -- the materialised mask.  "Log-linear attention, and what a logarithm
  buys", section 1 writes every variant as P = A (.) M, O = P V with A = Q K^T;
  section 2 gives the Fenwick buckets (greedily take the largest power of two
  that fits in what remains; bucket l >= 1 holds 2^(l-1) tokens, plus a
  size-one sentinel) and the per-level weights lambda_t^(l); section 3 composes
  the Mamba-2 scalar-decay mask with the level mask by an elementwise product.
  So M[t, s] = lambda_t^(level(t, s)) * exp(A_t - A_s) for s <= t, where
  A_t = a_0 + ... + a_t, and the level of s comes from enumerating the buckets
  greedily (not from a closed-form bit formula).
* Form B -- the token-by-token Fenwick recurrence of section 2, in C
  (loglin_oracle.c), which also serves decode.
* The backward pass -- the gradients of Form A by the chain rule
  (form_a_grads), pinned by finite differences of Form A.
* The log-linear Gated DeltaNet -- section 1 says Gated DeltaNet differs from
  Mamba-2 in how it structures A (the query-key interaction), not the mask M,
  and section 3 lifts such a layer by composing its temporal mask with the
  level mask.  gdn_form_a writes that out with the masked (parallel) form of
  the gated delta rule of the Gated DeltaNet paper (the page's source 3);
  gdn_form_b (C) runs the Fenwick recurrence with the gated delta-rule
  transition on every bucket state.

Readings of points the page leaves open (positions 0-indexed, oldest tokens in
the largest bucket, lambda indexed by the query, the decay convention) are
listed with the reasons in the design notes at the repository root.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "loglin_oracle.c")
# LLO_SANITIZE=1 selects a build with AddressSanitizer and UndefinedBehaviorSanitizer
# (the process must preload gcc's libasan; see tests/test_host_sanitizers.py)
_SANITIZE = os.environ.get("LLO_SANITIZE") == "1"
_LIB = os.path.join(_HERE, "liblloracle_san.so" if _SANITIZE else "liblloracle.so")

LLO_OK, LLO_EARG, LLO_ECAP, LLO_ELIVE, LLO_ENOMEM = 0, 1, 2, 3, 4


def build(force: bool = False) -> str:
    """Compile the C part of the oracle with gcc (plain -O2, no tuning)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
               "-g"] if _SANITIZE else []
        subprocess.check_call(
            ["gcc", "-O2", "-std=c99", *san, "-shared", "-fPIC", _SRC, "-o", tmp, "-lm", "-lpthread"]
        )
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        _lib = ctypes.CDLL(build())
        dp = ctypes.POINTER(ctypes.c_double)
        ip = ctypes.POINTER(ctypes.c_int64)
        _lib.llo_fwd_recurrent.argtypes = [dp, dp, dp, dp, dp, dp, dp, ctypes.c_long, ctypes.c_long,
                                           ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int]
        _lib.llo_fwd_recurrent.restype = ctypes.c_int
        _lib.llo_decode.argtypes = [dp, ip, dp, dp, dp, dp, dp, dp, ctypes.c_long, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int]
        _lib.llo_decode.restype = ctypes.c_int
        _lib.llo_gdn_fwd_recurrent.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp, ctypes.c_long,
                                               ctypes.c_long, ctypes.c_int, ctypes.c_int,
                                               ctypes.c_int, ctypes.c_int]
        _lib.llo_gdn_fwd_recurrent.restype = ctypes.c_int
        _lib.llo_gdn_decode.argtypes = [dp, ip, dp, dp, dp, dp, dp, dp, dp, ctypes.c_long,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int]
        _lib.llo_gdn_decode.restype = ctypes.c_int
    return _lib


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(x: np.ndarray, ctype=ctypes.c_double):
    return x.ctypes.data_as(ctypes.POINTER(ctype))


def default_threads() -> int:
    return max(1, len(os.sched_getaffinity(0)))


# --------------------------------------------------------------------------
# Fenwick buckets by greedy enumeration (section 2)

def fenwick_buckets(t: int):
    """Buckets of the prefix seen by the query at 0-indexed position t.

    Returns a list of (level, start, stop) half-open token ranges.  The t
    earlier tokens 0..t-1 are cut greedily: take the largest power of two 2^p
    that fits in what remains, oldest tokens first; that bucket gets level
    p + 1 and holds 2^p tokens.  Token t itself is the size-one sentinel at
    level 0.
    """
    if t < 0:
        raise ValueError("t must be >= 0")
    out = []
    rem, start = t, 0
    while rem > 0:
        p = 0
        while (1 << (p + 1)) <= rem:
            p += 1
        out.append((p + 1, start, start + (1 << p)))
        start += 1 << p
        rem -= 1 << p
    out.append((0, t, t + 1))
    return out


def live_slots(n: int) -> list[int]:
    """Level slots that hold a bucket once tokens 0..n-1 have been absorbed.

    They are the levels of the buckets that query n-1 sees (section 2: the
    newest token at level 0 and the greedy buckets of the older ones), read
    off the greedy enumeration above.  Empty for n = 0.
    """
    if n <= 0:
        return []
    return sorted(lev for lev, _, _ in fenwick_buckets(n - 1))


def level_row(t: int, length: int | None = None) -> np.ndarray:
    """int8 row: level of key s for query t (s <= t), -1 for s > t."""
    n = t + 1 if length is None else length
    row = np.full(n, -1, dtype=np.int8)
    for lev, a, b in fenwick_buckets(t):
        row[a:min(b, n)] = lev
    return row


def level_map(T: int) -> np.ndarray:
    """int8 [T, T] level map, -1 above the diagonal."""
    m = np.full((T, T), -1, dtype=np.int8)
    for t in range(T):
        m[t, : t + 1] = level_row(t)
    return m


def bucket_bound(t: int) -> int:
    """The page's bound on the number of buckets: ceil(log2 t + 1) + 1."""
    return int(np.ceil(np.log2(float(t)) + 1.0)) + 1


# --------------------------------------------------------------------------
# Form A: materialised mask

def form_a(q, k, v, a, lam) -> np.ndarray:
    """O = ((Q K^T) (.) M) V with the mask written out, per (batch, head) slice.

    q, k [..., T, dk]; v [..., T, dv]; a [..., T]; lam [..., T, L].
    Leading dimensions are flattened into slices.  Meant for T up to a few
    thousand (it allocates T x T per slice).
    """
    q, k, v, a, lam = map(_f64, (q, k, v, a, lam))
    lead = q.shape[:-2]
    T, dk = q.shape[-2:]
    dv = v.shape[-1]
    L = lam.shape[-1]
    lev = level_map(T).astype(np.int64)
    tri = lev >= 0
    if T > 0 and lev.max() >= L:
        raise ValueError(f"lambda has {L} levels; T={T} needs {lev.max() + 1}")
    qf, kf, vf = q.reshape(-1, T, dk), k.reshape(-1, T, dk), v.reshape(-1, T, dv)
    af, lf = a.reshape(-1, T), lam.reshape(-1, T, L)
    out = np.zeros((qf.shape[0], T, dv))
    rows = np.arange(T)[:, None]
    for i in range(qf.shape[0]):
        A = np.cumsum(af[i])
        decay = np.where(tri, np.exp(np.where(tri, A[:, None] - A[None, :], 0.0)), 0.0)
        lvl = np.where(tri, lf[i][rows, np.maximum(lev, 0)], 0.0)
        M = decay * lvl
        out[i] = ((qf[i] @ kf[i].T) * M) @ vf[i]
    return out.reshape(*lead, T, dv)


def form_a_rows(q, k, v, a, lam, rows) -> np.ndarray:
    """Form A for selected query rows of one (batch, head) slice.

    q, k [T, dk]; v [T, dv]; a [T]; lam [T, L]; rows: iterable of positions.
    Returns [len(rows), dv].  Each row costs O(t (dk + dv)).
    """
    a = np.asarray(a, dtype=np.float64)
    A = np.cumsum(a)
    rows = [int(r) for r in rows]
    out = np.zeros((len(rows), v.shape[-1]))
    for n, t in enumerate(rows):
        lev = level_row(t).astype(np.int64)
        w = np.asarray(lam[t], dtype=np.float64)[lev] * np.exp(A[t] - A[: t + 1])
        scores = np.asarray(k[: t + 1], dtype=np.float64) @ np.asarray(q[t], dtype=np.float64)
        out[n] = (scores * w) @ np.asarray(v[: t + 1], dtype=np.float64)
    return out


# --------------------------------------------------------------------------
# Gradients of Form A (the backward pass)

def _running_sum_grad(W):
    """dA_t = sum_s W[t, s] - sum_t' W[t', t] for W = dP (.) P."""
    return W.sum(axis=1) - W.sum(axis=0)


def _suffix_sum(x):
    """y_j = sum_{t >= j} x_t."""
    return np.cumsum(x[::-1])[::-1]


def form_a_grads(q, k, v, a, lam, dout):
    """Gradients of sum(O * dout) for O = form_a(q, k, v, a, lam), in fp64.

    "Log-linear attention, and what a logarithm buys", section 3 trains the
    mixer forward and backward, and section 6 notes that the gradients of the
    lambda terms have to be derived by hand.  This is the chain rule through
    section 1's masked form O = P V with P = (Q K^T) (.) M and
    M[t, s] = lambda_t^(level(t, s)) exp(A_t - A_s), s <= t, A the running
    sum of a:

      dP = dO V^T                 (cotangent of P, kept below the diagonal)
      dV = P^T dO
      dQ = (dP (.) M) K,          dK = (dP (.) M)^T Q
      dlambda_t^(l) = sum over the keys s of level l of dP[t, s] (q_t . k_s) exp(A_t - A_s)
      dA_t = sum_s W[t, s] - sum_t' W[t', t],   W = dP (.) P
             (A_t enters row t of M with a plus sign and column t with a minus)
      da_j = sum_{t >= j} dA_t    (a_j is in A_t for every t >= j)

    Shapes as in form_a, dout like the output.  Returns (dq, dk, dv, da, dlam).
    """
    q, k, v, a, lam, dout = map(_f64, (q, k, v, a, lam, dout))
    lead = q.shape[:-2]
    T, dk = q.shape[-2:]
    dv = v.shape[-1]
    L = lam.shape[-1]
    lev = level_map(T).astype(np.int64)
    tri = lev >= 0
    if T > 0 and lev.max() >= L:
        raise ValueError(f"lambda has {L} levels; T={T} needs {lev.max() + 1}")
    qf, kf, vf = q.reshape(-1, T, dk), k.reshape(-1, T, dk), v.reshape(-1, T, dv)
    af, lf, gf = a.reshape(-1, T), lam.reshape(-1, T, L), dout.reshape(-1, T, dv)
    n = qf.shape[0]
    dq, dkk, dvv = np.zeros_like(qf), np.zeros_like(kf), np.zeros_like(vf)
    da, dlam = np.zeros_like(af), np.zeros_like(lf)
    rows = np.arange(T)[:, None]
    for i in range(n):
        A = np.cumsum(af[i])
        decay = np.where(tri, np.exp(np.where(tri, A[:, None] - A[None, :], 0.0)), 0.0)
        M = decay * np.where(tri, lf[i][rows, np.maximum(lev, 0)], 0.0)
        S = qf[i] @ kf[i].T
        P = S * M
        dP = np.where(tri, gf[i] @ vf[i].T, 0.0)
        dvv[i] = P.T @ gf[i]
        dq[i] = (dP * M) @ kf[i]
        dkk[i] = (dP * M).T @ qf[i]
        G = dP * S * decay  # derivative of the loss in the weight lambda_t^(level)
        for l in range(L):
            dlam[i][:, l] = np.sum(np.where(lev == l, G, 0.0), axis=1)
        da[i] = _suffix_sum(_running_sum_grad(dP * P))
    return (dq.reshape(*lead, T, dk), dkk.reshape(*lead, T, dk), dvv.reshape(*lead, T, dv),
            da.reshape(*lead, T), dlam.reshape(*lead, T, L))


# --------------------------------------------------------------------------
# Form B: the Fenwick recurrence (C)

def form_b(q, k, v, a, lam, nthreads: int | None = None, return_states: bool = False):
    """Token-by-token Fenwick recurrence over whole sequences (fp64).

    Shapes as in form_a.  With return_states, also returns the level states
    after the last token, [..., L, dk, dv] (S = sum k v^T orientation).
    """
    q, k, v, a, lam = map(_f64, (q, k, v, a, lam))
    lead = q.shape[:-2]
    T, dk = q.shape[-2:]
    dv = v.shape[-1]
    L = lam.shape[-1]
    BH = int(np.prod(lead)) if lead else 1
    out = np.zeros((BH, T, dv))
    st = np.zeros((BH, L, dk, dv)) if return_states else None
    rc = _load().llo_fwd_recurrent(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(lam), _ptr(out),
                                   _ptr(st) if st is not None else None, BH, T, dk, dv, L,
                                   nthreads or default_threads())
    if rc != LLO_OK:
        raise RuntimeError(f"oracle recurrence failed with code {rc}")
    out = out.reshape(*lead, T, dv)
    if return_states:
        return out, st.reshape(*lead, L, dk, dv)
    return out


def decode(states, pos, q, k, v, a, lam, nthreads: int | None = None):
    """Continue P independent (sequence, head) pairs by `steps` tokens.

    states [P, L, dk, dv]; pos [P] next positions; q, k [steps, P, dk];
    v [steps, P, dv]; a [steps, P]; lam [steps, P, L].
    Returns (out [steps, P, dv], states_after, pos_after).
    """
    st = _f64(states).copy()
    ps = np.ascontiguousarray(np.asarray(pos, dtype=np.int64)).copy()
    q, k, v, a, lam = map(_f64, (q, k, v, a, lam))
    steps, P, dk = q.shape
    dv = v.shape[-1]
    L = st.shape[1]
    out = np.zeros((steps, P, dv))
    rc = _load().llo_decode(_ptr(st), _ptr(ps, ctypes.c_int64), _ptr(q), _ptr(k), _ptr(v),
                            _ptr(a), _ptr(lam), _ptr(out), P, steps, dk, dv, L,
                            nthreads or default_threads())
    if rc != LLO_OK:
        raise RuntimeError(f"oracle decode failed with code {rc}")
    return out, st, ps


# --------------------------------------------------------------------------
# Log-linear Gated DeltaNet

def gdn_form_a(q, k, v, a, beta, lam) -> np.ndarray:
    """Log-linear Gated DeltaNet with the mask written out, per slice (fp64).

    The gated delta rule (the Gated DeltaNet paper, the page's source 3) is
    S_t = exp(a_t) (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T with
    o_t = S_t^T q_t.  Its masked form P = A (.) M^S, O = P V has the
    1-semiseparable decay mask M^S[t, s] = exp(A_t - A_s) of Mamba-2 and the
    query-key interaction
        A = (Q K^T (.) L) (I + diag(beta) (K K^T (.) (L - I)))^-1 diag(beta),
    L the lower triangle with the diagonal; the decay factors out of the
    inverse because it is a diagonal similarity (section 1: Gated DeltaNet
    changes A, not M).  Section 3 lifts it by the elementwise product with the
    level mask: P = A (.) M^S (.) M^H, M^H[t, s] = lambda_t^(level(t, s)).

    q, k [..., T, dk]; v [..., T, dv]; a, beta [..., T]; lam [..., T, L].
    Allocates T x T per slice (meant for T up to a few thousand).
    """
    from scipy.linalg import solve_triangular

    q, k, v, a, beta, lam = map(_f64, (q, k, v, a, beta, lam))
    lead = q.shape[:-2]
    T, dk = q.shape[-2:]
    dv = v.shape[-1]
    L = lam.shape[-1]
    lev = level_map(T).astype(np.int64)
    tri = lev >= 0                      # s <= t
    strict = np.tril(np.ones((T, T), dtype=bool), -1)
    if T > 0 and lev.max() >= L:
        raise ValueError(f"lambda has {L} levels; T={T} needs {lev.max() + 1}")
    qf, kf, vf = q.reshape(-1, T, dk), k.reshape(-1, T, dk), v.reshape(-1, T, dv)
    af, bf, lf = a.reshape(-1, T), beta.reshape(-1, T), lam.reshape(-1, T, L)
    out = np.zeros((qf.shape[0], T, dv))
    rows = np.arange(T)[:, None]
    for i in range(qf.shape[0]):
        A = np.cumsum(af[i])
        # unit lower-triangular system of the delta rule, solved for diag(beta)
        system = np.eye(T) + bf[i][:, None] * np.where(strict, kf[i] @ kf[i].T, 0.0)
        inv_beta = solve_triangular(system, np.diag(bf[i]), lower=True, unit_diagonal=True)
        interaction = np.where(tri, qf[i] @ kf[i].T, 0.0) @ inv_beta
        decay = np.where(tri, np.exp(np.where(tri, A[:, None] - A[None, :], 0.0)), 0.0)
        lvl = np.where(tri, lf[i][rows, np.maximum(lev, 0)], 0.0)
        out[i] = (interaction * decay * lvl) @ vf[i]
    return out.reshape(*lead, T, dv)


def gdn_form_b(q, k, v, a, beta, lam, nthreads: int | None = None, return_states: bool = False):
    """Log-linear Gated DeltaNet by the token-by-token Fenwick recurrence (C,
    fp64): every carried or merged bucket state goes through
    exp(a_t) (I - beta_t k_t k_t^T) at each step and beta_t k_t v_t^T enters
    level 0.  Shapes as in gdn_form_a; with return_states also the level
    states after the last token, [..., L, dk, dv]."""
    q, k, v, a, beta, lam = map(_f64, (q, k, v, a, beta, lam))
    lead = q.shape[:-2]
    T, dk = q.shape[-2:]
    dv = v.shape[-1]
    L = lam.shape[-1]
    BH = int(np.prod(lead)) if lead else 1
    out = np.zeros((BH, T, dv))
    st = np.zeros((BH, L, dk, dv)) if return_states else None
    rc = _load().llo_gdn_fwd_recurrent(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(beta), _ptr(lam),
                                       _ptr(out), _ptr(st) if st is not None else None, BH, T,
                                       dk, dv, L, nthreads or default_threads())
    if rc != LLO_OK:
        raise RuntimeError(f"oracle Gated DeltaNet recurrence failed with code {rc}")
    out = out.reshape(*lead, T, dv)
    if return_states:
        return out, st.reshape(*lead, L, dk, dv)
    return out


def gdn_decode(states, pos, q, k, v, a, beta, lam, nthreads: int | None = None):
    """Continue P (sequence, head) pairs of the log-linear Gated DeltaNet by
    `steps` tokens; as decode() with beta [steps, P]."""
    st = _f64(states).copy()
    ps = np.ascontiguousarray(np.asarray(pos, dtype=np.int64)).copy()
    q, k, v, a, beta, lam = map(_f64, (q, k, v, a, beta, lam))
    steps, P, dk = q.shape
    dv = v.shape[-1]
    L = st.shape[1]
    out = np.zeros((steps, P, dv))
    rc = _load().llo_gdn_decode(_ptr(st), _ptr(ps, ctypes.c_int64), _ptr(q), _ptr(k), _ptr(v),
                                _ptr(a), _ptr(beta), _ptr(lam), _ptr(out), P, steps, dk, dv, L,
                                nthreads or default_threads())
    if rc != LLO_OK:
        raise RuntimeError(f"oracle Gated DeltaNet decode failed with code {rc}")
    return out, st, ps
