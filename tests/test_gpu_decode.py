"""GPU parity of the Fenwick decode step against the fp64 oracle recurrence.

Page: "Log-linear attention, and what a logarithm buys", section 2 (decode
recurrence).  States are compared per (sequence, head, level) slice.
"""
import numpy as np
import pytest
import torch

from log_linear_token_amd import inputs as I
from log_linear_token_amd import loglin as LL
from oracle import reference as ref
from tests.helpers import TOL_BF16, TOL_F32, banner, slice_rel_err, state_rel_err, to_dev

pytestmark = pytest.mark.gpu


def _decode_gpu(d, states_np, dtype=torch.bfloat16, steps=None):
    cfg = d["cfg"]
    steps = cfg.steps if steps is None else steps
    st = LL.loglin_state_init(cfg.nseq, cfg.H, cfg.dk, cfg.dv, cfg.Lmax)
    LL.loglin_state_load(st, d["pos"], to_dev(states_np) if states_np is not None else None)
    q, k, v = to_dev(d["q"][:steps], dtype), to_dev(d["k"][:steps], dtype), to_dev(d["v"][:steps], dtype)
    a, lam = to_dev(d["a"][:steps]), to_dev(d["lam"][:steps])
    outs = torch.empty((steps, cfg.nseq, cfg.H, cfg.dv), device="cuda")
    for s in range(steps):
        LL.loglin_decode_step(st, q[s], k[s], v[s], a[s], lam[s], out=outs[s])
    pos, lv = LL.loglin_state_export(st)
    torch.cuda.synchronize()
    res = outs.cpu().numpy(), pos.numpy(), lv.cpu().numpy()
    LL.loglin_state_free(st)
    return res


def _oracle(d, states_np, pairs, steps):
    """Run the oracle for the listed (seq, head) pairs; returns out [steps, P, dv], states, pos."""
    cfg = d["cfg"]
    st = np.stack([states_np[s, h] for s, h in pairs]).astype(np.float64)
    pos = np.array([d["pos"][s] for s, _ in pairs], np.int64)
    sel = lambda x: np.stack([x[:steps, s, h] for s, h in pairs], axis=1)  # noqa: E731
    return ref.decode(st, pos, sel(d["q"]), sel(d["k"]), sel(d["v"]),
                      np.stack([d["a"][:steps, s, h] for s, h in pairs], axis=1),
                      sel(d["lam"]))


def _live_mask_ok(levels, pos, Lmax, live_nonzero=True):
    """Exported slots that are not live must be exactly zero; live slots must
    hold data (checked unless decay may have flushed old levels to zero)."""
    for s, n in enumerate(pos):
        live = set(ref.live_slots(int(n)))
        for lv in range(Lmax):
            nz = bool(np.any(levels[s, :, lv] != 0))
            if lv not in live and nz:
                return False, (s, int(n), lv, "dead slot not zero")
            if lv in live and live_nonzero and not nz:
                return False, (s, int(n), lv, "live slot empty")
    return True, None


@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (128, 128), (64, 16)])
def test_true_prefill_then_decode(dk, dv):
    """States built by the oracle recurrence from real tokens, then 40 GPU steps."""
    banner(f"decode true prefill dk={dk} dv={dv}")
    rng = np.random.default_rng(dk * 7 + dv)
    cfg = I.CONFIGS["decode"].scaled(nseq=4, H=2, dk=dk, dv=dv, Lmax=12, steps=40,
                                     max_prefill=600)
    d = I.make_decode(cfg, "base", seed=dk + dv, fill=False)
    d["pos"] = np.array([0, 1, 37, 512], np.int64)  # empty, one token, ragged, power of two
    states = np.zeros((cfg.nseq, cfg.H, cfg.Lmax, dk, dv), np.float32)
    for s, n in enumerate(d["pos"]):
        if n == 0:
            continue
        for h in range(cfg.H):
            q = rng.standard_normal((n, dk)) / np.sqrt(dk)
            k = rng.standard_normal((n, dk)) / np.sqrt(dk)
            v = rng.standard_normal((n, dv))
            a = -np.logaddexp(0, rng.standard_normal(n) - 3.0)
            lam = rng.random((n, cfg.Lmax))
            _, st = ref.form_b(q, k, v, a, lam, return_states=True)
            states[s, h] = st.astype(np.float32)
    out, pos, lv = _decode_gpu(d, states)
    pairs = [(s, h) for s in range(cfg.nseq) for h in range(cfg.H)]
    o_ref, st_ref, pos_ref = _oracle(d, states, pairs, cfg.steps)
    got = out.reshape(cfg.steps, -1, dv).transpose(1, 0, 2)
    assert slice_rel_err(got, o_ref.transpose(1, 0, 2), 1) <= TOL_BF16
    assert np.array_equal(pos, pos_ref.reshape(cfg.nseq, cfg.H)[:, 0])
    lv_pairs = lv.reshape(-1, cfg.Lmax, dk, dv)
    assert state_rel_err(lv_pairs, st_ref) <= TOL_BF16
    ok, where = _live_mask_ok(lv, pos, cfg.Lmax)
    assert ok, where


def test_decode_from_empty_matches_materialised_mask():
    """fp32 inputs from position 0: outputs equal Form A of the whole sequence."""
    banner("decode from empty, f32")
    rng = np.random.default_rng(3)
    T, dk, dv, L = 300, 32, 16, 10
    q = (rng.standard_normal((T, dk)) / np.sqrt(dk)).astype(np.float32)
    k = (rng.standard_normal((T, dk)) / np.sqrt(dk)).astype(np.float32)
    v = rng.standard_normal((T, dv)).astype(np.float32)
    a = (-np.logaddexp(0, rng.standard_normal(T) - 4)).astype(np.float32)
    lam = rng.random((T, L)).astype(np.float32)
    st = LL.loglin_state_init(1, 1, dk, dv, L)
    outs = []
    for t in range(T):
        o = LL.loglin_decode_step(st, to_dev(q[t:t + 1, None]).reshape(1, 1, dk),
                                  to_dev(k[t:t + 1]).reshape(1, 1, dk),
                                  to_dev(v[t:t + 1]).reshape(1, 1, dv),
                                  to_dev(a[t:t + 1]).reshape(1, 1),
                                  to_dev(lam[t:t + 1]).reshape(1, 1, L))
        outs.append(o.reshape(dv))
    got = torch.stack(outs).cpu().numpy()
    LL.loglin_state_free(st)
    want = ref.form_a(q, k, v, a, lam)
    assert slice_rel_err(got, want, 0) <= TOL_F32


def test_synthetic_prefill_reduced():
    banner("decode synthetic prefill, reduced batch")
    cfg = I.CONFIGS["decode"].scaled(nseq=8, H=4, steps=64)
    d = I.make_decode(cfg, "base", seed=11, live_slots=ref.live_slots)
    out, pos, lv = _decode_gpu(d, d["states"])
    pairs = [(s, h) for s in range(cfg.nseq) for h in range(cfg.H)]
    o_ref, st_ref, _ = _oracle(d, d["states"], pairs, cfg.steps)
    got = out.reshape(cfg.steps, -1, cfg.dv).transpose(1, 0, 2)
    assert slice_rel_err(got, o_ref.transpose(1, 0, 2), 1) <= TOL_BF16
    assert state_rel_err(lv.reshape(-1, cfg.Lmax, cfg.dk, cfg.dv), st_ref) <= TOL_BF16
    ok, where = _live_mask_ok(lv, pos, cfg.Lmax)
    assert ok, where


@pytest.mark.parametrize("variant", ["base", "unit"])
def test_decode_workload_full_size(variant):
    """128 sequences x 32 heads, 17 levels of 128 x 128, 256 steps on the GPU;
    the oracle follows 24 sampled (sequence, head) pairs through every step."""
    cfg = I.CONFIGS["decode"]
    banner(f"decode full size {variant}")
    d = I.make_decode(cfg, variant, live_slots=ref.live_slots)
    out, pos, lv = _decode_gpu(d, d["states"])
    rng = np.random.default_rng(4)
    pairs = sorted({(int(s), int(h)) for s, h in zip(rng.integers(0, cfg.nseq, 24),
                                                     rng.integers(0, cfg.H, 24))})
    o_ref, st_ref, pos_ref = _oracle(d, d["states"], pairs, cfg.steps)
    got = np.stack([out[:, s, h] for s, h in pairs], axis=0)
    err_o = slice_rel_err(got, o_ref.transpose(1, 0, 2), 1)
    got_st = np.stack([lv[s, h] for s, h in pairs])
    err_s = state_rel_err(got_st, st_ref)
    print(f"  decode {variant}: out err {err_o:.3e} state err {err_s:.3e}", flush=True)
    assert err_o <= TOL_BF16 and err_s <= TOL_BF16
    assert np.array_equal(pos, d["pos"] + cfg.steps)
    # with the workload's decay (about e^-180 over 256 steps) the oldest levels
    # underflow fp32, so only the no-decay variant requires live slots to be nonzero
    ok, where = _live_mask_ok(lv, pos, cfg.Lmax, live_nonzero=(variant == "unit"))
    assert ok, where


def test_capacity_is_enforced():
    banner("decode capacity")
    st = LL.loglin_state_init(2, 1, 16, 16, 4)
    with pytest.raises(LL.LoglinError) as ei:
        LL.loglin_state_load(st, [0, 9])
    assert ei.value.status == LL.LOGLIN_ECAPACITY
    LL.loglin_state_load(st, [0, 8])
    z = torch.zeros((2, 1, 16), device="cuda")
    with pytest.raises(LL.LoglinError) as ei:
        LL.loglin_decode_step(st, z, z, z, torch.zeros((2, 1), device="cuda"),
                              torch.zeros((2, 1, 4), device="cuda"))
    assert ei.value.status == LL.LOGLIN_ECAPACITY
    LL.loglin_state_load(st, [0, 7])
    LL.loglin_decode_step(st, z, z, z, torch.zeros((2, 1), device="cuda"),
                          torch.zeros((2, 1, 4), device="cuda"))
    pos, _ = LL.loglin_state_export(st, levels=False)
    assert list(pos.numpy()) == [1, 8]
    LL.loglin_state_free(st)


def test_decode_agrees_with_chunked_forward():
    """The two GPU paths of the same mixer: decode from empty vs chunked forward."""
    banner("decode vs chunked forward")
    cfg = I.CONFIGS["fwd2k"].scaled(B=1, H=4, T=512, dk=64, dv=64, C=64, L=11)
    d = I.make_fwd(cfg, "weak", seed=5)
    fwd = LL.loglin_fwd_chunked(to_dev(d["q"], torch.bfloat16), to_dev(d["k"], torch.bfloat16),
                                to_dev(d["v"], torch.bfloat16), to_dev(d["a"]), to_dev(d["lam"]),
                                64).cpu().numpy()
    st = LL.loglin_state_init(1, 4, 64, 64, 11)
    q = to_dev(d["q"][0].transpose(1, 0, 2), torch.bfloat16)
    k = to_dev(d["k"][0].transpose(1, 0, 2), torch.bfloat16)
    v = to_dev(d["v"][0].transpose(1, 0, 2), torch.bfloat16)
    a = to_dev(d["a"][0].T)
    lam = to_dev(d["lam"][0].transpose(1, 0, 2))
    outs = [LL.loglin_decode_step(st, q[t][None], k[t][None], v[t][None], a[t][None],
                                  lam[t][None]) for t in range(cfg.T)]
    dec = torch.stack(outs).cpu().numpy()[:, 0].transpose(1, 0, 2)[None]
    LL.loglin_state_free(st)
    want = ref.form_b(d["q"], d["k"], d["v"], d["a"], d["lam"])
    assert slice_rel_err(dec, want, 2) <= TOL_BF16
    assert slice_rel_err(fwd, want, 2) <= TOL_BF16


def _tok(x, t):
    return to_dev(np.ascontiguousarray(x[:, :, t]))


@pytest.mark.parametrize("dk,dv", [(32, 16), (128, 128)])
def test_window_export_matches_recurrence_states(dk, dv):
    """Decode from empty with fp32 inputs; export the states inside a window,
    at its last token and right after a boundary, and compare every level with
    the oracle recurrence's states after the same tokens (levels 0..6 of the
    window are summed from raw rows on export)."""
    banner(f"decode window export dk={dk} dv={dv}")
    rng = np.random.default_rng(dk + dv)
    B, H, T = 1, 2, 200
    L = (T - 1).bit_length() + 1
    q = (rng.standard_normal((B, H, T, dk)) / np.sqrt(dk)).astype(np.float32)
    k = (rng.standard_normal((B, H, T, dk)) / np.sqrt(dk)).astype(np.float32)
    v = rng.standard_normal((B, H, T, dv)).astype(np.float32)
    a = (-np.logaddexp(0, rng.standard_normal((B, H, T)) - 5)).astype(np.float32)
    lam = rng.random((B, H, T, L)).astype(np.float32)
    st = LL.loglin_state_init(B, H, dk, dv, L)
    checks = {37, 63, 64, 65, 128, 129, 200}
    for t in range(T):
        LL.loglin_decode_step(st, _tok(q, t), _tok(k, t), _tok(v, t), _tok(a, t), _tok(lam, t))
        n = t + 1
        if n in checks:
            pos, lv = LL.loglin_state_export(st)
            assert int(pos[0]) == n
            _, want = ref.form_b(q[:, :, :n], k[:, :, :n], v[:, :, :n], a[:, :, :n],
                                 lam[:, :, :n], return_states=True)
            err = state_rel_err(lv.cpu().numpy().reshape(B * H, L, dk, dv),
                                want.reshape(B * H, L, dk, dv))
            assert err <= TOL_F32, (n, err)
            live = set(ref.live_slots(n))
            got = lv.cpu().numpy()
            for lev in range(L):
                if lev not in live:
                    assert not np.any(got[:, :, lev]), (n, lev)
    LL.loglin_state_free(st)


@pytest.mark.parametrize("stop", [40, 64, 100, 127])
def test_export_load_resume_matches_uninterrupted(stop):
    """Export mid-way (window rows become matrices), load into a new state,
    continue: outputs match the uninterrupted decode and the oracle."""
    banner(f"decode export/load/resume at {stop}")
    rng = np.random.default_rng(stop)
    B, H, T, dk, dv = 2, 2, 180, 64, 32
    L = (T - 1).bit_length() + 1
    q = (rng.standard_normal((B, H, T, dk)) / np.sqrt(dk)).astype(np.float32)
    k = (rng.standard_normal((B, H, T, dk)) / np.sqrt(dk)).astype(np.float32)
    v = rng.standard_normal((B, H, T, dv)).astype(np.float32)
    a = (-np.logaddexp(0, rng.standard_normal((B, H, T)) - 5)).astype(np.float32)
    lam = rng.random((B, H, T, L)).astype(np.float32)
    st = LL.loglin_state_init(B, H, dk, dv, L)
    outs = []
    for t in range(stop):
        outs.append(LL.loglin_decode_step(st, _tok(q, t), _tok(k, t), _tok(v, t), _tok(a, t),
                                          _tok(lam, t)).cpu().numpy())
    pos, lv = LL.loglin_state_export(st)
    st2 = LL.loglin_state_init(B, H, dk, dv, L)
    LL.loglin_state_load(st2, pos.numpy(), lv)
    for t in range(stop, T):
        o1 = LL.loglin_decode_step(st, _tok(q, t), _tok(k, t), _tok(v, t), _tok(a, t), _tok(lam, t))
        o2 = LL.loglin_decode_step(st2, _tok(q, t), _tok(k, t), _tok(v, t), _tok(a, t), _tok(lam, t))
        outs.append(o2.cpu().numpy())
        assert np.allclose(o1.cpu().numpy(), o2.cpu().numpy(), rtol=1e-5, atol=1e-5), t
    LL.loglin_state_free(st)
    LL.loglin_state_free(st2)
    got = np.stack(outs, axis=2)  # [B, H, T, dv]
    want = ref.form_a(q, k, v, a, lam)
    assert slice_rel_err(got, want, 2) <= TOL_F32


def test_one_state_serves_one_mixer():
    banner("decode state kind")
    st = LL.loglin_state_init(1, 1, 16, 16, 6)
    z = torch.zeros((1, 1, 16), device="cuda")
    s1 = torch.zeros((1, 1), device="cuda")
    lam = torch.zeros((1, 1, 6), device="cuda")
    LL.loglin_decode_step(st, z, z, z, s1, lam)
    with pytest.raises(LL.LoglinError) as ei:
        LL.loglin_gdn_decode_step(st, z, z, z, s1, s1, lam)
    assert ei.value.status == LL.LOGLIN_EINVAL
    LL.loglin_state_load(st, [1])  # a load starts over
    LL.loglin_gdn_decode_step(st, z, z, z, s1, s1, lam)
    with pytest.raises(LL.LoglinError):
        LL.loglin_decode_step(st, z, z, z, s1, lam)
    LL.loglin_state_free(st)


def test_decode_deterministic():
    """Two runs from the same state give bit-identical outputs and states."""
    banner("determinism decode")
    cfg = I.CONFIGS["decode"].scaled(nseq=2, H=2, steps=70)
    d = I.make_decode(cfg, "base", seed=11, live_slots=ref.live_slots)
    st = d["states"]
    o1, p1, s1 = _decode_gpu(d, st)
    o2, p2, s2 = _decode_gpu(d, st)
    assert np.array_equal(o1, o2) and np.array_equal(p1, p2) and np.array_equal(s1, s2)
