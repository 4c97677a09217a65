"""GPU parity of the log-linear Gated DeltaNet (chunked forward and decode)
against the fp64 oracle.

Page: "Log-linear attention, and what a logarithm buys" -- section 1 (Gated
DeltaNet changes the query-key interaction, not the mask), section 2 (the
Fenwick buckets and the decode recurrence), section 3 (the lift composes the
temporal mask with the level mask); the gated delta rule is that of the
Gated DeltaNet paper (the page's source 3).  Every case prints a banner
naming itself before touching the GPU.
"""
import numpy as np
import pytest
import torch

from log_linear_token_amd import inputs as I
from log_linear_token_amd import loglin as LL
from oracle import reference as ref
from tests.helpers import (TOL_BF16, TOL_F32, banner, in_dtype, slice_rel_err, state_rel_err,
                           to_dev)

pytestmark = pytest.mark.gpu


def _run(d, C=64):
    cfg = d["cfg"]
    dt = in_dtype(cfg.dtype)
    q, k, v = to_dev(d["q"], dt), to_dev(d["k"], dt), to_dev(d["v"], dt)
    out = LL.loglin_gdn_fwd_chunked(q, k, v, to_dev(d["a"]), to_dev(d["beta"]), to_dev(d["lam"]), C)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _tol(cfg):
    return TOL_BF16 if cfg.dtype == "bf16" else TOL_F32


def _oracle_a(d):
    return ref.gdn_form_a(d["q"], d["k"], d["v"], d["a"], d["beta"], d["lam"])


def _cfg(T, dk, dv, dtype, L=None, B=2, H=2):
    L = L or max(1, (T - 1).bit_length() + 1)
    return I.CONFIGS["gdn2k"].scaled(B=B, H=H, T=T, dk=dk, dv=dv, C=64, L=L, dtype=dtype)


SMALL = [
    # (T, dk, dv, dtype): one token, inside one chunk, chunk edges, ragged tails,
    # several chunk levels
    (1, 64, 64, "f32"), (63, 64, 16, "f32"), (64, 128, 32, "f32"), (65, 64, 64, "f32"),
    (300, 128, 64, "f32"), (777, 64, 32, "f32"),
    (1, 128, 64, "bf16"), (64, 64, 64, "bf16"), (129, 128, 16, "bf16"), (500, 64, 64, "bf16"),
    (1000, 128, 64, "bf16"), (1600, 64, 32, "bf16"),
]


@pytest.mark.parametrize("variant", ["base", "unit", "weak"])
@pytest.mark.parametrize("T,dk,dv,dtype", SMALL)
def test_gdn_small_vs_masked_form(T, dk, dv, dtype, variant):
    banner(f"gdn small T={T} dk={dk} dv={dv} {dtype} {variant}")
    cfg = _cfg(T, dk, dv, dtype, L=max(1, (T - 1).bit_length() + 1) + (T % 2))
    d = I.make_gdn(cfg, variant, seed=T + dk + dv)
    got = _run(d)
    want = _oracle_a(d)
    err = slice_rel_err(got, want, 2)
    print(f"  gdn T={T} {dtype} {variant}: {err:.3e}", flush=True)
    assert err <= _tol(cfg), err


@pytest.mark.parametrize("C", [16, 32, 128])
def test_gdn_chunk_argument_does_not_change_the_result(C):
    banner(f"gdn C={C}")
    d = I.make_gdn(_cfg(700, 64, 64, "bf16"), "weak", seed=C)
    got = _run(d, C=C)
    assert np.array_equal(got, _run(d, C=64))


@pytest.mark.parametrize("stage", ["intra_only", "inter_only"])
def test_gdn_stage_isolation(stage):
    """lambda zero on the chunk levels tests the per-chunk block alone; zero on
    the levels inside a chunk tests the level walk alone (unit decay)."""
    banner(f"gdn stage isolation {stage}")
    d = I.make_gdn(_cfg(1500, 128, 64, "bf16", B=1, H=3), "unit", seed=21)
    if stage == "intra_only":
        d["lam"][..., 7:] = 0.0
    else:
        d["lam"][..., :7] = 0.0
    got = _run(d)
    want = _oracle_a(d)
    assert np.max(np.abs(want)) > 0.1
    err = slice_rel_err(got, want, 2)
    assert err <= TOL_BF16, err


@pytest.mark.parametrize("level", [7, 8, 9, 10, 11])
def test_gdn_one_hot_chunk_level(level):
    """lambda one-hot on one chunk level (weak decay): one level state of the
    walk read per chunk, against the masked form."""
    banner(f"gdn one-hot level {level}")
    d = I.make_gdn(_cfg(2048 + 37, 64, 32, "bf16", B=1, H=2), "weak", seed=level)
    d["lam"][:] = 0.0
    d["lam"][..., level] = 1.0
    got = _run(d)
    want = _oracle_a(d)
    assert np.max(np.abs(want)) > 0.01
    err = slice_rel_err(got, want, 2)
    assert err <= TOL_BF16, err


def test_gdn_deterministic():
    banner("gdn determinism")
    d = I.make_gdn(_cfg(1000, 128, 64, "bf16"), "base", seed=3)
    assert np.array_equal(_run(d), _run(d))


@pytest.mark.parametrize("variant", ["base", "unit", "weak"])
def test_gdn2k_workload(variant):
    banner(f"gdn2k {variant} (full size)")
    d = I.make_gdn(I.CONFIGS["gdn2k"], variant)
    got = _run(d)
    want = ref.gdn_form_b(d["q"], d["k"], d["v"], d["a"], d["beta"], d["lam"])
    err = slice_rel_err(got, want, 2)
    print(f"  gdn2k {variant}: {err:.3e}", flush=True)
    assert err <= TOL_BF16, err


@pytest.mark.parametrize("variant", ["base", "weak"])
def test_gdn8k_workload(variant):
    """The full 8K batch on the GPU; the oracle recurrence follows two whole
    slices (all 8192 positions)."""
    cfg = I.CONFIGS["gdn8k"]
    banner(f"gdn8k {variant} (full size)")
    d = I.make_gdn(cfg, variant)
    got = _run(d)
    errs = []
    for b, h in [(0, 0), (3, 15)]:
        want = ref.gdn_form_b(d["q"][b, h], d["k"][b, h], d["v"][b, h], d["a"][b, h],
                              d["beta"][b, h], d["lam"][b, h])
        errs.append(slice_rel_err(got[b, h], want, 0))
    print(f"  gdn8k {variant}: {max(errs):.3e}", flush=True)
    assert max(errs) <= TOL_BF16, errs


def test_gdn_rejects_unsupported_dims():
    q = torch.zeros((1, 1, 64, 32), device="cuda")
    a = torch.zeros((1, 1, 64), device="cuda")
    lam = torch.zeros((1, 1, 64, 8), device="cuda")
    with pytest.raises(LL.LoglinError) as ei:
        LL.loglin_gdn_fwd_chunked(q, q, q, a, a, lam, 64)
    assert ei.value.status == LL.LOGLIN_EUNSUPPORTED


# ------------------------------------------------------------------ decode

def _gdn_decode_gpu(d, states_np, steps, dtype=torch.bfloat16):
    cfg = d["cfg"]
    st = LL.loglin_state_init(cfg.nseq, cfg.H, cfg.dk, cfg.dv, cfg.Lmax)
    LL.loglin_state_load(st, d["pos"], to_dev(states_np) if states_np is not None else None)
    q, k, v = (to_dev(d[n][:steps], dtype) for n in ("q", "k", "v"))
    a, beta, lam = to_dev(d["a"][:steps]), to_dev(d["beta"][:steps]), to_dev(d["lam"][:steps])
    outs = torch.empty((steps, cfg.nseq, cfg.H, cfg.dv), device="cuda")
    for s in range(steps):
        LL.loglin_gdn_decode_step(st, q[s], k[s], v[s], a[s], beta[s], lam[s], out=outs[s])
    pos, lv = LL.loglin_state_export(st)
    torch.cuda.synchronize()
    res = outs.cpu().numpy(), pos.numpy(), lv.cpu().numpy()
    LL.loglin_state_free(st)
    return res


def _gdn_decode_oracle(d, states_np, pairs, steps):
    sel = lambda x: np.stack([x[:steps, s, h] for s, h in pairs], axis=1)  # noqa: E731
    st = np.stack([states_np[s, h] for s, h in pairs]).astype(np.float64)
    pos = np.array([d["pos"][s] for s, _ in pairs], np.int64)
    return ref.gdn_decode(st, pos, sel(d["q"]), sel(d["k"]), sel(d["v"]), sel(d["a"]),
                          sel(d["beta"]), sel(d["lam"]))


def test_gdn_decode_synthetic_prefill_reduced():
    banner("gdn decode synthetic prefill, reduced batch")
    cfg = I.CONFIGS["gdn_decode"].scaled(nseq=8, H=4, steps=64)
    d = I.make_decode(cfg, "base", seed=12, live_slots=ref.live_slots)
    out, pos, lv = _gdn_decode_gpu(d, d["states"], cfg.steps)
    pairs = [(s, h) for s in range(cfg.nseq) for h in range(cfg.H)]
    o_ref, st_ref, pos_ref = _gdn_decode_oracle(d, d["states"], pairs, cfg.steps)
    got = out.reshape(cfg.steps, -1, cfg.dv).transpose(1, 0, 2)
    assert slice_rel_err(got, o_ref.transpose(1, 0, 2), 1) <= TOL_BF16
    assert state_rel_err(lv.reshape(-1, cfg.Lmax, cfg.dk, cfg.dv), st_ref) <= TOL_BF16
    assert np.array_equal(pos, pos_ref.reshape(cfg.nseq, cfg.H)[:, 0])


def test_gdn_decode_from_empty_matches_masked_form():
    """fp32 inputs from position 0: outputs equal the masked form of the whole
    sequence."""
    banner("gdn decode from empty, f32")
    cfg = _cfg(300, 32, 16, "f32", B=1, H=1)
    d = I.make_gdn(cfg, "weak", seed=4)
    T, L = cfg.T, cfg.L
    st = LL.loglin_state_init(1, 1, 32, 16, L)
    outs = []
    for t in range(T):
        g = lambda x, n: to_dev(np.ascontiguousarray(x[0, 0, t])).reshape(1, 1, n)  # noqa: E731
        o = LL.loglin_gdn_decode_step(st, g(d["q"], 32), g(d["k"], 32), g(d["v"], 16),
                                      to_dev(d["a"][0, 0, t:t + 1]).reshape(1, 1),
                                      to_dev(d["beta"][0, 0, t:t + 1]).reshape(1, 1),
                                      g(d["lam"], L))
        outs.append(o.reshape(16))
    got = torch.stack(outs).cpu().numpy()
    LL.loglin_state_free(st)
    want = _oracle_a(d)[0, 0]
    err = slice_rel_err(got, want, 0)
    assert err <= TOL_F32, err


def test_gdn_decode_agrees_with_chunked_forward():
    """The two GPU paths of the same mixer: decode from empty vs chunked forward."""
    banner("gdn decode vs chunked forward")
    cfg = _cfg(400, 64, 64, "bf16", B=1, H=4)
    d = I.make_gdn(cfg, "weak", seed=5)
    fwd = _run(d)
    st = LL.loglin_state_init(1, 4, 64, 64, cfg.L)
    tr = lambda x: to_dev(np.ascontiguousarray(x[0].swapaxes(0, 1)), torch.bfloat16)  # noqa: E731
    q, k, v = tr(d["q"]), tr(d["k"]), tr(d["v"])
    a, beta = to_dev(d["a"][0].T.copy()), to_dev(d["beta"][0].T.copy())
    lam = to_dev(np.ascontiguousarray(d["lam"][0].swapaxes(0, 1)))
    outs = [LL.loglin_gdn_decode_step(st, q[t][None], k[t][None], v[t][None], a[t][None],
                                      beta[t][None], lam[t][None]) for t in range(cfg.T)]
    dec = torch.stack(outs).cpu().numpy()[:, 0].transpose(1, 0, 2)[None]
    LL.loglin_state_free(st)
    want = ref.gdn_form_b(d["q"], d["k"], d["v"], d["a"], d["beta"], d["lam"])
    assert slice_rel_err(dec, want, 2) <= TOL_BF16
    assert slice_rel_err(fwd, want, 2) <= TOL_BF16


def test_gdn_decode_workload_full_size():
    """128 sequences x 32 heads, 17 levels of 128 x 128, 256 steps on the GPU;
    the oracle follows 16 sampled (sequence, head) pairs through every step."""
    cfg = I.CONFIGS["gdn_decode"]
    banner("gdn decode full size")
    d = I.make_decode(cfg, "base", live_slots=ref.live_slots)
    out, pos, lv = _gdn_decode_gpu(d, d["states"], cfg.steps)
    rng = np.random.default_rng(6)
    pairs = sorted({(int(s), int(h)) for s, h in zip(rng.integers(0, cfg.nseq, 16),
                                                     rng.integers(0, cfg.H, 16))})
    o_ref, st_ref, _ = _gdn_decode_oracle(d, d["states"], pairs, cfg.steps)
    got = np.stack([out[:, s, h] for s, h in pairs], axis=0)
    err_o = slice_rel_err(got, o_ref.transpose(1, 0, 2), 1)
    err_s = state_rel_err(np.stack([lv[s, h] for s, h in pairs]), st_ref)
    print(f"  gdn decode: out err {err_o:.3e} state err {err_s:.3e}", flush=True)
    assert err_o <= TOL_BF16 and err_s <= TOL_BF16
    assert np.array_equal(pos, d["pos"] + cfg.steps)
