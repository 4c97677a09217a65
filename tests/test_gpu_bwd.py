"""GPU parity of the backward pass against the fp64 oracle's gradients.

Page: "Log-linear attention, and what a logarithm buys", section 3 (the mixer
is trained through the same chunked form, forward and backward) and section 6
(the lambda gradients are derived by hand).  Every gradient -- dq, dk, dv,
the decay gradient and dlambda -- is compared element by element with
oracle.reference.form_a_grads on the same seeded inputs, over single chunks,
ragged tails, every chunk size and head-dim mix, and several coarse levels.
"""
import numpy as np
import pytest
import torch

from log_linear_token_amd import loglin as LL
from oracle import reference as ref
from tests.helpers import TOL_BF16, TOL_F32, banner, slice_rel_err, to_dev

pytestmark = pytest.mark.gpu

NAMES = ["dq", "dk", "dv", "dlog_decay", "dlam"]


def _inputs(B, H, T, dk, dv, L, seed, mu=-1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, T, dk)) / np.sqrt(dk)
    k = rng.standard_normal((B, H, T, dk)) / np.sqrt(dk)
    v = rng.standard_normal((B, H, T, dv))
    g = rng.standard_normal((B, H, T, dv))
    a = (-np.logaddexp(0, rng.normal(mu, 0.5, (B, H, T)))).astype(np.float32).astype(np.float64)
    lam = rng.random((B, H, T, L)).astype(np.float32).astype(np.float64)
    return q, k, v, a, lam, g


def _round(x, dtype):
    return to_dev(x, dtype).float().cpu().numpy().astype(np.float64)


def _check(B, H, T, dk, dv, C, dtype, L=None, seed=0, mu=-1.0):
    L = L or max(1, (T - 1).bit_length() + 1)
    q, k, v, a, lam, g = _inputs(B, H, T, dk, dv, L, seed, mu)
    dev = [to_dev(x, dtype) for x in (q, k, v)]
    got = LL.loglin_bwd_chunked(*dev, to_dev(a), to_dev(lam), to_dev(g, dtype), C)
    got = [x.cpu().numpy() for x in got]
    want = ref.form_a_grads(*(_round(x, dtype) for x in (q, k, v)), a, lam, _round(g, dtype))
    tol = TOL_F32 if dtype == torch.float32 else TOL_BF16
    errs = {}
    for n, x, y in zip(NAMES, got, want):
        errs[n] = slice_rel_err(x, y, 2)
    print("  " + " ".join(f"{n} {e:.2e}" for n, e in errs.items()), flush=True)
    for n, e in errs.items():
        assert e <= tol, (n, e)
    return got


CASES = [
    # B, H, T, dk, dv, C, dtype: one token, one ragged chunk, exact chunks,
    # many coarse levels, every chunk size, mixed head dims
    (1, 2, 1, 16, 16, 16, torch.float32),
    (1, 2, 37, 16, 32, 16, torch.float32),
    (1, 1, 64, 32, 16, 16, torch.float32),
    (2, 1, 200, 64, 64, 32, torch.float32),
    (1, 2, 300, 32, 64, 64, torch.float32),
    (1, 1, 513, 128, 128, 128, torch.float32),
    (1, 2, 1, 64, 64, 64, torch.bfloat16),
    (1, 2, 40, 128, 64, 64, torch.bfloat16),
    (1, 2, 130, 16, 16, 16, torch.bfloat16),
    (2, 2, 1000, 64, 64, 64, torch.bfloat16),
    (1, 2, 777, 128, 64, 64, torch.bfloat16),
    (1, 1, 1100, 64, 128, 32, torch.bfloat16),
    (1, 1, 2048, 128, 128, 128, torch.bfloat16),
    # the node scan in two levels (bf16, a multiple of 16 chunks, at least
    # 32): two groups with a ragged last chunk, three groups, 16-token chunks
    (1, 2, 2047, 64, 64, 64, torch.bfloat16),
    (1, 1, 3072, 128, 64, 64, torch.bfloat16),
    (1, 1, 1024, 32, 32, 16, torch.bfloat16),
]


@pytest.mark.parametrize("B,H,T,dk,dv,C,dtype", CASES)
def test_bwd_vs_oracle(B, H, T, dk, dv, C, dtype):
    banner(f"bwd B={B} H={H} T={T} dk={dk} dv={dv} C={C} {dtype}")
    _check(B, H, T, dk, dv, C, dtype, seed=T + dk + C)


def test_bwd_extra_levels_get_zero():
    """lambda with more levels than the sequence uses: those get no gradient."""
    banner("bwd extra levels")
    got = _check(1, 1, 100, 16, 16, 16, torch.float32, L=12, seed=5)
    assert not np.any(got[4][..., 8:])


def test_bwd_long_memory_head_shape():
    """The long-memory decay and head shape of the 8K-token workload, one head."""
    banner("bwd T=4096 dk=128 dv=64 C=64 bf16 long memory")
    _check(1, 1, 4096, 128, 64, 64, torch.bfloat16, seed=9, mu=-2.0)


def test_bwd_empty_is_noop():
    banner("bwd T=0")
    z = torch.empty((1, 1, 0, 16), device="cuda")
    out = LL.loglin_bwd_chunked(z, z, z, torch.empty((1, 1, 0), device="cuda"),
                                torch.empty((1, 1, 0, 4), device="cuda"), z, 16)
    assert all(x.numel() == 0 for x in out)


@pytest.mark.parametrize("dq_blocks", ["one", "two"])
def test_bwd_full_8k_workload_weak_decay(monkeypatch, dq_blocks):
    """The 8K-token workload at full size (B=4, H=16, T=8192, d_k=128, d_v=64,
    C=64, L=15), launched as the benchmark launches it, with the weak decay
    (a = -softplus(N(-8, 0.5))) so that every coarse level carries weight:
    the last (batch, head) slice against the oracle's gradients in full.  The
    dq pass runs as one block of 128 columns (the benchmark's launch) and, with
    LOGLIN_BWD_DQ=fused64, as two 64-column blocks."""
    from log_linear_token_amd import inputs as I

    if dq_blocks == "two":
        monkeypatch.setenv("LOGLIN_BWD_DQ", "fused64")
    else:
        monkeypatch.delenv("LOGLIN_BWD_DQ", raising=False)
    cfg = I.CONFIGS["fwd8k"]
    banner(f"bwd full fwd8k weak dq blocks={dq_blocks} B={cfg.B} H={cfg.H} T={cfg.T} dk={cfg.dk} dv={cfg.dv} C={cfg.C}")
    d = I.make_fwd(cfg, "weak")
    g = np.random.default_rng(cfg.seed + 5).standard_normal((cfg.B, cfg.H, cfg.T, cfg.dv)).astype(np.float32)
    dt = torch.bfloat16
    gd = to_dev(g, dt)
    got = LL.loglin_bwd_chunked(to_dev(d["q"], dt), to_dev(d["k"], dt), to_dev(d["v"], dt),
                                to_dev(d["a"]), to_dev(d["lam"]), gd, cfg.C)
    torch.cuda.synchronize()
    b, h = cfg.B - 1, cfg.H - 1
    got = [x[b, h].cpu().numpy() for x in got]
    g_r = gd[b, h].float().cpu().numpy().astype(np.float64)
    want = ref.form_a_grads(d["q"][b, h], d["k"][b, h], d["v"][b, h], d["a"][b, h], d["lam"][b, h], g_r)
    errs = {n: slice_rel_err(x[None], y[None], 1) for n, x, y in zip(NAMES, got, want)}
    print("  " + " ".join(f"{n} {e:.2e}" for n, e in errs.items()), flush=True)
    for n, e in errs.items():
        assert e <= TOL_BF16, (n, e)


def test_bwd_deterministic():
    """Two backward passes over the same inputs give bit-identical gradients."""
    banner("determinism bwd T=2047")
    B, H, T, dk, dv, C = 1, 2, 2047, 64, 64, 64
    L = (T - 1).bit_length() + 1
    q, k, v, a, lam, g = _inputs(B, H, T, dk, dv, L, seed=9)
    dev = [to_dev(x, torch.bfloat16) for x in (q, k, v)]
    args = (*dev, to_dev(a), to_dev(lam), to_dev(g, torch.bfloat16), C)
    r1 = [x.cpu().numpy() for x in LL.loglin_bwd_chunked(*args)]
    r2 = [x.cpu().numpy() for x in LL.loglin_bwd_chunked(*args)]
    for n, x, y in zip(NAMES, r1, r2):
        assert np.array_equal(x, y), n


@pytest.mark.parametrize("mode", ["walk", "blocks"])
@pytest.mark.parametrize("B,H,T,dk,dv", [(1, 2, 2047, 64, 64), (1, 1, 3072, 128, 64),
                                         (2, 2, 1000, 64, 64), (1, 1, 4100, 128, 64),
                                         (1, 1, 10000, 64, 64)])
def test_bwd_rstate_paths(monkeypatch, mode, B, H, T, dk, dv):
    """The block states R(j) of the dk / dv stage built by one walk over the
    query chunks (segments, parts of the blocks that span segments, a ragged
    last chunk) and by one block per R(j): both give the oracle's gradients."""
    if mode == "blocks":
        monkeypatch.setenv("LOGLIN_BWD_RSTATE", "blocks")
    else:
        monkeypatch.delenv("LOGLIN_BWD_RSTATE", raising=False)
    banner(f"bwd R(j) {mode} B={B} H={H} T={T} dk={dk} dv={dv}")
    _check(B, H, T, dk, dv, 64, torch.bfloat16, seed=T, mu=-3.0)


@pytest.mark.parametrize("mode", ["fused", "chunked"])
@pytest.mark.parametrize("B,H,T,dk,C", [(1, 2, 1, 128, 64), (1, 2, 40, 64, 64), (2, 1, 777, 128, 64), (1, 1, 700, 64, 16),
                                        (1, 1, 3000, 128, 32), (1, 2, 2048, 64, 128),
                                        (1, 1, 5000, 128, 64)])
def test_bwd_dq_paths(monkeypatch, mode, B, H, T, dk, C):
    """dq and dlambda from the fused pass over (dO, v, k) (which also gives
    q . dq for the decay gradient) and from the chunk-state path: both give
    the oracle's gradients (d_v = 64, one token, a partial tile, ragged
    tails, every chunk size the other stages use)."""
    if mode == "chunked":
        monkeypatch.setenv("LOGLIN_BWD_DQ", "chunked")
    else:
        monkeypatch.delenv("LOGLIN_BWD_DQ", raising=False)
    banner(f"bwd dq {mode} B={B} H={H} T={T} dk={dk} C={C}")
    _check(B, H, T, dk, 64, C, torch.bfloat16, seed=T + dk, mu=-3.0)


@pytest.mark.parametrize("mode", ["walk", "chunks"])
@pytest.mark.parametrize("B,H,T,mu", [(1, 1, 100, -1.0), (2, 1, 777, -3.0), (1, 2, 2112, -8.0),
                                      (1, 1, 3072, -3.0), (1, 1, 4100, -1.0), (1, 1, 8192, -8.0)])
def test_bwd_dkv_paths(monkeypatch, mode, B, H, T, mu):
    """dk and dv by the reverse walk over each segment's chunks (block states
    of the levels inside a segment built in registers, the blocks of every
    clear bit combined before the products, the levels spanning segments
    from the R(j) walk) and by one block per chunk: both give the oracle's
    gradients, over two chunks, ragged tails, odd chunk counts and many
    coarse levels, under weak decay too (the full 8K workload test runs
    whole 32-chunk segments)."""
    if mode == "chunks":
        monkeypatch.setenv("LOGLIN_BWD_DKV", "chunks")
    else:
        monkeypatch.delenv("LOGLIN_BWD_DKV", raising=False)
    banner(f"bwd dk/dv {mode} B={B} H={H} T={T} mu={mu}")
    _check(B, H, T, 128, 64, 64, torch.bfloat16, seed=T + 1, mu=mu)


def test_bwd_one_block_dq_ragged_rows():
    """The one-block dq pass (64 (batch, head) pairs, so that its plan takes
    segments of 16 tiles) on a ragged sequence: T = 4095 leaves 63 tokens in
    the last tile, and L = 15 levels against the 13 the sequence uses makes
    T L odd (the dlambda rows go out with 4-byte stores from unaligned
    starts) and leaves two levels whose gradient must be exactly zero.  The
    first and the last (batch, head) slices against the oracle."""
    B, H, T, dk, dv, C, L = 4, 16, 4095, 128, 64, 64, 15
    banner(f"bwd one-block dq ragged B={B} H={H} T={T} L={L}")
    q, k, v, a, lam, g = _inputs(B, H, T, dk, dv, L, seed=43, mu=-3.0)
    dt = torch.bfloat16
    got = LL.loglin_bwd_chunked(to_dev(q, dt), to_dev(k, dt), to_dev(v, dt), to_dev(a), to_dev(lam),
                                to_dev(g, dt), C)
    torch.cuda.synchronize()
    lu = (T - 1).bit_length() + 1
    assert not got[4][..., lu:].any().item()
    for b, h in ((0, 0), (B - 1, H - 1)):
        sl = lambda x: x[b, h][None, None]
        want = ref.form_a_grads(*(_round(sl(x), dt) for x in (q, k, v)), sl(a), sl(lam), _round(sl(g), dt))
        errs = {n: slice_rel_err(x[b, h][None, None].cpu().numpy(), y, 2) for n, x, y in zip(NAMES, got, want)}
        print("  " + " ".join(f"{n} {e:.2e}" for n, e in errs.items()), flush=True)
        for n, e in errs.items():
            assert e <= TOL_BF16, (n, b, h, e)


def test_bwd_unaligned_gradient_outputs():
    """dlambda and dlog_decay may start anywhere on 4 bytes: the one-block dq
    pass (64 (batch, head) pairs, T = 4096, T L a multiple of 4) then writes
    the dlambda rows with 4-byte stores.  The gradients are bitwise those of
    a call with 16-byte aligned outputs."""
    B, H, T, dk, dv, C = 4, 16, 4096, 128, 64, 64
    L = (T - 1).bit_length() + 1
    banner(f"bwd unaligned dlambda B={B} H={H} T={T} L={L}")
    q, k, v, a, lam, g = _inputs(B, H, T, dk, dv, L, seed=47, mu=-3.0)
    dt = torch.bfloat16
    args = (to_dev(q, dt), to_dev(k, dt), to_dev(v, dt), to_dev(a), to_dev(lam), to_dev(g, dt), C)
    want = LL.loglin_bwd_chunked(*args)
    dev = want[0].device
    shapes = [x.shape for x in want]
    grads = [torch.full(sh, float("nan"), dtype=torch.float32, device=dev) for sh in shapes[:3]]
    for sh in shapes[3:]:
        n = int(np.prod(sh))
        buf = torch.full((n + 1,), float("nan"), dtype=torch.float32, device=dev)
        grads.append(buf[1:].view(sh))
    assert grads[4].data_ptr() % 16 == 4 and grads[3].data_ptr() % 16 == 4
    got = LL.loglin_bwd_chunked(*args, grads=tuple(grads))
    torch.cuda.synchronize()
    for n, x, y in zip(NAMES, got, want):
        assert torch.equal(x, y), n


def test_bwd_many_heads_coarse_walk():
    """64 (batch, head) pairs of 4096 tokens (B=4, H=16, d_k=128, d_v=64,
    C=64, weak decay): the dk / dv walk runs 16-chunk segments and the R(j)
    walk builds only the two levels spanning them, in 8-chunk segments of
    its own (two blocks per compute unit), whose parts the dk / dv walk sums.
    The first and the last (batch, head) slices against the oracle."""
    B, H, T, dk, dv, C = 4, 16, 4096, 128, 64, 64
    L = (T - 1).bit_length() + 1
    banner(f"bwd coarse walk B={B} H={H} T={T}")
    q, k, v, a, lam, g = _inputs(B, H, T, dk, dv, L, seed=41, mu=-8.0)
    dt = torch.bfloat16
    got = LL.loglin_bwd_chunked(to_dev(q, dt), to_dev(k, dt), to_dev(v, dt), to_dev(a), to_dev(lam),
                                to_dev(g, dt), C)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (B - 1, H - 1)):
        sl = lambda x: x[b, h][None, None]
        want = ref.form_a_grads(*(_round(sl(x), dt) for x in (q, k, v)), sl(a), sl(lam), _round(sl(g), dt))
        errs = {n: slice_rel_err(x[b, h][None, None].cpu().numpy(), y, 2) for n, x, y in zip(NAMES, got, want)}
        print("  " + " ".join(f"{n} {e:.2e}" for n, e in errs.items()), flush=True)
        for n, e in errs.items():
            assert e <= TOL_BF16, (n, b, h, e)
