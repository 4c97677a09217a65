"""The allocation-free forward (loglin_fwd_chunked_noalloc) against the
forward that takes a workspace argument: the same kernels on the same
inputs, so the outputs must agree bit for bit, on two calls in a row (the
second on a smaller input, so it runs on what the first left in the shared
scratch array), and sizes beyond the array are rejected without a launch."""
import numpy as np
import pytest
import torch

from log_linear_token_amd import inputs as I
from log_linear_token_amd import loglin as LL
from tests.helpers import banner, to_dev

pytestmark = pytest.mark.gpu


def _dev_inputs(cfg, variant, seed):
    d = I.make_fwd(cfg, variant, seed=seed)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    return (to_dev(d["q"], dt), to_dev(d["k"], dt), to_dev(d["v"], dt), to_dev(d["a"]),
            to_dev(d["lam"]))


CALLS = [
    # (name of the workload whose distributions are drawn, overrides): the
    # first call needs the larger workspace, the second a smaller one
    ("fwd8k", dict(B=2, H=8)),
    ("fwd2k", dict(B=1, H=4, T=1000)),
]


@pytest.mark.parametrize("order", ["large_then_small", "fp32_then_bf16"])
def test_noalloc_matches_workspace_forward(order):
    banner(f"no-alloc forward {order}")
    if order == "large_then_small":
        cases = [I.CONFIGS[n].scaled(**kw) for n, kw in CALLS]
    else:
        cases = [I.CONFIGS["tiny"].scaled(B=2, H=3, T=3000, dk=32, dv=32, C=32, L=13),
                 I.CONFIGS["fwd2k"].scaled(B=1, H=2, T=700, L=11)]
    for i, cfg in enumerate(cases):
        need = LL.loglin_fwd_workspace_bytes(cfg.B, cfg.H, cfg.T, cfg.dk, cfg.dv, cfg.C,
                                             torch.bfloat16 if cfg.dtype == "bf16"
                                             else torch.float32)
        assert 0 < need <= LL.NOALLOC_SCRATCH_BYTES
        q, k, v, a, lam = _dev_inputs(cfg, "weak", seed=100 + i)
        want = LL.loglin_fwd_chunked(q, k, v, a, lam, cfg.C)
        out = torch.full_like(want, float("nan"))
        got = LL.loglin_fwd_chunked_noalloc(q, k, v, a, lam, cfg.C, out=out)
        torch.cuda.synchronize()
        assert got.data_ptr() == out.data_ptr()
        assert torch.equal(got, want), (i, float((got - want).abs().max()))
        assert bool(torch.isfinite(got).all())


def test_noalloc_rejects_sizes_beyond_the_array():
    banner("no-alloc forward: oversized request")
    # fp32 inputs take the chunked path, whose workspace here is 256 MiB
    B, H, T, dk, dv, C, L = 4, 16, 8192, 128, 64, 64, 15
    assert LL.loglin_fwd_workspace_bytes(B, H, T, dk, dv, C, torch.float32) > \
        LL.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, H, T, dk), device="cuda")
    v = torch.zeros((B, H, T, dv), device="cuda")
    a = torch.zeros((B, H, T), device="cuda")
    lam = torch.zeros((B, H, T, L), device="cuda")
    out = torch.full((B, H, T, dv), 3.0, device="cuda")
    with pytest.raises(LL.LoglinError) as ei:
        LL.loglin_fwd_chunked_noalloc(q, q, v, a, lam, C, out=out)
    assert ei.value.status == LL.LOGLIN_EUNSUPPORTED
    assert "workspace" in str(ei.value)
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())  # nothing ran


def test_noalloc_rejects_what_the_forward_rejects():
    banner("no-alloc forward: invalid sizes")
    q = torch.zeros((1, 1, 64, 16), device="cuda")
    a = torch.zeros((1, 1, 64), device="cuda")
    lam = torch.zeros((1, 1, 64, 8), device="cuda")
    with pytest.raises(LL.LoglinError) as ei:
        LL.loglin_fwd_chunked_noalloc(q, q, q, a, lam, 48)  # chunk size not supported
    assert ei.value.status == LL.LOGLIN_EUNSUPPORTED
    with pytest.raises(LL.LoglinError) as ei:
        LL.loglin_fwd_chunked_noalloc(q, q, q, a, lam[..., :3].contiguous(), 16)  # too few levels
    assert ei.value.status == LL.LOGLIN_EINVAL


def test_noalloc_forward_replayed_from_a_graph():
    """The allocation-free forward captured once in a HIP graph
    (torch.cuda.CUDAGraph) and replayed four times, with an eager forward of
    other inputs (which reuses the shared scratch array) and host
    synchronisations between the replays: every replay writes the eager
    output bit for bit into the captured output tensor."""
    banner("no-alloc forward replayed from a graph")
    cfg = I.CONFIGS["fwd8k"].scaled(B=2, H=4)
    q, k, v, a, lam = _dev_inputs(cfg, "weak", seed=21)
    ocfg = I.CONFIGS["fwd2k"].scaled(B=1, H=4, T=1000)
    other = _dev_inputs(ocfg, "base", seed=22)
    want = LL.loglin_fwd_chunked_noalloc(q, k, v, a, lam, cfg.C)  # also the scratch's set-up
    other_want = LL.loglin_fwd_chunked_noalloc(*other, ocfg.C)
    torch.cuda.synchronize()
    out = torch.full_like(want, float("nan"))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        LL.loglin_fwd_chunked_noalloc(q, k, v, a, lam, cfg.C, out=out)
    torch.cuda.synchronize()
    for r in range(4):
        out.fill_(float("nan"))
        got_other = LL.loglin_fwd_chunked_noalloc(*other, ocfg.C)
        torch.cuda.synchronize()
        assert torch.equal(got_other, other_want), r
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want), (r, float((out - want).abs().nan_to_num(1e30).max()))
