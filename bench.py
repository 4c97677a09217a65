#!/usr/bin/env python3
"""Benchmark of the log-linear (Fenwick) token mixer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

A step is one chunked forward over the fwd8k batch (B=4, H=16, T=8192,
dk=128, dv=64, bf16 inputs, C=64, L=15) with inputs already resident in HBM;
`value` is forward tokens/s (B*T tokens per step).  In the same run the
Fenwick decode step is timed on the decode workload (128 sequences x 32
heads, 17 levels of 128 x 128 fp32 states, 256 steps) and reported under
"decode".  Each kernel is also timed alone with HIP events on the stream it
is launched on; "roofline" is the one with the largest share of the step.
The fp64 CPU oracle is timed on a bounded sample of the same workload
("cpu_baseline").  Prints exactly one JSON line on stdout; progress goes to
stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from log_linear_token_amd import inputs as I  # noqa: E402
from log_linear_token_amd import loglin as LL  # noqa: E402

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0    # dense bf16 MFMA, TFLOP/s


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "all_workloads_hbm_traffic.txt")


def sources_hash(files: str) -> str:
    """sha256[:16] of the concatenated contents of comma-separated source files."""
    h = hashlib.sha256()
    for f in files.split(","):
        with open(os.path.join(ROOT, f), "rb") as src:
            h.update(src.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary, or
    None when there is none or the kernel's sources have changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            for ln in f:
                parts = ln.split()
                if len(parts) == 5 and parts[0] == "traffic" and parts[1] == kernel:
                    if sources_hash(parts[3]) != parts[4]:
                        return None
                    return float(parts[2])
    except OSError:
        return None
    return None


NSETS = 3  # input/output copies the timed steps rotate through


def rotating_forward(cfg, q, k, v, a, lam, ws):
    """A forward over NSETS copies of the inputs and outputs, the next copy
    on every call: each step reads inputs that the previous steps did not
    touch, so none of them is served from the 256 MB last-level cache (every
    copy of the 8K workload's inputs is 335 MB)."""
    sets = [(q, k, v, a, lam, torch.empty((cfg.B, cfg.H, cfg.T, cfg.dv), device="cuda"))]
    for _ in range(NSETS - 1):
        sets.append(tuple(x.clone() for x in (q, k, v, a, lam)) +
                    (torch.empty((cfg.B, cfg.H, cfg.T, cfg.dv), device="cuda"),))
    state = {"i": 0}

    def fwd(mask=LL.STAGE_ALL):
        qq, kk, vv, aa, ll, oo = sets[state["i"] % NSETS]
        state["i"] += 1
        LL.loglin_fwd_chunked_stages(qq, kk, vv, aa, ll, cfg.C, mask, out=oo, workspace=ws)

    return fwd, sets


SETTLE_MS = 40.0  # untimed run of a workload before its warm-up steps (clock settling)


def settle(fn) -> int:
    """Run fn() back to back until SETTLE_MS of wall time has passed (the
    GPU kept busy, synchronising every 16 calls); returns the calls made."""
    n = 0
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < SETTLE_MS:
        for _ in range(16):
            fn()
        n += 16
        torch.cuda.synchronize()
    return n


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def timed(fn, reps: int, stream) -> float:
    """Average milliseconds of fn() over reps launches, HIP events on `stream`."""
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(reps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / reps


# --------------------------------------------------------------------- byte and flop models

def _causal_blocks(c: int) -> int:
    """16 x 16 blocks on or below the diagonal of a c x c causal tile."""
    nb = c // 16
    return nb * (nb + 1) // 2


def fwd_models(cfg, plan) -> dict:
    """Algorithmic bytes and flops per launch of each forward kernel.

    Bytes count what each kernel must move at least once: its inputs read
    once, its outputs written once, and every distinct carried state it reads
    or writes once (fp32 d_k x d_v).  Flops count the MFMA work of the causal
    16 x 16 blocks of each intra tile, the tile (or chunk) states, and one
    d_k x d_v product per row per coarse level read.  bf16 inputs.
    """
    B, H, T, dk, dv, L = cfg.B, cfg.H, cfg.T, cfg.dk, cfg.dv, cfg.L
    BH = B * H
    lu = (T - 1).bit_length() + 1          # levels the sequence uses
    st = dk * dv * 4
    tok_in = 2 * (2 * dk + dv) + 4 + 4 * lu  # q, k, v bf16 + a + lambda per token-head
    tok_out = 4 * dv
    tile = plan["tile"]
    ntiles = -(-T // tile)
    nseg = plan["nseg"]
    intra = _causal_blocks(tile) * 2 * 16 * 16 * (dk + dv)
    if plan["path"] == "fused":
        segt = plan["seg_tiles"]
        tiles_pre = min(ntiles, (nseg - 1) * segt)   # tiles before the last segment
        # per segment: tile states folded inside it, local levels read, top levels read
        local_reads = 0
        top_reads = 0
        states = 0
        for s in range(nseg):
            n = min(segt, ntiles - s * segt)
            local_reads += sum(bin(il).count("1") for il in range(n))
            top_reads += n * bin(s).count("1")
            states += n - 1
        nsub = plan["state_split"]
        return {
            "seg_state": {"bytes": BH * tiles_pre * tile * (2 * (dk + dv) + 4)
                          + BH * (nseg - 1) * nsub * (st + 4),
                          "flops": BH * tiles_pre * tile * 2 * dk * dv},
            # reads the sub-range states, writes each node as bf16 fragments
            "fenwick_scan": {"bytes": BH * (nseg - 1) * (nsub * (st + 4) + st // 2 + 8),
                             "flops": 0},
            "fused_fwd": {"bytes": BH * T * (tok_in + tok_out) + BH * (nseg - 1) * (st + 8),
                          "flops": BH * (ntiles * intra + (states + local_reads + top_reads)
                                         * tile * 2 * dk * dv)},
        }
    N = ntiles
    pops = sum(bin(i).count("1") for i in range(N))
    return {
        "chunk_state": {"bytes": BH * T * (2 * (dk + dv) + 4) + BH * N * (st + 4),
                        "flops": BH * N * tile * 2 * dk * dv},
        "fenwick_scan": {"bytes": BH * (N - 1) * (2 * st + 4 + 8), "flops": 0},
        "chunk_output": {"bytes": BH * T * (tok_in + tok_out) + BH * (N - 1) * (st + 8),
                         "flops": BH * (N * intra + pops * tile * 2 * dk * dv)},
    }


def decode_bytes(pos0: np.ndarray, H: int, dk: int, dv: int, Lmax: int, steps: int) -> float:
    """Average algorithmic bytes per decode step (steps counted from a load).

    The step keeps levels 0..6 of position t as the raw k, v rows (fp32, plus
    the running decay sum) of t's 64-token window and levels >= 7 as fp32
    d_k x d_v matrices.  Inside a window (t mod 64 = m > 0) it reads the m
    earlier rows and the live matrix levels (set bits >= 6 of t) and writes
    one row.  At a window boundary (m = 0) it reads the finished window's 64
    rows and the matrix levels 7..j below the merge, writes the merged level
    j+1, and reads the live levels above.  Until the first boundary after a
    load the loaded levels 0..6 are matrices and the step works on matrices
    only: it reads the popcount(t-1) live levels above 0 (and the loaded
    level 0 on the first step) and writes the merged level.  Plus q, k, v
    (bf16), a, lambda, the level scales (read and written), the level-0
    vectors and out."""
    st = dk * dv * 4
    row = (dk + dv) * 4 + 4
    small = (2 * dk + dv) * 2 + 4 + Lmax * 4 + 2 * Lmax * 4 + 2 * (dk + dv) * 4 + dv * 4
    pc = lambda x: bin(x).count("1")  # noqa: E731
    tot = 0.0
    for p0 in (int(x) for x in pos0):
        for s in range(steps):
            t = p0 + s
            if t >= 1 and (t & ~63) >= p0:          # window levels
                m = t & 63
                if m > 0:
                    b = m * row + row + pc(t >> 6) * st
                else:
                    j = (t & -t).bit_length() - 1
                    b = row + st + pc(t >> (j + 1)) * st
                    if t - 64 >= p0:
                        b += 64 * row + (j - 6) * st
                    else:
                        b += pc((t - 1) & ((1 << j) - 1)) * st + (st if s == 0 else 0)
            elif t >= 1:                             # matrix levels after a load
                b = (pc(t - 1) + (1 if s == 0 else 0) + 1) * st
            else:
                b = row
            tot += b
    return (tot * H + len(pos0) * H * small * steps) / steps


# --------------------------------------------------------------------- ceilings and sweeps

def measure_ceilings() -> dict:
    """The HBM rates a plain stream reaches on this GPU, measured in this run:
    a 2 GiB device-to-device copy (read + write bytes) and a row-wise
    reduction over 2 GiB (bytes read, 0.1 % written).  Kernels are reported against the
    8 TB/s spec and against these."""
    n = (2 << 30) // 4
    src = torch.ones(n, device="cuda")
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()
    for _ in range(3):
        dst.copy_(src)
    ms_copy = timed(lambda: dst.copy_(src), 10, stream)
    rows = torch.empty(n // 1024, device="cuda")
    rsum = lambda: torch.sum(src.view(-1, 1024), dim=1, out=rows)  # noqa: E731
    for _ in range(3):
        rsum()
    ms_read = timed(rsum, 10, stream)
    copy = 2 * n * 4 / (ms_copy / 1e3) / 1e9
    read = (n + n // 1024) * 4 / (ms_read / 1e3) / 1e9
    log(f"ceilings: copy {copy:.0f} GB/s (read + write), read-only {read:.0f} GB/s")
    del src, dst
    torch.cuda.empty_cache()
    return {"copy_GB/s": round(copy, 1), "read_GB/s": round(read, 1),
            "spec_GB/s": HBM_PEAK_GBS,
            "method": "torch copy_ of 2 GiB fp32 (bytes read + written) and torch.sum of "
                      "2 GiB fp32 over rows of 1024 (bytes read + the row sums written), 10 "
                      "timed launches each after 3 warm-ups"}


def bench_sweep() -> dict:
    """Scaling checks against the page's complexity claims (its opening:
    O(T log T) training compute; section 3: the inter-chunk stage is
    O(T log(T/C))).  Forward over T = 2K..64K at a fixed 2^18 tokens per
    step (B = 2^18 / T, H = 16, dk = 128, dv = 64, C = 64, the 8K workload's
    distributions); reports ms per step, ns per token-head and that time over
    log2(T/C).  Decode: every sequence of the decode workload at the same
    position t = 2^k - 1 + 64 u (u a few whole windows in), so the number of
    live matrix levels is popcount(t >> 6); ms per step against the modelled
    bytes."""
    out = {"forward": [], "decode": []}
    base = I.CONFIGS["fwd8k"]
    stream = torch.cuda.current_stream()
    for T in (2048, 4096, 8192, 16384, 32768, 65536):
        cfg = base.scaled(B=(1 << 18) // T, T=T, L=(T - 1).bit_length() + 1)
        g = torch.Generator(device="cuda")
        g.manual_seed(cfg.seed + T)
        shp = (cfg.B, cfg.H, T)
        q = (torch.randn(shp + (cfg.dk,), device="cuda", generator=g) / cfg.dk ** 0.5).to(torch.bfloat16)
        k = (torch.randn(shp + (cfg.dk,), device="cuda", generator=g) / cfg.dk ** 0.5).to(torch.bfloat16)
        v = torch.randn(shp + (cfg.dv,), device="cuda", generator=g).to(torch.bfloat16)
        a = -torch.nn.functional.softplus(-2.0 + 0.5 * torch.randn(shp, device="cuda", generator=g))
        lam = torch.nn.functional.softplus(torch.randn(shp + (cfg.L,), device="cuda", generator=g))
        ws = torch.empty(max(1, LL.loglin_fwd_workspace_bytes(cfg.B, cfg.H, T, cfg.dk, cfg.dv, cfg.C,
                                                              torch.bfloat16)),
                         dtype=torch.uint8, device="cuda")
        o = torch.empty(shp + (cfg.dv,), device="cuda")
        run = lambda: LL.loglin_fwd_chunked(q, k, v, a, lam, cfg.C, out=o, workspace=ws)  # noqa
        for _ in range(20):
            run()
        ms = timed(run, 30, stream)
        ns_th = ms * 1e6 / (cfg.B * cfg.H * T)
        out["forward"].append({"T": T, "B": cfg.B, "ms": round(ms, 4),
                               "ns_per_token_head": round(ns_th, 4),
                               "ns_per_token_head_per_log2_T_over_C": round(ns_th / np.log2(T / cfg.C), 4)})
        log(f"sweep T={T}: {ms:.3f} ms, {ns_th:.3f} ns per token-head")
        del q, k, v, a, lam, ws, o
    torch.cuda.empty_cache()
    dc = I.CONFIGS["decode"]
    nseq, H, dk, dv, Lmax = dc.nseq, dc.H, dc.dk, dc.dv, dc.Lmax
    st = LL.loglin_state_init(nseq, H, dk, dv, Lmax)
    g = torch.Generator(device="cuda")
    g.manual_seed(dc.seed)
    levels = torch.randn((nseq, H, Lmax, dk, dv), device="cuda", generator=g) / dk ** 0.5
    qd = torch.randn((nseq, H, dk), device="cuda", generator=g).to(torch.bfloat16)
    ad = -torch.nn.functional.softplus(torch.randn((nseq, H), device="cuda", generator=g))
    ld = torch.rand((nseq, H, Lmax), device="cuda", generator=g)
    od = torch.empty((nseq, H, dv), device="cuda")
    for kbits in (7, 9, 11, 13, 15):
        # position (2^kbits - 1) rounded down to a window start, then 2 windows
        # of steps: the timed steps run inside windows, with popcount(t >> 6)
        # matrix levels live
        p0 = ((1 << kbits) - 1) & ~63
        LL.loglin_state_load(st, np.full(nseq, p0, np.int64), levels)
        steps = 128
        it = iter(range(steps))
        stp = lambda: (next(it), LL.loglin_decode_step(st, qd, qd, qd, ad, ld, out=od))  # noqa
        ms = timed(stp, steps, stream)
        pcs = [bin((p0 + s) >> 6).count("1") for s in range(steps)]
        byts = decode_bytes(np.full(nseq, p0, np.int64), H, dk, dv, Lmax, steps)
        out["decode"].append({"start_position": p0, "mean_live_matrix_levels": round(float(np.mean(pcs)), 3),
                              "ms_per_step": round(ms, 4), "model_GB_per_step": round(byts / 1e9, 4),
                              "GB/s": round(byts / (ms / 1e3) / 1e9, 1)})
        log(f"sweep decode from {p0}: {ms:.3f} ms/step, {np.mean(pcs):.2f} matrix levels")
    LL.loglin_state_free(st)
    del levels
    torch.cuda.empty_cache()
    return out


# --------------------------------------------------------------------- CPU baseline

def cpu_baseline(cfg, d) -> dict:
    """The fp64 oracle recurrence on a bounded sample of the same workload."""
    from oracle import reference as ref
    threads = ref.default_threads()
    nslices = cfg.B * cfg.H  # every slice: about 10-30 s of CPU work on 16 cores
    idx = [(s // cfg.H, s % cfg.H) for s in range(nslices)]
    pick = lambda x: np.stack([x[b, h] for b, h in idx])  # noqa: E731
    q, k, v, a, lam = (pick(d[n]) for n in ("q", "k", "v", "a", "lam"))
    log(f"cpu baseline: oracle recurrence on {nslices} of {cfg.B * cfg.H} (batch, head) slices, "
        f"{threads} threads")
    t0 = time.perf_counter()
    ref.form_b(q, k, v, a, lam, nthreads=threads)
    dt = time.perf_counter() - t0
    # a token of the workload is one position of one sequence across all H heads
    toks = nslices * cfg.T / cfg.H
    # one core, on two slices
    n1 = 2
    t0 = time.perf_counter()
    ref.form_b(q[:n1], k[:n1], v[:n1], a[:n1], lam[:n1], nthreads=1)
    dt1 = time.perf_counter() - t0
    return {"value": toks / dt, "unit": "tokens/s", "cores": min(threads, nslices),
            "kind": "oracle",
            "sample": f"fp64 Fenwick recurrence over {nslices} of the {cfg.B * cfg.H} "
                      f"(batch, head) slices of fwd8k, all {cfg.T} positions each "
                      f"({dt:.1f} s wall); tokens counted as slices*T/H",
            "value_1core": n1 * cfg.T / cfg.H / dt1,
            "sample_1core": f"the same recurrence on {n1} slices with one thread ({dt1:.1f} s wall)",
            "cpu_model": _cpu_model()}


def cpu_baseline_other() -> dict:
    """The oracle on bounded samples of the other workloads, scaled to each
    workload's own unit: the 2K forward (all 16 slices, ten times), the 64K
    forward (the first 8192 positions of eight slices: the recurrence's cost
    per token grows only with the live levels, so this overstates its 64K
    rate slightly), and decode (512 of the 4096 (sequence, head) pairs for
    64 steps, scaled to steps of the whole batch)."""
    from oracle import reference as ref
    threads = ref.default_threads()
    res = {}
    c2 = I.CONFIGS["fwd2k"]
    d2 = I.make_fwd(c2, "base")
    reps = 10
    t0 = time.perf_counter()
    for _ in range(reps):
        ref.form_b(d2["q"], d2["k"], d2["v"], d2["a"], d2["lam"], nthreads=threads)
    dt = time.perf_counter() - t0
    res["fwd2k"] = {"value": reps * c2.B * c2.T / dt, "unit": "tokens/s",
                    "cores": min(threads, c2.B * c2.H), "kind": "oracle",
                    "sample": f"fp64 recurrence over all {c2.B * c2.H} slices, {reps} times "
                    f"({dt:.1f} s wall)"}
    ns5, T5 = 8, 8192
    c5 = I.CONFIGS["long64k"].scaled(B=1, H=ns5, T=T5, L=(T5 - 1).bit_length() + 1)
    d5 = I.make_fwd(c5, "base")
    t0 = time.perf_counter()
    ref.form_b(d5["q"], d5["k"], d5["v"], d5["a"], d5["lam"], nthreads=threads)
    dt = time.perf_counter() - t0
    H5 = I.CONFIGS["long64k"].H
    res["long64k"] = {"value": ns5 * T5 / H5 / dt, "unit": "tokens/s", "cores": min(threads, ns5),
                      "kind": "oracle", "sample": f"fp64 recurrence over the first {T5} positions "
                      f"of {ns5} of the 16 slices ({dt:.1f} s wall); tokens counted as slices*T/H"}
    dc = I.CONFIGS["decode"].scaled(nseq=128, H=4, steps=64)
    dd = I.make_decode(dc, "base", live_slots=ref.live_slots)
    P = dc.nseq * dc.H
    sel = lambda x: x.reshape((dc.steps, P) + x.shape[3:])  # noqa: E731
    t0 = time.perf_counter()
    ref.decode(dd["states"].reshape(P, dc.Lmax, dc.dk, dc.dv), np.repeat(dd["pos"], dc.H),
               sel(dd["q"]), sel(dd["k"]), sel(dd["v"]), sel(dd["a"]), sel(dd["lam"]),
               nthreads=threads)
    dt = time.perf_counter() - t0
    full = I.CONFIGS["decode"]
    res["decode"] = {"value": dc.steps * P / (full.nseq * full.H) / dt, "unit": "steps/s",
                     "cores": min(threads, P), "kind": "oracle",
                     "sample": f"fp64 recurrence, {P} of the {full.nseq * full.H} (sequence, head) "
                     f"pairs for {dc.steps} steps ({dt:.1f} s wall), scaled to steps of all pairs"}
    log(f"cpu baseline other: {res}")
    return res


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# --------------------------------------------------------------------- main

def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # the GPU needs some tens of milliseconds of work to reach its steady clock:
    # the default warm-up covers that (200 forward steps of the 8K workload
    # take about 35 ms)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--decode-steps", type=int, default=256)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the sequence-length and decode-popcount sweeps")
    ap.add_argument("--no-gdn", action="store_true",
                    help="skip the log-linear Gated DeltaNet forward and decode")
    ap.add_argument("--no-other", action="store_true",
                    help="skip the 2K and 64K forward workloads")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (for scaling HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus})", file=sys.stderr)
        return 2
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2

    if args.copy_calibration:
        n = 1 << 30
        src = torch.ones(n // 4, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}))
        return 0

    cfg = I.CONFIGS["fwd8k"]
    log(f"generating fwd8k inputs (B={cfg.B} H={cfg.H} T={cfg.T} dk={cfg.dk} dv={cfg.dv})")
    d = I.make_fwd(cfg, "base")
    dev = lambda x, dt=torch.float32: torch.from_numpy(x).to("cuda").to(dt).contiguous()  # noqa
    q, k, v = (dev(d[n], torch.bfloat16) for n in ("q", "k", "v"))
    a, lam = dev(d["a"]), dev(d["lam"])
    ws = torch.empty(LL.loglin_fwd_workspace_bytes(cfg.B, cfg.H, cfg.T, cfg.dk, cfg.dv, cfg.C, torch.bfloat16),
                     dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    fwd, sets = rotating_forward(cfg, q, k, v, a, lam, ws)

    # Measured ceilings of this GPU (copy and read-only streams) and the
    # sequence-length sweep run right before the headline timing, with the
    # headline's inputs already resident (no host work in between).
    ceilings = measure_ceilings()
    sweep = None if args.no_sweep else bench_sweep()

    # The GPU reaches its steady clock only after some tens of milliseconds of
    # sustained work, and the host-side input generation above leaves it idle:
    # the headline forward runs untimed for SETTLE_MS first, then the W
    # warm-up steps, then exactly K timed steps.
    settle_steps = settle(fwd)
    for _ in range(args.warmup):
        fwd()
    torch.cuda.synchronize()
    log(f"timing {args.steps} forward steps")
    t0 = time.perf_counter()
    ms = timed(fwd, args.steps, stream)
    wall = time.perf_counter() - t0
    tokens = cfg.B * cfg.T
    value = tokens / (ms / 1e3)
    log(f"forward: {ms:.3f} ms/step ({value:.3e} tokens/s; wall {wall:.2f} s)")

    # per-kernel timing on the same stream.  The state and output kernels are
    # launched alone; the scan is too short to keep the GPU busy between two
    # calls from Python, so it is timed as (state + scan) - state.
    plan = LL.loglin_fwd_plan(cfg.B, cfg.H, cfg.T, cfg.dk, cfg.dv, cfg.C, torch.bfloat16)
    log(f"plan: {plan}")
    models = fwd_models(cfg, plan)
    names = list(models)  # kernel names in launch order
    kernels = {}
    reps = max(5, args.steps)

    def stage_ms(mask):
        fwd(mask)
        return timed(lambda: fwd(mask), reps, stream)

    for name, mask in zip(names, (LL.STAGE_CHUNK_STATE, LL.STAGE_SCAN, LL.STAGE_OUTPUT)):
        if mask == LL.STAGE_SCAN:
            kms = max(stage_ms(LL.STAGE_CHUNK_STATE | LL.STAGE_SCAN) - stage_ms(LL.STAGE_CHUNK_STATE), 1e-6)
        else:
            kms = stage_ms(mask)
        m = models[name]
        kernels[name] = {"ms": kms, "GB/s": m["bytes"] / (kms / 1e3) / 1e9,
                         "TFLOP/s": m["flops"] / (kms / 1e3) / 1e12,
                         "alg_bytes": m["bytes"], "alg_flops": m["flops"]}
        log(f"  {name}: {kms:.3f} ms, {kernels[name]['GB/s']:.0f} GB/s, "
            f"{kernels[name]['TFLOP/s']:.1f} TFLOP/s")
    fwd()  # leave a complete output behind
    dom = max(kernels, key=lambda n: kernels[n]["ms"])
    km = kernels[dom]
    roof = {"kernel": dom, "bound": "hbm", "achieved": round(km["GB/s"], 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(km["GB/s"] / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(dom),
            "frac_of_measured_copy": round(km["GB/s"] / ceilings["copy_GB/s"], 4),
            "frac_of_measured_read": round(km["GB/s"] / ceilings["read_GB/s"], 4),
            "mfma": mfma_entry(km)}

    result = {
        "metric": "fwd tokens/s + MFMA util, log-linear mixer T=8192; decode steps/s",
        "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "settle": {"ms": SETTLE_MS, "untimed_steps": settle_steps,
                   "note": "untimed run of the forward before the warm-up steps (GPU clock settling)"},
        "config": {"workload": "fwd8k", "B": cfg.B, "H": cfg.H, "T": cfg.T, "dk": cfg.dk,
                   "dv": cfg.dv, "C": cfg.C, "L": cfg.L, "parallelism": "none"},
        "roofline": roof,
        "kernels": {n: {kk: (round(vv, 4) if isinstance(vv, float) else vv)
                        for kk, vv in m.items()} for n, m in kernels.items()},
        "plan": plan,
        "ceilings": ceilings,
    }
    if sweep is not None:
        result["sweep"] = sweep
    result["prefill_states"] = bench_prefill(cfg, sets, stream, args.steps)
    if not args.no_backward:
        result["backward"] = bench_backward(cfg, sets, stream, max(5, args.steps // 4))
    del q, k, v, a, lam, ws, sets, fwd
    torch.cuda.empty_cache()

    if not args.no_other:
        result["other_workloads"] = [bench_fwd_other(n, args.steps, args.warmup)
                                     for n in ("fwd2k", "long64k")]
    if not args.no_decode:
        result["decode"] = bench_decode(args.decode_steps)
    if not args.no_gdn:
        result["gated_deltanet"] = {"forward": bench_gdn_fwd(args.steps, args.warmup),
                                    "decode": bench_gdn_decode(args.decode_steps)}
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, d)
        result["cpu_baseline_other"] = cpu_baseline_other()
    print(json.dumps(result), flush=True)
    return 0


def mfma_entry(km: dict) -> dict:
    """MFMA side of a forward kernel: achieved bf16 TFLOP/s against the dense
    peak and against what HBM allows at the kernel's arithmetic intensity."""
    ai = km["alg_flops"] / km["alg_bytes"]
    attainable = min(BF16_PEAK_TFLOPS, ai * HBM_PEAK_GBS / 1e3)
    return {"achieved": round(km["TFLOP/s"], 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(km["TFLOP/s"] / BF16_PEAK_TFLOPS, 4),
            "flop_per_byte": round(ai, 1), "attainable": round(attainable, 1),
            "frac_of_attainable": round(km["TFLOP/s"] / attainable, 4)}


def bench_fwd_other(name: str, steps: int, warmup: int) -> dict:
    """Forward throughput of another workload at 1 GPU: the whole path per
    step, and the output kernel alone against the HBM and MFMA rooflines."""
    cfg = I.CONFIGS[name]
    log(f"{name}: generating inputs (B={cfg.B} H={cfg.H} T={cfg.T} dk={cfg.dk} dv={cfg.dv})")
    d = I.make_fwd(cfg, "base")
    dev = lambda x, dt=torch.float32: torch.from_numpy(x).to("cuda").to(dt).contiguous()  # noqa
    q, k, v = (dev(d[n], torch.bfloat16) for n in ("q", "k", "v"))
    a, lam = dev(d["a"]), dev(d["lam"])
    del d
    ws = torch.empty(max(1, LL.loglin_fwd_workspace_bytes(cfg.B, cfg.H, cfg.T, cfg.dk, cfg.dv, cfg.C,
                                                          torch.bfloat16)),
                     dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    fwd, sets = rotating_forward(cfg, q, k, v, a, lam, ws)

    settle(fwd)
    for _ in range(warmup):
        fwd()
    ms = timed(fwd, steps, stream)
    plan = LL.loglin_fwd_plan(cfg.B, cfg.H, cfg.T, cfg.dk, cfg.dv, cfg.C, torch.bfloat16)
    models = fwd_models(cfg, plan)
    name_out = list(models)[-1]
    fwd(LL.STAGE_OUTPUT)
    kms = timed(lambda: fwd(LL.STAGE_OUTPUT), steps, stream)
    m = models[name_out]
    km = {"ms": kms, "GB/s": m["bytes"] / (kms / 1e3) / 1e9, "TFLOP/s": m["flops"] / (kms / 1e3) / 1e12,
          "alg_bytes": m["bytes"], "alg_flops": m["flops"]}
    tps = cfg.B * cfg.T / (ms / 1e3)
    log(f"{name}: {ms:.3f} ms/step, {tps:.3e} tokens/s; {name_out} {kms:.3f} ms, "
        f"{km['GB/s']:.0f} GB/s")
    del q, k, v, a, lam, ws, sets, fwd
    torch.cuda.empty_cache()
    return {"workload": name, "tokens_per_s": tps, "ms_per_step": ms,
            "config": {"B": cfg.B, "H": cfg.H, "T": cfg.T, "dk": cfg.dk, "dv": cfg.dv, "C": cfg.C,
                       "L": cfg.L},
            "plan": plan,
            "roofline": {"kernel": name_out, "bound": "hbm", "achieved": round(km["GB/s"], 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(km["GB/s"] / HBM_PEAK_GBS, 4),
                         "alg_bytes": m["bytes"], "traffic": measured_traffic(f"{name}_{name_out}"),
                         "mfma": mfma_entry(km)}}


def bench_prefill(cfg, sets, stream, steps: int) -> dict:
    """The prefill -> decode hand-over on the 8K workload: the Fenwick level
    states after all T tokens.  Algorithmic bytes: k, v (bf16) and a read
    once, the live level states written once."""
    B, H, T, dk, dv = cfg.B, cfg.H, cfg.T, cfg.dk, cfg.dv
    Lmax = (T - 1).bit_length() + 1
    out = torch.empty((B, H, Lmax, dk, dv), device="cuda")
    ws = torch.empty(max(1, LL.loglin_prefill_workspace_bytes(B, H, T, dk, dv, Lmax)),
                     dtype=torch.uint8, device="cuda")
    state = {"i": 0}

    def run():
        _, kk, vv, aa, _, _ = sets[state["i"] % len(sets)]
        state["i"] += 1
        LL.loglin_prefill_states(kk, vv, aa, Lmax, out=out, workspace=ws)

    settle(run)
    for _ in range(5):
        run()
    ms = timed(run, max(5, steps // 4), stream)
    live = 1 + bin(T - 1).count("1")
    byts = B * H * (T * (2 * dk + 2 * dv + 4) + live * dk * dv * 4)
    gbs = byts / (ms / 1e3) / 1e9
    log(f"prefill states: {ms:.3f} ms, {gbs:.0f} GB/s")
    return {"ms": ms, "alg_bytes": byts, "GB/s": round(gbs, 1),
            "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}


def bwd_model(cfg) -> dict:
    """Algorithmic bytes and flops of one backward pass.

    Bytes: q, k, v and dO read once (input dtype), a and the lu levels of
    lambda read once, dq, dk, dv, da and the lu levels of dlambda written
    once (fp32); the carried states (the swapped chunk states and their nodes,
    the R states) are not counted: a pass that kept them on chip would not
    move them.  Flops: per chunk the five C x C products of the causal block
    (scores, dP, and the dq, dk, dv contractions), full tiles, plus per chunk
    the swapped chunk state and one state product per coarse level a chunk
    reads (dq) or feeds (dk, dv, R)."""
    B, H, T, dk, dv, C = cfg.B, cfg.H, cfg.T, cfg.dk, cfg.dv, cfg.C
    lu = (T - 1).bit_length() + 1
    per_tok = 2 * (2 * dk + 2 * dv) + 4 + 4 * lu + 4 * (2 * dk + dv) + 4 + 4 * lu
    byts = B * H * T * per_tok
    N = T // C
    coarse = sum(bin(i).count("1") for i in range(N))  # node reads of dq, and R feeds of dk/dv
    intra = N * 2 * C * C * (3 * dk + 2 * dv)  # Q K^T, dO V^T, dq, dk (over dk); dv (over dv)
    states = N * 2 * C * dk * dv * 2 + coarse * 2 * C * dk * dv * 4  # G', R; dq, dk, dv reads
    return {"bytes": byts, "flops": B * H * (intra + states)}


def bench_backward(cfg, sets, stream, steps: int) -> dict:
    """The backward pass on the 8K workload: dq, dk, dv, the decay and lambda
    gradients, rotating through the forward's input copies."""
    B, H, T, dk, dv = cfg.B, cfg.H, cfg.T, cfg.dk, cfg.dv
    ws = torch.empty(LL.loglin_bwd_workspace_bytes(B, H, T, dk, dv, cfg.C, torch.bfloat16),
                     dtype=torch.uint8, device="cuda")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(cfg.seed + 1)
    douts = [torch.randn((B, H, T, dv), device="cuda", generator=gen).to(torch.bfloat16)
             for _ in sets]
    grads = [torch.empty((B, H, T, dk), device="cuda"), torch.empty((B, H, T, dk), device="cuda"),
             torch.empty((B, H, T, dv), device="cuda"), torch.empty((B, H, T), device="cuda"),
             torch.empty((B, H, T, cfg.L), device="cuda")]
    state = {"i": 0}

    def run():
        j = state["i"] % len(sets)
        qq, kk, vv, aa, ll, _ = sets[j]
        state["i"] += 1
        LL.loglin_bwd_chunked(qq, kk, vv, aa, ll, douts[j], cfg.C, grads=grads, workspace=ws)

    settle(run)
    for _ in range(10):
        run()
    ms = timed(run, steps, stream)
    m = bwd_model(cfg)
    gbs = m["bytes"] / (ms / 1e3) / 1e9
    tfl = m["flops"] / (ms / 1e3) / 1e12
    tps = B * T / (ms / 1e3)
    log(f"backward: {ms:.3f} ms, {tps:.3e} tokens/s, {gbs:.0f} GB/s, {tfl:.0f} TFLOP/s")
    del ws, douts, grads
    return {"ms": ms, "tokens_per_s": tps, "alg_bytes": m["bytes"], "alg_flops": m["flops"],
            "GB/s": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
            "TFLOP/s": round(tfl, 1), "frac_mfma": round(tfl / BF16_PEAK_TFLOPS, 4),
            "traffic": measured_traffic("backward")}


def bench_decode(steps: int) -> dict:
    cfg = I.CONFIGS["decode"]
    log(f"decode: {cfg.nseq} sequences x {cfg.H} heads, Lmax={cfg.Lmax}, {steps} steps")
    d = I.make_decode(cfg.scaled(steps=steps), "base", fill=False)
    pos = d["pos"]
    # synthetic pre-filled states drawn on the device: N(0, 1/dk) in every
    # slot (the loader ignores the slots that are not live at a position, so
    # the kernel's work depends only on the positions)
    g = torch.Generator(device="cuda")
    g.manual_seed(cfg.seed)
    levels = torch.randn((cfg.nseq, cfg.H, cfg.Lmax, cfg.dk, cfg.dv), device="cuda",
                         generator=g) * (1.0 / np.sqrt(cfg.dk))
    st = LL.loglin_state_init(cfg.nseq, cfg.H, cfg.dk, cfg.dv, cfg.Lmax)
    q, k, v = (torch.from_numpy(d[n]).to("cuda").to(torch.bfloat16) for n in ("q", "k", "v"))
    a, lam = torch.from_numpy(d["a"]).to("cuda"), torch.from_numpy(d["lam"]).to("cuda")
    out = torch.empty((cfg.nseq, cfg.H, cfg.dv), device="cuda")
    stream = torch.cuda.current_stream()
    # warm-up: the same steps from the same loaded state, repeated for at
    # least SETTLE_MS (clock settling); the state is then loaded again for
    # the timed steps
    t0 = time.perf_counter()
    while True:
        LL.loglin_state_load(st, pos, levels)
        for s in range(min(steps, 64)):
            LL.loglin_decode_step(st, q[s], k[s], v[s], a[s], lam[s], out=out)
        torch.cuda.synchronize()
        if (time.perf_counter() - t0) * 1e3 >= SETTLE_MS:
            break
    LL.loglin_state_load(st, pos, levels)
    del levels
    it = iter(range(steps))

    def step():
        s = next(it)
        LL.loglin_decode_step(st, q[s], k[s], v[s], a[s], lam[s], out=out)

    ms = timed(step, steps, stream)
    LL.loglin_state_free(st)
    sps = 1e3 / ms
    byts = decode_bytes(pos, cfg.H, cfg.dk, cfg.dv, cfg.Lmax, steps)
    gbs = byts / (ms / 1e3) / 1e9
    log(f"decode: {ms:.3f} ms/step, {sps:.1f} steps/s, {gbs:.0f} GB/s")
    return {"steps_per_s": sps, "tokens_per_s": sps * cfg.nseq, "ms_per_step": ms,
            "steps": steps, "config": {"workload": "decode", "nseq": cfg.nseq, "H": cfg.H,
                                       "dk": cfg.dk, "dv": cfg.dv, "Lmax": cfg.Lmax},
            "roofline": {"kernel": "decode_step", "bound": "hbm", "achieved": round(gbs, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic("decode_step"),
                         "alg_bytes_per_step": byts}}


# --------------------------------------------------------------------- Gated DeltaNet



def gdn_models(cfg) -> dict:
    """Algorithmic bytes and flops per launch of the two Gated DeltaNet kernels
    (64-token chunks, bf16 inputs).

    Chunk kernel: reads q, k, v, a, beta and the 7 intra-chunk levels of
    lambda once; writes the chunk's output and, for every chunk but the last
    of a sequence, its read-out queries q' (64 x dk, bf16), transition F
    (dk x dk, two bf16 pieces) and state U (dk x dv, fp32).  Flops: the products of full 16 x 16
    tiles it computes -- Q K^T and K K^T on the 10 lower tiles, the block
    inverse, W, U0, the chunk block Y Tb, P V, q', F and U.
    Level walk: reads q', F, U and the coarse lambda of every chunk once and
    the output once, writes the output once (the level states stay in LDS).
    Flops: per chunk one read-out per live level (64 x dk x dv) and one
    transition per level carried (dk x dk x dv).
    """
    B, H, T, dk, dv, L = cfg.B, cfg.H, cfg.T, cfg.dk, cfg.dv, cfg.L
    BH = B * H
    N = -(-T // 64)
    nst = N - 1                      # chunks whose q', F and U are written
    tile = 16 * 16 * 2
    # a 16 x 16 output tile contracted over K costs tile * K flops; the lower
    # tiles of a 64-token chunk contract over 16 (ti + 1) tokens, 10 * 16 in all
    intra = (2 * 10 * tile * dk          # Q K^T and K K^T, lower tiles
             + 12 * 16 * tile            # the off-diagonal blocks of the inverse
             + 10 * 16 * tile * dk // 16 * 2  # W and q' (W: Tb Kd; q': Y W)
             + 10 * 16 * tile * dv // 16 * 2  # U0 = Tb V and P V
             + 20 * 16 * tile)           # Y Tb on the lower tiles
    states = 64 * 2 * dk * dk + 64 * 2 * dk * dv
    per_chunk = 2 * 64 * dk + 4 * dk * dk + 4 * dk * dv   # q' bf16, F hi + lo, U fp32
    chunk_bytes = BH * T * (2 * (2 * dk + dv) + 8 + 4 * min(L, 7) + 4 * dv) + BH * nst * per_chunk
    walk_reads = sum(bin(i).count("1") for i in range(N))
    walk_trans = sum(1 + bin(i >> ((i + 1) & -(i + 1)).bit_length()).count("1")
                     for i in range(N - 1))
    lu = (T - 1).bit_length() + 1
    walk_bytes = BH * nst * per_chunk + BH * T * (4 * max(0, lu - 7) + 8 * dv)
    return {
        "gdn_chunk": {"bytes": chunk_bytes, "flops": BH * (N * intra + nst * states)},
        "gdn_levels": {"bytes": walk_bytes,
                       "flops": BH * (walk_reads * 64 * 2 * dk * dv + walk_trans * 2 * dk * dk * dv)},
    }


def bench_gdn_fwd(steps: int, warmup: int) -> dict:
    """Log-linear Gated DeltaNet forward on the gdn8k workload (the fwd8k
    shape with a writing strength beta): the whole step, then each kernel
    alone, against the HBM and bf16 matrix-core rooflines."""
    cfg = I.CONFIGS["gdn8k"]
    log(f"gdn8k: generating inputs (B={cfg.B} H={cfg.H} T={cfg.T} dk={cfg.dk} dv={cfg.dv})")
    d = I.make_gdn(cfg, "base")
    dev = lambda x, dt=torch.float32: torch.from_numpy(x).to("cuda").to(dt).contiguous()  # noqa
    base = tuple(dev(d[n], torch.bfloat16) for n in ("q", "k", "v")) + \
        tuple(dev(d[n]) for n in ("a", "beta", "lam"))
    del d
    sets = [base + (torch.empty((cfg.B, cfg.H, cfg.T, cfg.dv), device="cuda"),)]
    for _ in range(NSETS - 1):
        sets.append(tuple(x.clone() for x in base) +
                    (torch.empty((cfg.B, cfg.H, cfg.T, cfg.dv), device="cuda"),))
    ws = torch.empty(LL.loglin_gdn_fwd_workspace_bytes(cfg.B, cfg.H, cfg.T, cfg.dk, cfg.dv, cfg.C,
                                                       torch.bfloat16),
                     dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    state = {"i": 0}

    def fwd(mask=LL.GDN_STAGE_ALL):
        q, k, v, a, b, lam, out = sets[state["i"] % NSETS]
        state["i"] += 1
        LL.loglin_gdn_fwd_chunked(q, k, v, a, b, lam, cfg.C, out=out, workspace=ws, stage_mask=mask)

    settle(fwd)
    for _ in range(warmup):
        fwd()
    ms = timed(fwd, steps, stream)
    tps = cfg.B * cfg.T / (ms / 1e3)
    models = gdn_models(cfg)
    kernels = {}
    for name, mask in (("gdn_chunk", LL.GDN_STAGE_CHUNK), ("gdn_levels", LL.GDN_STAGE_LEVELS)):
        fwd(mask)
        kms = timed(lambda: fwd(mask), max(5, steps), stream)
        m = models[name]
        tfl = m["flops"] / (kms / 1e3) / 1e12
        gbs = m["bytes"] / (kms / 1e3) / 1e9
        kernels[name] = {"ms": round(kms, 4), "TFLOP/s": round(tfl, 1),
                         # algorithmic flops over the bf16 matrix-core peak the
                         # kernels run on: a lower bound on that pipe's use (the
                         # fp32-accurate products issue two or three bf16 ones)
                         "frac_bf16_mfma": round(tfl / BF16_PEAK_TFLOPS, 4),
                         "GB/s": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                         "alg_bytes": m["bytes"], "alg_flops": m["flops"],
                         "traffic": measured_traffic(name)}
        log(f"  {name}: {kms:.3f} ms, {tfl:.1f} TFLOP/s algorithmic, {gbs:.0f} GB/s")
    log(f"gdn8k forward: {ms:.3f} ms/step, {tps:.3e} tokens/s")
    del sets, ws, base
    torch.cuda.empty_cache()
    return {"workload": "gdn8k", "tokens_per_s": tps, "ms_per_step": ms,
            "config": {"B": cfg.B, "H": cfg.H, "T": cfg.T, "dk": cfg.dk, "dv": cfg.dv, "L": cfg.L},
            "kernels": kernels}


def gdn_decode_bytes(pos0: np.ndarray, H: int, dk: int, dv: int, Lmax: int, steps: int) -> float:
    """Average algorithmic bytes per Gated DeltaNet decode step: at position
    t >= 1 the popcount(t-1) live levels above 0 are read and the popcount(t)
    levels above 0 after the step are written (the merged one and every
    carried one: the rank-one part of the transition changes each matrix);
    on the first step after a load level 0 is a loaded matrix and is read.
    Plus q, k, v (bf16), a, beta, lambda, the scales, the level-0 vectors
    and out."""
    st = dk * dv * 4
    small = (2 * dk + dv) * 2 + 8 + Lmax * 4 + 2 * Lmax * 4 + 2 * (dk + dv) * 4 + dv * 4
    tot = 0.0
    for s in range(steps):
        t = pos0 + s
        rd = np.array([bin(int(x) - 1).count("1") + (1 if s == 0 else 0) if x >= 1 else 0 for x in t])
        wr = np.array([bin(int(x)).count("1") if x >= 1 else 0 for x in t])
        tot += float(np.sum(rd + wr)) * st * H + len(t) * H * small
    return tot / steps


def bench_gdn_decode(steps: int) -> dict:
    cfg = I.CONFIGS["gdn_decode"]
    log(f"gdn decode: {cfg.nseq} sequences x {cfg.H} heads, Lmax={cfg.Lmax}, {steps} steps")
    d = I.make_decode(cfg.scaled(steps=steps), "base", fill=False)
    pos = d["pos"]
    g = torch.Generator(device="cuda")
    g.manual_seed(cfg.seed)
    levels = torch.randn((cfg.nseq, cfg.H, cfg.Lmax, cfg.dk, cfg.dv), device="cuda",
                         generator=g) * (1.0 / np.sqrt(cfg.dk))
    st = LL.loglin_state_init(cfg.nseq, cfg.H, cfg.dk, cfg.dv, cfg.Lmax)
    q, k, v = (torch.from_numpy(d[n]).to("cuda").to(torch.bfloat16) for n in ("q", "k", "v"))
    a, beta, lam = (torch.from_numpy(d[n]).to("cuda") for n in ("a", "beta", "lam"))
    out = torch.empty((cfg.nseq, cfg.H, cfg.dv), device="cuda")
    stream = torch.cuda.current_stream()
    t0 = time.perf_counter()
    while True:  # warm-up repeated for at least SETTLE_MS, as for decode
        LL.loglin_state_load(st, pos, levels)
        for s in range(min(steps, 64)):
            LL.loglin_gdn_decode_step(st, q[s], k[s], v[s], a[s], beta[s], lam[s], out=out)
        torch.cuda.synchronize()
        if (time.perf_counter() - t0) * 1e3 >= SETTLE_MS:
            break
    LL.loglin_state_load(st, pos, levels)
    del levels
    it = iter(range(steps))

    def step():
        s = next(it)
        LL.loglin_gdn_decode_step(st, q[s], k[s], v[s], a[s], beta[s], lam[s], out=out)

    ms = timed(step, steps, stream)
    LL.loglin_state_free(st)
    sps = 1e3 / ms
    byts = gdn_decode_bytes(pos, cfg.H, cfg.dk, cfg.dv, cfg.Lmax, steps)
    gbs = byts / (ms / 1e3) / 1e9
    log(f"gdn decode: {ms:.3f} ms/step, {sps:.1f} steps/s, {gbs:.0f} GB/s")
    return {"steps_per_s": sps, "tokens_per_s": sps * cfg.nseq, "ms_per_step": ms, "steps": steps,
            "config": {"workload": "gdn_decode", "nseq": cfg.nseq, "H": cfg.H, "dk": cfg.dk,
                       "dv": cfg.dv, "Lmax": cfg.Lmax},
            "roofline": {"kernel": "gdn_decode_step", "bound": "hbm", "achieved": round(gbs, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "alg_bytes_per_step": byts, "traffic": measured_traffic("gdn_decode_step")}}


if __name__ == "__main__":
    sys.exit(main())
