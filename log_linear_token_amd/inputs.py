"""Seeded synthetic inputs for the log-linear token mixer.

This module only draws random numbers and rounds them to the storage dtype; it
holds none of the mixer's arithmetic, so both the HIP path and the CPU oracle
can be fed from it.  Every array is returned as float32 (bf16 workloads hold
values that are exactly representable in bf16, rounded to nearest-even), so
that both sides consume identical values.

Workloads (shapes and distributions of the forward and decode settings the
mixer is measured on):

  tiny      B=1  H=1  T=64    dk=dv=16        fp32 C=16  L=8
  fwd2k     B=2  H=8  T=2048  dk=dv=64        bf16 C=64  L=13  (q, k L2-normalised)
  fwd8k     B=4  H=16 T=8192  dk=128 dv=64    bf16 C=64  L=15  (long-memory decay)
  decode    128 sequences, H=32, dk=dv=128, fp32 states, Lmax=17, 256 steps
  long64k   B=1  H=16 T=65536 dk=dv=128       bf16 C=128 L=18
  gdn8k     the fwd8k shape, log-linear Gated DeltaNet (beta added, q, k L2-normalised)
  gdn2k     the fwd2k shape, log-linear Gated DeltaNet
  gdn_decode the decode shape, log-linear Gated DeltaNet (beta per step)
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import numpy as np


@dataclass(frozen=True)
class FwdConfig:
    name: str
    cid: int
    B: int
    H: int
    T: int
    dk: int
    dv: int
    C: int
    L: int
    dtype: str          # "f32" or "bf16"
    qk: str             # "scaled": N(0,1)/sqrt(dk);  "l2": N(0,1) then unit L2 norm over dk
    decay_mu: float     # a = -softplus(N(decay_mu, decay_sigma))
    decay_sigma: float
    lam: str            # "uniform": U[0,1];  "softplus": softplus(N(0,1))

    @property
    def seed(self) -> int:
        return 20260000 + self.cid

    @property
    def tokens(self) -> int:
        return self.B * self.T

    def scaled(self, **kw) -> "FwdConfig":
        """Same distributions, other sizes (for parity cases the oracle finishes quickly)."""
        return replace(self, **kw)


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    cid: int
    nseq: int
    H: int
    dk: int
    dv: int
    Lmax: int
    steps: int
    max_prefill: int
    dtype: str

    @property
    def seed(self) -> int:
        return 20260000 + self.cid

    def scaled(self, **kw) -> "DecodeConfig":
        return replace(self, **kw)


CONFIGS = {
    "tiny": FwdConfig("tiny", 1, 1, 1, 64, 16, 16, 16, 8, "f32", "scaled", 0.0, 1.0, "uniform"),
    "fwd2k": FwdConfig("fwd2k", 2, 2, 8, 2048, 64, 64, 64, 13, "bf16", "l2", 0.0, 1.0, "uniform"),
    "fwd8k": FwdConfig("fwd8k", 3, 4, 16, 8192, 128, 64, 64, 15, "bf16", "scaled", -2.0, 0.5,
                       "softplus"),
    "decode": DecodeConfig("decode", 4, 128, 32, 128, 128, 17, 256, 32768, "bf16"),
    "long64k": FwdConfig("long64k", 5, 1, 16, 65536, 128, 128, 128, 18, "bf16", "scaled", -3.0,
                         0.5, "uniform"),
    # log-linear Gated DeltaNet (make_gdn adds beta): the 8K and 2K shapes
    "gdn8k": FwdConfig("gdn8k", 6, 4, 16, 8192, 128, 64, 64, 15, "bf16", "l2", -2.0, 0.5,
                       "softplus"),
    "gdn2k": FwdConfig("gdn2k", 7, 2, 8, 2048, 64, 64, 64, 13, "bf16", "l2", 0.0, 1.0,
                       "uniform"),
    "gdn_decode": DecodeConfig("gdn_decode", 8, 128, 32, 128, 128, 17, 256, 32768, "bf16"),
}


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    nan = np.isnan(x)
    out = r.astype(np.uint32).view(np.float32).copy()
    out[nan] = np.float32("nan")
    return out


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, x).astype(np.float32)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    return round_bf16(x) if dtype == "bf16" else x


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return (1.0 / (1.0 + np.exp(-x.astype(np.float64)))).astype(np.float32)


def make_gdn(cfg: FwdConfig, variant: str = "base", seed: int | None = None) -> dict:
    """Inputs of a log-linear Gated DeltaNet forward: make_fwd's q, k, v, a, lam
    (q, k unit L2 norm over dk whatever cfg.qk says, as the delta rule needs
    ||k|| <= 1 for beta <= 1 to keep its transition contractive) plus the
    writing strength beta [B,H,T] = sigmoid(N(0,1)), drawn after the rest
    from the same generator."""
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    d = _draw_fwd(replace(cfg, qk="l2"), variant, rng)
    d["beta"] = _sigmoid(rng.standard_normal((cfg.B, cfg.H, cfg.T), dtype=np.float32))
    return d


def make_fwd(cfg: FwdConfig, variant: str = "base", seed: int | None = None) -> dict:
    """Draw q, k, v, a, lam for one forward workload.

    variant: "base" (the workload's own decay), "unit" (a = 0: no decay),
    "weak" (a = -softplus(N(-8, 0.5)), about 3e-4 per token).
    Returns a dict of float32 arrays q, k [B,H,T,dk], v [B,H,T,dv], a [B,H,T],
    lam [B,H,T,L] plus the config.
    """
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    return _draw_fwd(cfg, variant, rng)


def _draw_fwd(cfg: FwdConfig, variant: str, rng: np.random.Generator) -> dict:
    shp = (cfg.B, cfg.H, cfg.T)
    q = rng.standard_normal(shp + (cfg.dk,), dtype=np.float32)
    k = rng.standard_normal(shp + (cfg.dk,), dtype=np.float32)
    if cfg.qk == "l2":
        q /= np.maximum(np.linalg.norm(q, axis=-1, keepdims=True), 1e-12)
        k /= np.maximum(np.linalg.norm(k, axis=-1, keepdims=True), 1e-12)
    else:
        q *= np.float32(1.0 / math.sqrt(cfg.dk))
        k *= np.float32(1.0 / math.sqrt(cfg.dk))
    v = rng.standard_normal(shp + (cfg.dv,), dtype=np.float32)
    if variant == "base":
        a = -_softplus(cfg.decay_mu + cfg.decay_sigma * rng.standard_normal(shp, dtype=np.float32))
    elif variant == "unit":
        a = np.zeros(shp, dtype=np.float32)
    elif variant == "weak":
        a = -_softplus(-8.0 + 0.5 * rng.standard_normal(shp, dtype=np.float32))
    else:
        raise ValueError(f"unknown variant {variant!r}")
    if cfg.lam == "uniform":
        lam = rng.random(shp + (cfg.L,), dtype=np.float32)
    else:
        lam = _softplus(rng.standard_normal(shp + (cfg.L,), dtype=np.float32))
    return {
        "cfg": cfg,
        "q": _store(q, cfg.dtype),
        "k": _store(k, cfg.dtype),
        "v": _store(v, cfg.dtype),
        "a": np.ascontiguousarray(a, dtype=np.float32),
        "lam": np.ascontiguousarray(lam, dtype=np.float32),
    }


def make_decode(cfg: DecodeConfig, variant: str = "base", seed: int | None = None,
                fill: bool = True, live_slots=None) -> dict:
    """Draw a synthetic pre-filled decode state and the per-step inputs.

    Every sequence gets a random prefill length n in [1, max_prefill].  With
    fill=True the level slots are filled with N(0, 1/dk) fp32 values: only
    the slots live_slots(n) lists (the others zero) when the caller passes
    that function, every slot otherwise.  This module does not know which
    slots a position uses; the state loader ignores the others.  Per step:
    q, k, v [steps, nseq, H, d] (bf16 values, N(0,1)/sqrt(dk)),
    a [steps, nseq, H], lam [steps, nseq, H, Lmax].  With fill=False the
    states are returned as None (callers that only need the per-step inputs,
    or fill the device state themselves).
    """
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    pos = rng.integers(1, cfg.max_prefill + 1, size=cfg.nseq).astype(np.int64)
    sshape = (cfg.nseq, cfg.H, cfg.Lmax, cfg.dk, cfg.dv)
    states = None
    if fill:
        states = np.zeros(sshape, dtype=np.float32)
        sd = np.float32(1.0 / math.sqrt(cfg.dk))
        for s in range(cfg.nseq):
            slots = range(cfg.Lmax) if live_slots is None else live_slots(int(pos[s]))
            for lv in slots:
                states[s, :, lv] = sd * rng.standard_normal((cfg.H, cfg.dk, cfg.dv),
                                                            dtype=np.float32)
    st = (cfg.steps, cfg.nseq, cfg.H)
    inv = np.float32(1.0 / math.sqrt(cfg.dk))
    q = rng.standard_normal(st + (cfg.dk,), dtype=np.float32) * inv
    k = rng.standard_normal(st + (cfg.dk,), dtype=np.float32) * inv
    v = rng.standard_normal(st + (cfg.dv,), dtype=np.float32) * np.float32(1.0 / math.sqrt(cfg.dv))
    if variant == "base":
        a = -_softplus(rng.standard_normal(st, dtype=np.float32))
    elif variant == "unit":
        a = np.zeros(st, dtype=np.float32)
    else:
        raise ValueError(f"unknown variant {variant!r}")
    lam = rng.random(st + (cfg.Lmax,), dtype=np.float32)
    # writing strength of the Gated DeltaNet step (drawn last; unused by the
    # scalar-gated mixer)
    beta = _sigmoid(rng.standard_normal(st, dtype=np.float32))
    return {
        "cfg": cfg,
        "pos": pos,
        "beta": beta,
        "states": states,
        "q": _store(q, cfg.dtype),
        "k": _store(k, cfg.dtype),
        "v": _store(v, cfg.dtype),
        "a": np.ascontiguousarray(a, dtype=np.float32),
        "lam": np.ascontiguousarray(lam, dtype=np.float32),
    }
