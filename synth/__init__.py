"""Seeded synthetic inputs for the dual-phase policy step.

This module only *draws numbers*: workload shapes, weight tensors, prefix hidden
states and initial noise.  It holds none of the policy's arithmetic, so both the
CPU oracle (through the tests) and the HIP library (through the Python binding)
can take their inputs from here without sharing any computation.

Distributions (the workload descriptions give them; the pages print no weights):
  * prefix hidden states and the initial action noise X^0 ~ N(0, 1), float32;
  * every linear weight ~ N(0, 0.02^2), drawn in float32 and, for the bf16
    workloads, rounded to the nearest bfloat16 (ties to even) so the CPU and GPU
    see the same representable values;
  * every RMSNorm gain w ~ N(0, 0.02^2) (the norm applies (1 + w));
  * ternary weights q ~ U{-1, 0, +1} i.i.d., one fp32 scale per tensor equal to
    E|N(0, 0.02^2)| = 0.02 * sqrt(2/pi) (the per-tensor absmean of the latent
    Gaussian the codes stand in for).

Streams: numpy.random.SeedSequence(seed).spawn(n) gives one independent stream
per weight tensor in boundary order, then one for the prefix, then one for the
noise, so a tensor's values do not depend on which other tensors were drawn.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, asdict, replace
from typing import Dict, List, Tuple

import numpy as np

__all__ = [
    "PolicyConfig", "CONFIGS", "config", "weight_specs", "make_weights",
    "make_prefix", "make_noise", "make_all", "TERNARY_BETA",
]

# fp32(0.02 * sqrt(2/pi)): mean absolute value of N(0, 0.02^2).
TERNARY_BETA = float(np.float32(0.02 * math.sqrt(2.0 / math.pi)))


@dataclass(frozen=True)
class PolicyConfig:
    name: str
    precision: str          # "f32", "bf16" or "w2a8" (ternary prefix, bf16 expert)
    batch: int              # independent observations per call
    n_prefix: int           # prefix tokens per observation
    # prefix encoder
    d_p: int
    L_p: int
    Hq: int
    Hkv: int
    hd: int
    F_p: int
    # action expert
    d_e: int
    L_e: int
    Hq_e: int
    Hkv_e: int
    hd_e: int
    F_e: int
    # action chunk and solver
    H: int
    d_a: int
    steps: int
    rms_eps: float = 1e-6
    attn: str = "cross"     # "cross" (projected final states, Eq. 2) or "joint" (per-layer prefix K/V)

    def to_dict(self) -> dict:
        return asdict(self)


_EXPERT_1024 = dict(d_e=1024, L_e=18, Hq_e=8, Hkv_e=1, hd_e=256, F_e=4096)
_BACKBONE_2048 = dict(d_p=2048, L_p=18, Hq=8, Hkv=1, hd=256, F_p=16384)

CONFIGS: Tuple[PolicyConfig, ...] = (
    # tiny fp32 policy: 64-token prefix, 2+2 layers of width 128, 8x7 chunk, 4 steps
    PolicyConfig("tiny_fp32", "f32", 1, 64, 128, 2, 4, 4, 32, 512,
                 128, 2, 4, 4, 32, 512, 8, 7, 4),
    # single camera bf16: 288-token prefix (256 patches + 24 text + 8 state)
    PolicyConfig("single_camera_bf16", "bf16", 1, 288, **_BACKBONE_2048,
                 **_EXPERT_1024, H=50, d_a=32, steps=10),
    # dual arm bf16: 816-token prefix (3 x 256 patches + 40 text + 8 state)
    PolicyConfig("dual_arm_bf16", "bf16", 1, 816, **_BACKBONE_2048,
                 **_EXPERT_1024, H=16, d_a=14, steps=4),
    # batched throughput: 16 observations of 512 tokens each
    PolicyConfig("batched16_bf16", "bf16", 16, 512, **_BACKBONE_2048,
                 **_EXPERT_1024, H=50, d_a=32, steps=10),
    # ternary W2A8 prefix (30 layers, d=2560, 20 heads x 128, MLP 6912), bf16 expert
    PolicyConfig("ternary_w2a8", "w2a8", 1, 320, 2560, 30, 20, 20, 128, 6912,
                 **_EXPERT_1024, H=8, d_a=7, steps=4),
)


def config(i_or_name, **overrides) -> PolicyConfig:
    """Workload by index (0..4) or name, optionally with fields replaced."""
    if isinstance(i_or_name, int):
        c = CONFIGS[i_or_name]
    else:
        c = next(c for c in CONFIGS if c.name == i_or_name)
    return replace(c, **overrides) if overrides else c


def weight_specs(cfg: PolicyConfig) -> List[Tuple[str, Tuple[int, ...], str]]:
    """(name, shape, kind) for every weight tensor, in the library's boundary order.

    kind is "gain" (RMSNorm gain, fp32), "linear" ([out, in], fp32 or bf16) or
    "ternary" ([out, in] codes in {-1, 0, 1}).
    """
    lin_p = "ternary" if cfg.precision == "w2a8" else "linear"
    qw, kvw = cfg.Hq * cfg.hd, cfg.Hkv * cfg.hd
    qe, kve = cfg.Hq_e * cfg.hd_e, cfg.Hkv_e * cfg.hd_e
    specs = []
    for l in range(cfg.L_p):
        p = f"prefix.{l}."
        specs += [
            (p + "w1", (cfg.d_p,), "gain"),
            (p + "wq", (qw, cfg.d_p), lin_p),
            (p + "wk", (kvw, cfg.d_p), lin_p),
            (p + "wv", (kvw, cfg.d_p), lin_p),
            (p + "wo", (cfg.d_p, qw), lin_p),
            (p + "w2", (cfg.d_p,), "gain"),
            (p + "wg", (cfg.F_p, cfg.d_p), lin_p),
            (p + "wu", (cfg.F_p, cfg.d_p), lin_p),
            (p + "wd", (cfg.d_p, cfg.F_p), lin_p),
        ]
    joint = cfg.attn == "joint"
    if not joint:
        specs.append(("prefix.norm", (cfg.d_p,), "gain"))
        for e in range(cfg.L_e):
            specs += [
                (f"cache.{e}.wk", (kve, cfg.d_p), "linear"),
                (f"cache.{e}.wv", (kve, cfg.d_p), "linear"),
            ]
    specs.append(("expert.w_in", (cfg.d_e, cfg.d_a), "linear"))
    for e in range(cfg.L_e):
        p = f"expert.{e}."
        specs += [
            (p + "a1", (cfg.d_e,), "gain"),
            (p + "wqs", (qe, cfg.d_e), "linear"),
            (p + "wks", (kve, cfg.d_e), "linear"),
            (p + "wvs", (kve, cfg.d_e), "linear"),
            (p + "wos", (cfg.d_e, qe), "linear"),
        ]
        if not joint:
            specs += [
                (p + "a2", (cfg.d_e,), "gain"),
                (p + "wqc", (qe, cfg.d_e), "linear"),
                (p + "woc", (cfg.d_e, qe), "linear"),
            ]
        specs += [
            (p + "a3", (cfg.d_e,), "gain"),
            (p + "wg", (cfg.F_e, cfg.d_e), "linear"),
            (p + "wu", (cfg.F_e, cfg.d_e), "linear"),
            (p + "wd", (cfg.d_e, cfg.F_e), "linear"),
        ]
    specs.append(("expert.norm", (cfg.d_e,), "gain"))
    specs.append(("expert.w_out", (cfg.d_a, cfg.d_e), "linear"))
    return specs


def _round_bf16(x: np.ndarray) -> np.ndarray:
    """Nearest bfloat16 value (ties to even) of float32 data, kept as float32."""
    import torch
    t = torch.from_numpy(x)
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def _draw(kind: str, shape, seed_seq, bf16: bool) -> np.ndarray:
    rng = np.random.default_rng(seed_seq)
    if kind == "ternary":
        return rng.integers(-1, 2, size=shape, dtype=np.int8)
    out = np.empty(shape, dtype=np.float32)
    rng.standard_normal(out=out, dtype=np.float32)
    out *= np.float32(0.02)
    if kind == "linear" and bf16:
        out = _round_bf16(out)
    return out


def _streams(cfg: PolicyConfig, seed: int):
    n = len(weight_specs(cfg))
    return np.random.SeedSequence(seed).spawn(n + 2)


def make_weights(cfg: PolicyConfig, seed: int, workers: int | None = None
                 ) -> Tuple[Dict[str, np.ndarray], Dict[str, float]]:
    """All weights by name, plus the fp32 scale of every ternary tensor."""
    specs = weight_specs(cfg)
    streams = _streams(cfg, seed)
    bf16 = cfg.precision in ("bf16", "w2a8")
    workers = workers or min(8, os.cpu_count() or 1)
    with ThreadPoolExecutor(max_workers=workers) as ex:
        arrays = list(ex.map(lambda i: _draw(specs[i][2], specs[i][1], streams[i], bf16),
                             range(len(specs))))
    weights = {s[0]: a for s, a in zip(specs, arrays)}
    betas = {s[0]: TERNARY_BETA for s in specs if s[2] == "ternary"}
    return weights, betas


def make_prefix(cfg: PolicyConfig, seed: int) -> np.ndarray:
    """Prefix hidden states Z0 [B, N, d_p] ~ N(0, 1), float32."""
    rng = np.random.default_rng(_streams(cfg, seed)[-2])
    out = np.empty((cfg.batch, cfg.n_prefix, cfg.d_p), dtype=np.float32)
    rng.standard_normal(out=out, dtype=np.float32)
    return out


def make_noise(cfg: PolicyConfig, seed: int) -> np.ndarray:
    """Initial action noise X^0 [B, H, d_a] ~ N(0, 1), float32."""
    rng = np.random.default_rng(_streams(cfg, seed)[-1])
    out = np.empty((cfg.batch, cfg.H, cfg.d_a), dtype=np.float32)
    rng.standard_normal(out=out, dtype=np.float32)
    return out


def make_all(cfg: PolicyConfig, seed: int):
    w, b = make_weights(cfg, seed)
    return w, b, make_prefix(cfg, seed), make_noise(cfg, seed)
