"""Seeded synthetic inputs for the selective-scan and SSD hot path.

This module is shared by the fp64 oracle side (tests, bench's CPU baseline)
and the HIP side (tests, bench, smoke). It draws random numbers and rounds
them to the storage dtype; it holds none of the method's arithmetic (no
discretisation, no recurrence, no softplus of the inputs). The one formula it
evaluates is the inverse of softplus, used only to place the per-channel bias
so that the median step size lands in a requested interval.

Recipe (stated once, used everywhere):
  * numpy ``Generator(PCG64)`` seeded with ``SeedSequence(seed)``; ``seed``
    defaults to ``1000 + config index``. The sequence is spawned into
    independent children in the fixed order
    ``[x, delta_raw, z, B, C, Dskip, dt0, h0, A]``.
  * Normal draws are fp32 (``standard_normal(dtype=float32)``); uniform draws
    are fp64. Storage dtype ``bf16`` means round-to-nearest-even of the fp32
    draw to bfloat16; arrays are returned as float32 holding those exactly
    representable values, so both sides read bit-identical inputs.
  * ``x, z, B, C, Dskip ~ N(0,1)``; ``delta_raw ~ N(0, 0.5^2)``.
  * step size: per channel (per head for SSD) ``dt0 = exp(U(ln lo, ln hi))``
    and ``bias = log(expm1(dt0))``, so ``softplus(0 + bias) = dt0``: the
    interval bounds the per-channel median step, the N(0, 0.5^2) raw part
    spreads it by roughly e^{+-1} at two sigma. Nothing is clamped.
  * scan: ``A[d, n] = -(n + 1)``; SSD: ``A_h = -U(1, 16)``.
  * B and C have layout (batch, L, N): one group shared by every channel.
  * short convolution: its own seed sequence spawned as ``[x, w, bias, x0]``;
    ``x, x0 ~ N(0,1)``, ``w ~ N(0, 1/K)``, ``bias ~ N(0, 0.1^2)`` (fp32 weights).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

__all__ = [
    "ScanConfig", "SSDConfig", "CONFIGS", "CONFIG_ORDER",
    "round_bf16", "bf16_bits", "scan_inputs", "ssd_inputs", "make_inputs", "conv_inputs",
]


@dataclasses.dataclass(frozen=True)
class ScanConfig:
    name: str
    index: int
    batch: int
    seqlen: int
    dim: int
    dstate: int
    dtype: str            # "f32" or "bf16": storage of x, delta, z, B, C, y
    dt_min: float
    dt_max: float
    kind: str = "scan"

    @property
    def elements(self) -> int:
        return self.batch * self.seqlen * self.dim * self.dstate


@dataclasses.dataclass(frozen=True)
class SSDConfig:
    name: str
    index: int
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    dstate: int
    chunk: int
    dtype: str
    dt_min: float
    dt_max: float
    a_lo: float
    a_hi: float
    kind: str = "ssd"

    @property
    def elements(self) -> int:
        return self.batch * self.seqlen * self.nheads * self.headdim * self.dstate


# The five workloads. Shapes are those of real layers: d_model x expand 2 for
# the Mamba-1 scans (N=16), 64 heads x 64 head dim with N=128 for the
# Mamba-2 SSD form.
CONFIGS = {
    "S1": ScanConfig("tiny_scan_fp32", 0, 1, 256, 64, 16, "f32", 1e-3, 1e-1),
    "S2": ScanConfig("mamba130m_layer_scan_bf16", 1, 8, 2048, 1536, 16, "bf16", 1e-3, 1e-1),
    "S3": ScanConfig("mamba2p8b_layer_scan_bf16", 2, 4, 8192, 5120, 16, "bf16", 1e-3, 1e-1),
    "S4": ScanConfig("long_context_scan_bf16", 3, 1, 131072, 2048, 16, "bf16", 1e-4, 1e-2),
    "S5": SSDConfig("mamba2_ssd_bf16", 4, 2, 8192, 64, 64, 128, 256, "bf16", 1e-3, 1e-1, 1.0, 16.0),
}
CONFIG_ORDER = ["S1", "S2", "S3", "S4", "S5"]

_STREAMS = ["x", "delta", "z", "B", "C", "Dskip", "dt0", "h0", "A"]


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return float32
    holding the rounded values. NaNs stay NaN (quiet bit set)."""
    src = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty_like(src)
    su = src.reshape(-1).view(np.uint32)
    ou = out.reshape(-1).view(np.uint32)
    block = 1 << 24            # bounded temporaries for large arrays
    for i in range(0, su.size, block):
        u = su[i:i + block]
        # add half an ulp of bf16 (plus the kept lsb for ties); no overflow below NaN
        r = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
        nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
        r = np.where(nan, u | np.uint32(0x00400000), r)
        ou[i:i + block] = r & np.uint32(0xFFFF0000)
    return out


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) of float32 values, round-to-nearest-even."""
    return (round_bf16(a).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _rngs(seed: int):
    children = np.random.SeedSequence(seed).spawn(len(_STREAMS))
    return {k: np.random.Generator(np.random.PCG64(s)) for k, s in zip(_STREAMS, children)}


def _normal(rng, shape, scale, dtype):
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        a *= np.float32(scale)
    return round_bf16(a) if dtype == "bf16" else a


def _bias_for(rng, count, lo, hi):
    """Per-channel bias whose softplus is a log-uniform median step in [lo, hi]."""
    dt0 = np.exp(rng.uniform(math.log(lo), math.log(hi), size=count))
    return np.log(np.expm1(dt0)).astype(np.float32)


def scan_inputs(batch: int, seqlen: int, dim: int, dstate: int, dtype: str = "f32",
                seed: int = 0, dt_range=(1e-3, 1e-1), with_h0: bool = False,
                with_z: bool = True, with_D: bool = True, with_bias: bool = True,
                ngroups: int = 1) -> dict:
    """Inputs of one selective-scan call.

    Returns float32 numpy arrays (bf16-exact values when ``dtype == "bf16"``):
    x, delta, z: (batch, L, D); Bm, Cm: (batch, L, N), or (batch, L, G, N) with
    ``ngroups`` G > 1; A: (D, N);
    delta_bias, Dskip: (D,); h0: (batch, D, N) or None.
    """
    r = _rngs(seed)
    out = {"dtype": dtype, "kind": "scan"}
    out["x"] = _normal(r["x"], (batch, seqlen, dim), 1.0, dtype)
    out["delta"] = _normal(r["delta"], (batch, seqlen, dim), 0.5, dtype)
    out["z"] = _normal(r["z"], (batch, seqlen, dim), 1.0, dtype) if with_z else None
    bc = (batch, seqlen, dstate) if ngroups == 1 else (batch, seqlen, ngroups, dstate)
    out["Bm"] = _normal(r["B"], bc, 1.0, dtype)
    out["Cm"] = _normal(r["C"], bc, 1.0, dtype)
    out["Dskip"] = r["Dskip"].standard_normal(size=dim, dtype=np.float32) if with_D else None
    out["delta_bias"] = _bias_for(r["dt0"], dim, *dt_range) if with_bias else None
    out["A"] = np.ascontiguousarray(
        np.broadcast_to(-np.arange(1, dstate + 1, dtype=np.float32), (dim, dstate)))
    out["h0"] = (r["h0"].standard_normal(size=(batch, dim, dstate), dtype=np.float32)
                 if with_h0 else None)
    return out


def ssd_inputs(batch: int, seqlen: int, nheads: int, headdim: int, dstate: int,
               dtype: str = "bf16", seed: int = 0, dt_range=(1e-3, 1e-1),
               a_range=(1.0, 16.0), with_h0: bool = False, with_z: bool = False,
               with_D: bool = True, with_bias: bool = True, ngroups: int = 1) -> dict:
    """Inputs of one SSD (scalar A per head) call.

    x: (batch, L, H, P); dt: (batch, L, H) raw; dt_bias, A, Dskip: (H,);
    Bm, Cm: (batch, L, N), or (batch, L, G, N) with ``ngroups`` G > 1; z: (batch, L, H, P) or None; h0: (batch, H, P, N) or None.
    """
    r = _rngs(seed)
    out = {"dtype": dtype, "kind": "ssd"}
    out["x"] = _normal(r["x"], (batch, seqlen, nheads, headdim), 1.0, dtype)
    out["dt"] = _normal(r["delta"], (batch, seqlen, nheads), 0.5, dtype)
    out["z"] = _normal(r["z"], (batch, seqlen, nheads, headdim), 1.0, dtype) if with_z else None
    bc = (batch, seqlen, dstate) if ngroups == 1 else (batch, seqlen, ngroups, dstate)
    out["Bm"] = _normal(r["B"], bc, 1.0, dtype)
    out["Cm"] = _normal(r["C"], bc, 1.0, dtype)
    out["Dskip"] = r["Dskip"].standard_normal(size=nheads, dtype=np.float32) if with_D else None
    out["dt_bias"] = _bias_for(r["dt0"], nheads, *dt_range) if with_bias else None
    out["A"] = (-r["A"].uniform(a_range[0], a_range[1], size=nheads)).astype(np.float32)
    out["h0"] = (r["h0"].standard_normal(size=(batch, nheads, headdim, dstate), dtype=np.float32)
                 if with_h0 else None)
    return out


def make_inputs(key: str, seed: Optional[int] = None, **kw) -> dict:
    """Inputs of one of the five named workloads (``"S1"`` .. ``"S5"``)."""
    cfg = CONFIGS[key]
    seed = 1000 + cfg.index if seed is None else seed
    if cfg.kind == "scan":
        return scan_inputs(cfg.batch, cfg.seqlen, cfg.dim, cfg.dstate, cfg.dtype, seed,
                           (cfg.dt_min, cfg.dt_max), **kw)
    return ssd_inputs(cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.dstate, cfg.dtype,
                      seed, (cfg.dt_min, cfg.dt_max), (cfg.a_lo, cfg.a_hi), **kw)


def conv_inputs(batch: int, seqlen: int, dim: int, width: int = 4, dtype: str = "bf16",
                seed: int = 0, with_state: bool = False, with_bias: bool = True) -> dict:
    """Inputs of one causal depthwise conv1d call: x (batch, L, D) in the storage
    dtype, weight (D, K) and bias (D,) fp32, x0 (batch, K-1, D) history or None."""
    kids = np.random.SeedSequence(seed).spawn(4)
    r = [np.random.Generator(np.random.PCG64(c)) for c in kids]
    out = {"dtype": dtype, "kind": "conv"}
    out["x"] = _normal(r[0], (batch, seqlen, dim), 1.0, dtype)
    out["w"] = r[1].standard_normal(size=(dim, width), dtype=np.float32) * np.float32(1.0 / math.sqrt(width))
    out["bias"] = (r[2].standard_normal(size=dim, dtype=np.float32) * np.float32(0.1)) if with_bias else None
    out["x0"] = _normal(r[3], (batch, width - 1, dim), 1.0, dtype) if with_state else None
    return out
