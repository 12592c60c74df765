"""Seeded synthetic inputs for the SSD forward.

This module holds the workload recipe only (shapes, seeds, distributions).  It
contains none of the SSD arithmetic and is the one module shared by the HIP
path's callers and the fp64 oracle's callers: both consume exactly the bytes
produced here.

Recipe (one PCG64 stream per workload, drawn in this order):
  x  ~ N(0,1)             float32, shape [B,L,H,P]
  Bm ~ N(0,1)             float32, shape [B,L,G,N]
  Cm ~ N(0,1)             float32, shape [B,L,G,N]
  dt_raw ~ N(0,1)         float64, shape [B,L,H];  dt = softplus(dt_raw - shift) -> float32
  A_u ~ U(0, ln 16)       float64, shape [H];      A  = -exp(A_u)                -> float32
  D  ~ N(0,1)             float32, shape [H]
x, Bm and Cm are rounded to bfloat16 (round to nearest even) when the
workload's input dtype is bf16; the float32 arrays then hold the bf16 values
exactly.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    chunk: int
    in_dtype: str          # "f32" or "bf16" (applies to x, B, C)
    dt_shift: float
    seed: int
    note: str = ""

    @property
    def nchunks(self) -> int:
        return (self.seqlen + self.chunk - 1) // self.chunk

    @property
    def tokens(self) -> int:
        return self.batch * self.seqlen

    def shape_dict(self) -> Dict[str, int]:
        return dict(batch=self.batch, seqlen=self.seqlen, nheads=self.nheads, headdim=self.headdim,
                    dstate=self.dstate, ngroups=self.ngroups, chunk=self.chunk)


# The five synthetic workloads (Mamba-2-shaped layers).
WORKLOADS: Dict[str, Workload] = {
    w.name: w for w in [
        Workload("tiny_f32", 1, 256, 2, 16, 16, 1, 64, "f32", 2.0, 0, "tiny, all fp32"),
        Workload("mamba2_130m_layer", 4, 2048, 24, 64, 128, 1, 256, "bf16", 2.0, 1, "Mamba-2 130M-style layer"),
        Workload("mamba2_2p7b_layer", 2, 8192, 80, 64, 128, 1, 256, "bf16", 2.0, 2, "Mamba-2 2.7B-style layer"),
        Workload("long_seq_65k", 1, 65536, 32, 64, 128, 1, 256, "bf16", 4.0, 3, "long sequence, slow decay"),
        Workload("grouped_n256", 8, 4096, 64, 64, 256, 8, 128, "bf16", 2.0, 4, "N=256, 8 heads per B/C group"),
    ]
}
HEADLINE = "mamba2_2p7b_layer"


def bf16_round(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bits (uint16), round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = ((u >> 16) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + r) >> 16).astype(np.uint16)


def bf16_widen(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bits (uint16) -> float32 (exact)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class SSDInputs:
    """One batch of inputs.  ``x``/``Bm``/``Cm`` are float32 arrays holding the
    exact values the GPU sees; ``*_bits`` are the bf16 encodings when
    ``in_dtype == 'bf16'``."""
    x: np.ndarray
    dt: np.ndarray
    A: np.ndarray
    Bm: np.ndarray
    Cm: np.ndarray
    D: np.ndarray
    in_dtype: str
    chunk: int
    x_bits: Optional[np.ndarray] = None
    Bm_bits: Optional[np.ndarray] = None
    Cm_bits: Optional[np.ndarray] = None

    @property
    def shape(self):
        Bsz, L, H, P = self.x.shape
        return dict(batch=Bsz, seqlen=L, nheads=H, headdim=P, dstate=self.Bm.shape[3],
                    ngroups=self.Bm.shape[2], chunk=self.chunk)

    def to_torch(self, device="cuda"):
        """Upload to torch tensors: x/B/C in the input dtype, dt/A/D float32."""
        import torch
        out = {}
        for name in ("x", "Bm", "Cm"):
            if self.in_dtype == "bf16":
                bits = getattr(self, name + "_bits")
                t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
            else:
                t = torch.from_numpy(getattr(self, name))
            out[name] = t.to(device).contiguous()
        for name in ("dt", "A", "D"):
            out[name] = torch.from_numpy(getattr(self, name)).to(device).contiguous()
        return out


def softplus64(v: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, v)


def make_inputs(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, *, in_dtype="f32",
                dt_shift=2.0, seed=0, A_override=None, dt_override=None,
                log_a_range=(0.0, math.log(16.0))) -> SSDInputs:
    """Draw one seeded batch following the recipe in the module docstring.

    ``A_override`` / ``dt_override`` replace A (shape [H]) or dt (shape
    [B,L,H]) after the draws, for special cases (A = 0, slow decay, ...)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((batch, seqlen, nheads, headdim), dtype=np.float32)
    Bm = rng.standard_normal((batch, seqlen, ngroups, dstate), dtype=np.float32)
    Cm = rng.standard_normal((batch, seqlen, ngroups, dstate), dtype=np.float32)
    dt_raw = rng.standard_normal((batch, seqlen, nheads))
    a_u = rng.uniform(log_a_range[0], log_a_range[1], size=nheads)
    D = rng.standard_normal(nheads, dtype=np.float32)
    dt = softplus64(dt_raw - dt_shift).astype(np.float32)
    A = (-np.exp(a_u)).astype(np.float32)
    if A_override is not None:
        A = np.ascontiguousarray(np.broadcast_to(np.asarray(A_override, dtype=np.float32), (nheads,)))
    if dt_override is not None:
        dt = np.ascontiguousarray(np.broadcast_to(np.asarray(dt_override, dtype=np.float32),
                                                  (batch, seqlen, nheads)))
    inp = SSDInputs(x=x, dt=dt, A=A, Bm=Bm, Cm=Cm, D=D, in_dtype=in_dtype, chunk=chunk)
    if in_dtype == "bf16":
        for name in ("x", "Bm", "Cm"):
            bits = bf16_round(getattr(inp, name))
            setattr(inp, name + "_bits", bits)
            setattr(inp, name, bf16_widen(bits))
    elif in_dtype != "f32":
        raise ValueError(f"unknown input dtype {in_dtype!r}")
    return inp


def workload_inputs(name: str, **overrides) -> SSDInputs:
    w = WORKLOADS[name]
    kw = dict(in_dtype=w.in_dtype, dt_shift=w.dt_shift, seed=w.seed)
    kw.update(overrides)
    return make_inputs(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk, **kw)
