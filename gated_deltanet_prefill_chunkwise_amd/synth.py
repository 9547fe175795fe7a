"""Seeded synthetic inputs for the GDN-core prefill.

This module only draws random numbers and shapes them into the input
distribution of the workload; it holds none of the operator's arithmetic.
Both the HIP path (via the tests and the benchmark) and the fp64 oracle
(via the tests) consume what it returns.

Workload recipe (head geometry of the SparseGDN reading notes, Sec. 2.1:
Nq = 16 query/key heads, Nv = 32 value heads, d = dv = 128, value heads
2p and 2p+1 share query/key head p):

  q, k  ~ N(0, 1), then L2-normalised per (token, head)
  v     ~ N(0, 1)
  beta  = sigmoid(N(0, 1))
  a     = -softplus(N(0, 1)) * exp(u_h) / ln 2      (log2 retention per token)
          u_h ~ U(0, ln 4) per value head (U(0, ln 16) for the wide sweep)
  z     ~ N(0, 1)                                    (output gate, per token)

Two generators are provided:

* ``numpy_inputs``: numpy ``Generator(PCG64(seed))``, float64 draws in the
  order q, k, v, beta_pre, a_pre, u, z, per sequence.  Used for every size
  the CPU oracle handles.
* ``torch_inputs``: the same recipe drawn with a seeded torch generator on
  the target device (philox on the GPU).  Used for full-size benchmark
  inputs, where drawing ~1.6e9 normals on the host would take minutes.
  It is a different random stream from ``numpy_inputs``.

Values meant for a bf16 problem are rounded fp32 -> bf16 with
round-to-nearest-even; ``a`` always stays fp32.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np


def seed_for(config: int, layer: int = 0, sequence: int = 0) -> int:
    """Seed = 1e6 * config + 1e3 * layer + sequence."""
    return 1_000_000 * config + 1_000 * layer + sequence


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float values to the nearest bf16 (ties to even); returns float32."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    nan = np.isnan(f)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    out = (r & 0xFFFFFFFF).astype(np.uint32).view(np.float32).copy()
    out[nan] = np.float32("nan")
    return out


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) of values already representable in bf16."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


@dataclass
class Inputs:
    """One batch of GDN-core inputs, as float32 host arrays.

    For bf16 problems every array except ``a`` already holds bf16-representable
    values.  Shapes: q, k [B,T,Nq,d]; v, z [B,T,Nv,dv]; a, beta [B,T,Nv].
    """

    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    a: np.ndarray
    beta: np.ndarray
    z: np.ndarray | None
    dtype: str  # "bf16" or "f32"

    @property
    def shape(self):
        B, T, Nq, d = self.q.shape
        return B, T, Nq, self.v.shape[2], d, self.v.shape[3]


def _softplus(x):
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def numpy_inputs(seed: int, B: int, T: int, Nq: int, Nv: int, d: int = 128,
                 dv: int = 128, dtype: str = "bf16", with_z: bool = False,
                 u_max: float = math.log(4.0), decay_scale: float = 1.0) -> Inputs:
    """Draw one batch; sequence i uses PCG64(seed + i).

    ``decay_scale`` multiplies ``a`` (1/64 gives the slow-decay variant whose
    per-chunk retention stays visible across chunks).
    """
    qs, ks, vs, As, bs, zs = [], [], [], [], [], []
    for i in range(B):
        g = np.random.Generator(np.random.PCG64(seed + i))
        q = g.standard_normal((T, Nq, d))
        k = g.standard_normal((T, Nq, d))
        v = g.standard_normal((T, Nv, dv))
        beta_pre = g.standard_normal((T, Nv))
        a_pre = g.standard_normal((T, Nv))
        u = g.uniform(0.0, u_max, size=(Nv,))
        z = g.standard_normal((T, Nv, dv)) if with_z else None
        q = q / np.linalg.norm(q, axis=-1, keepdims=True)
        k = k / np.linalg.norm(k, axis=-1, keepdims=True)
        beta = 1.0 / (1.0 + np.exp(-beta_pre))
        a = -_softplus(a_pre) * np.exp(u)[None, :] / math.log(2.0) * decay_scale
        qs.append(q); ks.append(k); vs.append(v); As.append(a); bs.append(beta)
        zs.append(z)
    cast = bf16_round if dtype == "bf16" else (lambda x: np.asarray(x, np.float32))
    q = cast(np.stack(qs)); k = cast(np.stack(ks)); v = cast(np.stack(vs))
    beta = cast(np.stack(bs)); a = np.stack(As).astype(np.float32)
    z = cast(np.stack(zs)) if with_z else None
    return Inputs(q=q, k=k, v=v, a=a, beta=beta, z=z, dtype=dtype)


def torch_inputs(seed: int, B: int, T: int, Nq: int, Nv: int, d: int = 128,
                 dv: int = 128, dtype: str = "bf16", with_z: bool = False,
                 u_max: float = math.log(4.0), device: str = "cuda",
                 decay_scale: float = 1.0):
    """Same recipe drawn on ``device`` with a seeded torch generator.

    Returns a dict of device tensors: q, k, v, z (bf16 or fp32), a (fp32),
    beta (same dtype as v).
    """
    import torch

    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    out = {}

    def normal(shape):
        return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)

    q = normal((B, T, Nq, d))
    q = q / q.norm(dim=-1, keepdim=True)
    out["q"] = q.to(tdt)
    del q
    k = normal((B, T, Nq, d))
    k = k / k.norm(dim=-1, keepdim=True)
    out["k"] = k.to(tdt)
    del k
    out["v"] = normal((B, T, Nv, dv)).to(tdt)
    beta_pre = normal((B, T, Nv))
    out["beta"] = torch.sigmoid(beta_pre).to(tdt)
    a_pre = normal((B, T, Nv))
    u = torch.rand((B, 1, Nv), generator=gen, device=device) * u_max
    out["a"] = (-torch.nn.functional.softplus(a_pre) * torch.exp(u)
                / math.log(2.0) * decay_scale).float().contiguous()
    if with_z:
        out["z"] = normal((B, T, Nv, dv)).to(tdt)
    return out


def selector_stats(seed: int, B: int, C: int, Nv: int = 32, ties: bool = False):
    """Synthetic fp32 selection statistics for one batch.

    score [B, Nv, C]: non-negative tail-score-like values with a per-head scale;
    gamma [B, Nv, C]: chunk log2 retentions (<= 0), per-head rate spread over
    four decades so that some heads keep memory across chunks; eta [B, Nv]:
    positive gate energies.  ``ties=True`` puts scores on a coarse grid so that
    equal values (and equal rank keys) are common.
    """
    g = np.random.Generator(np.random.PCG64(seed))
    scale = g.uniform(0.2, 3.0, (B, Nv, 1))
    score = np.abs(g.standard_normal((B, Nv, C))) * scale + g.uniform(0.0, 0.5, (B, Nv, C))
    if ties:
        score = np.round(score * 4.0) / 4.0
    rate = np.exp(g.uniform(math.log(1e-4), math.log(4.0), (B, Nv, 1)))
    gamma = -64.0 * rate * np.abs(1.0 + 0.1 * g.standard_normal((B, Nv, C)))
    eta = g.uniform(0.05, 2.0, (B, Nv))
    return (score.astype(np.float32), gamma.astype(np.float32), eta.astype(np.float32))
