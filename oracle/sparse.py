"""SparseGDN operator in fp64: deferred W, event-sparse H, grouped O.

Test infrastructure only (see the package docstring).

The execution-only devices of the page (CSR scan, gap restore from a log-decay
prefix, compact snapshots, mapped reads; Sec. 2.2) change nothing in the
result, so this oracle evaluates the operator by its plain per-chunk
definition: every chunk is visited in order, skipped events only decay the
state (Sec. 2.6, Eqs. (17)-(18)), and outputs use two-chunk groups
(Sec. 2.7, Eqs. (22)-(24)).  The gap restore (Eq. (21)) and the group/chunk
difference identity (Eq. (25)) are checked against this in the tests.
"""
from __future__ import annotations

import math

import numpy as np

from . import gdn
from .gdn import BS, L, NB
from .selector import gate_energy, select, tail_score


def deferred_w(Cb, kc, solve: str = "blockadj"):
    """W of one chunk from staged coefficients.  Sec. 2.5, Eq. (15).

    Block-adjacent: W_0 = Cb_00 K_0, W_i = Cb_ii K_i + Cb_i,i-1 K_i-1 (block
    rows of 16 tokens).  Exact solve: the full lower-triangular Cb K.
    Cb [..., 64, 64], kc [..., 64, d] -> W [..., 64, d].
    """
    if solve == "exact":
        return Cb @ kc
    W = np.zeros(Cb.shape[:-2] + (L, kc.shape[-1]))
    for i in range(NB):
        ri = slice(i * BS, (i + 1) * BS)
        W[..., ri, :] = Cb[..., ri, ri] @ kc[..., ri, :]
        if i:
            rj = slice((i - 1) * BS, i * BS)
            W[..., ri, :] += Cb[..., ri, rj] @ kc[..., rj, :]
    return W


def sparse_prefill(q, k, v, a, beta, z=None, norm_weight=None, keep_budget=0.29,
                   solve="blockadj", s0=None, mask=None, return_all=False, tail=16,
                   fixed_tiers=False, unit_visibility=False, rank_key=None, tier_rate=None):
    """End-to-end SparseGDN prefill for a batch of sequences.

    Steps (Sec. 2.2 pipeline, Fig. 3): intra (local solve, U, staged Cb,
    tail score) -> selector (mask per head pair) -> H (event-sparse
    propagation) -> O (two-chunk groups).  The statistics handed to the
    selector are rounded to fp32, the precision the page keeps them in.
    ``mask`` [B, Nv/2, C] overrides the selector (then z is not needed).
    ``tail`` is the Tail window of Eq. (9) (8, 16, 32 or 64 rows); the
    selector ablations (``fixed_tiers``, ``unit_visibility``, ``rank_key``
    [B, Nv/2, C]) and the ``tier_rate`` override are those of
    ``selector.select``.

    H, per value head h in pair p (Eqs. (17)-(18) with Eqs. (1)-(2)):
        S_in(c) = S
        z_pc = 1: U'_c = U_c - W_c S,  S <- 2^gamma_c S + K_c^T (U'_c * 2^(gamma_c - g_c))
        z_pc = 0: U'_c = U_c,          S <- 2^gamma_c S
    O, per group r with c = 2r and entry state S_e = S_in(c) (Eqs. (22)-(24)):
        O_c     = d^-1/2 [2^g_c * (Q_c S_e) + A_cc U'_c]
        O_c+1   = d^-1/2 [2^(g_c+1 + gamma_c) * (Q_c+1 S_e) + A_c+1,c U'_c + A_c+1,c+1 U'_c+1]
        A_c+1,c[i,j] = <q_c+1,i, k_c,j> 2^(g_c+1,i + gamma_c - g_c,j)   (no mask)
    A chunk without a partner (odd C, last chunk) forms a one-chunk group.
    """
    q = np.asarray(q, np.float64)
    B, T, Nq, d = q.shape
    v = np.asarray(v, np.float64)
    Nv, dv = v.shape[2], v.shape[3]
    hq = gdn._qk_index(Nq, Nv)
    qc = gdn.chunk_view(q, hq)
    kc = gdn.chunk_view(k, hq)
    vc = gdn.chunk_view(v)
    bc = gdn.chunk_scalar(beta)
    g, gamma, P = gdn.decay_prefix(a)
    C = g.shape[2]
    U, _, Ct, Cb, _ = gdn.intra(kc, vc, bc, g, solve)
    score = tail_score(U, tail).astype(np.float32)
    gamma32 = gamma.astype(np.float32)
    eta = None
    sel = []
    if mask is None:
        if z is None:
            raise ValueError("the selector needs the output gate z")
        eta = gate_energy(z, norm_weight).astype(np.float32)
        sel = [select(score[b], gamma32[b], eta[b], keep_budget, fixed_tiers=fixed_tiers,
                      unit_visibility=unit_visibility,
                      rank_key=None if rank_key is None else rank_key[b],
                      tier_rate=tier_rate) for b in range(B)]
        mask = np.stack([s["mask"] for s in sel])
    mask = np.asarray(mask).astype(bool)
    zh = np.repeat(mask, 2, axis=1)                      # [B, Nv, C] per value head

    scale = 1.0 / math.sqrt(d)
    S = np.zeros((B, Nv, d, dv)) if s0 is None else np.array(s0, np.float64)
    Up = np.empty_like(U)
    G = (C + 1) // 2
    S_entry = np.empty((B, Nv, G, d, dv))                # group entry states S_2r
    S_in = np.empty((B, Nv, C, d, dv)) if return_all else None
    for c in range(C):
        if c % 2 == 0:
            S_entry[:, :, c // 2] = S
        if return_all:
            S_in[:, :, c] = S
        kept = zh[:, :, c][..., None, None]
        Wc = deferred_w(Cb[:, :, c], kc[:, :, c], solve)
        Upc = np.where(kept, U[:, :, c] - Wc @ S, U[:, :, c])
        Up[:, :, c] = Upc
        w = np.exp2(gamma[:, :, c][..., None] - g[:, :, c])
        write = np.swapaxes(kc[:, :, c], -1, -2) @ (Upc * w[..., None])
        S = np.exp2(gamma[:, :, c])[..., None, None] * S + np.where(kept, write, 0.0)

    incl = np.tril(np.ones((L, L), bool))
    full = np.ones((L, L), bool)
    Oc = np.empty((B, Nv, C, L, dv))
    for c0 in range(0, C, 2):
        Se = S_entry[:, :, c0 // 2]
        A00 = (qc[:, :, c0] @ np.swapaxes(kc[:, :, c0], -1, -2)) * \
            gdn._decay_matrix(g[:, :, c0], g[:, :, c0], incl)
        Oc[:, :, c0] = scale * (np.exp2(g[:, :, c0])[..., None] * (qc[:, :, c0] @ Se)
                                + A00 @ Up[:, :, c0])
        c1 = c0 + 1
        if c1 < C:
            gx = g[:, :, c1] + gamma[:, :, c0][..., None]          # g_c+1 + gamma_c
            A10 = (qc[:, :, c1] @ np.swapaxes(kc[:, :, c0], -1, -2)) * \
                gdn._decay_matrix(gx, g[:, :, c0], full)
            A11 = (qc[:, :, c1] @ np.swapaxes(kc[:, :, c1], -1, -2)) * \
                gdn._decay_matrix(g[:, :, c1], g[:, :, c1], incl)
            Oc[:, :, c1] = scale * (np.exp2(gx)[..., None] * (qc[:, :, c1] @ Se)
                                    + A10 @ Up[:, :, c0] + A11 @ Up[:, :, c1])
    o = Oc.transpose(0, 2, 3, 1, 4).reshape(B, C * L, Nv, dv)[:, :T]
    if return_all:
        return o, S, dict(U=U, Up=Up, Ct=Ct, Cb=Cb, g=g, gamma=gamma, P=P, score=score,
                          eta=eta, mask=mask.astype(np.uint8), sel=sel, S_in=S_in,
                          qc=qc, kc=kc)
    return o, S
