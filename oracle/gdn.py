"""Dense GDN core in fp64: the token recurrence and the chunk form.

Test infrastructure only (see the package docstring).

Conventions (all arrays float64):
  q, k : [B, T, Nq, d]     v : [B, T, Nv, dv]     a, beta : [B, T, Nv]
  value head h reads query/key head h // (Nv // Nq)
  a    : per-token log2 retention (a <= 0), alpha_t = 2**a_t
  s0   : optional initial state [B, Nv, d, dv] (zero when None)
Outputs o [B, T, Nv, dv] and the final state S [B, Nv, d, dv].
"""
from __future__ import annotations

import math

import numpy as np

L = 64          # chunk length (Sec. 2.1)
NB = 4          # 16-token blocks per chunk (Sec. 2.3)
BS = L // NB


def _qk_index(Nq: int, Nv: int) -> np.ndarray:
    return np.arange(Nv) // (Nv // Nq)


def recurrence(q, k, v, a, beta, s0=None):
    """Token-by-token gated delta rule: the plain definition of the operator.

    For every token t and value head h (state S is d x dv):
        S   <- 2**a_t * S                   (gate: decay first)
        u_t  = beta_t * (v_t - S^T k_t)     (delta-rule residual)
        S   <- S + k_t u_t^T                (write)
        o_t  = S^T q_t / sqrt(d)            (read after the write)
    Unrolling this inside a 64-token chunk gives exactly Sec. 2.1,
    Eqs. (1)-(4) with the local system of Sec. 2.3, Eqs. (5)-(6): the
    in-chunk log-decay g is inclusive of position i, and the output mask of
    Eq. (4) keeps j <= i.
    """
    q = np.asarray(q, np.float64); k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64); a = np.asarray(a, np.float64)
    beta = np.asarray(beta, np.float64)
    B, T, Nq, d = q.shape
    Nv, dv = v.shape[2], v.shape[3]
    hq = _qk_index(Nq, Nv)
    S = np.zeros((B, Nv, d, dv)) if s0 is None else np.array(s0, np.float64)
    o = np.empty((B, T, Nv, dv))
    scale = 1.0 / math.sqrt(d)
    for t in range(T):
        kt = k[:, t][:, hq]                       # [B, Nv, d]
        qt = q[:, t][:, hq]
        S *= np.exp2(a[:, t])[:, :, None, None]
        pred = np.einsum("bhd,bhde->bhe", kt, S)
        u = beta[:, t][:, :, None] * (v[:, t] - pred)
        S += kt[:, :, :, None] * u[:, :, None, :]
        o[:, t] = np.einsum("bhd,bhde->bhe", qt, S) * scale
    return o, S


def decode_step(q, k, v, a, beta, s):
    """One token of the recurrence per sequence: the decode step that follows a
    prefill, whose final state S_{C,h} is handed to autoregressive decoding
    (Sec. 2.6); the step is the per-token rule of `recurrence`.

    q, k [B, Nq, d]; v [B, Nv, dv]; a, beta [B, Nv]; s [B, Nv, d, dv].
    Returns o [B, Nv, dv] and the new state.
    """
    o, S = recurrence(np.asarray(q)[:, None], np.asarray(k)[:, None], np.asarray(v)[:, None],
                      np.asarray(a)[:, None], np.asarray(beta)[:, None], s)
    return o[:, 0], S


# ---------------------------------------------------------------------------
# chunk form
# ---------------------------------------------------------------------------

def pad_to_chunks(x: np.ndarray, axis: int = 1) -> np.ndarray:
    """Zero-pad the token axis to a multiple of 64.

    Reading of the page for T % 64 != 0 (it sets C = ceil(T/64) in Sec. 2.4):
    padded tokens have a = 0, beta = 0 and q = k = v = 0, so they neither decay
    nor write the state, and their outputs are discarded.
    """
    T = x.shape[axis]
    C = -(-T // L)
    pad = C * L - T
    if pad == 0:
        return x
    widths = [(0, 0)] * x.ndim
    widths[axis] = (0, pad)
    return np.pad(x, widths)


def decay_prefix(a):
    """In-chunk inclusive log2 decay g, chunk retention gamma and prefix P.

    g[c, i] = sum_{i' <= i} a[64c + i']   (Sec. 2.1, symbol table)
    gamma_c = g[c, 63]                    (Sec. 2.1)
    P_0 = 0, P_{c+1} = sum_{j <= c} gamma_j   (Sec. 2.6, Eqs. (19)-(20))
    a: [B, T, Nv] -> g [B, Nv, C, 64], gamma [B, Nv, C], P [B, Nv, C+1].
    """
    a = pad_to_chunks(np.asarray(a, np.float64))
    B, Tp, Nv = a.shape
    C = Tp // L
    ac = a.reshape(B, C, L, Nv).transpose(0, 3, 1, 2)     # [B, Nv, C, L]
    g = np.cumsum(ac, axis=-1)
    gamma = g[..., L - 1].copy()
    P = np.concatenate([np.zeros((B, Nv, 1)), np.cumsum(gamma, axis=-1)], axis=-1)
    return g, gamma, P


def chunk_view(x, Nv_index=None):
    """[B, T, H, e] -> [B, H, C, 64, e] after zero padding."""
    x = pad_to_chunks(np.asarray(x, np.float64))
    B, Tp, H, e = x.shape
    xc = x.reshape(B, Tp // L, L, H, e).transpose(0, 3, 1, 2, 4)
    if Nv_index is not None:
        xc = xc[:, Nv_index]
    return xc


def chunk_scalar(x):
    """[B, T, Nv] -> [B, Nv, C, 64] after zero padding."""
    x = pad_to_chunks(np.asarray(x, np.float64))
    B, Tp, Nv = x.shape
    return x.reshape(B, Tp // L, L, Nv).transpose(0, 3, 1, 2)


def _decay_matrix(gi, gj, mask):
    """2**(gi[:,None] - gj[None,:]) where mask, else 0.

    The exponent is selected before exp2, so entries outside the mask (whose
    exponent may be large and positive) never produce inf * 0.
    """
    diff = gi[..., :, None] - gj[..., None, :]
    return np.where(mask, np.exp2(np.where(mask, diff, 0.0)), 0.0)


def local_system(kc, betac, gc):
    """M = I + A_Delta with A_Delta[t,s] = beta_t <k_t,k_s> 2^(g_t-g_s) [s<t].

    Sec. 2.3, Eq. (5).  kc [..., 64, d], betac and gc [..., 64].
    """
    strict = np.tril(np.ones((L, L), bool), -1)
    G = kc @ np.swapaxes(kc, -1, -2)
    A = betac[..., :, None] * G * _decay_matrix(gc, gc, strict)
    return np.eye(L) + A


def invert_unit_lower(M):
    """Inverse of a unit lower-triangular matrix by forward substitution.

    Row t of X = M^{-1} satisfies X[t] = e_t - sum_{s<t} M[t,s] X[s].
    Works on [..., n, n] batches.
    """
    n = M.shape[-1]
    X = np.zeros_like(M)
    for t in range(n):
        if t:
            X[..., t, :] = -np.einsum("...s,...sj->...j", M[..., t, :t], X[..., :t, :])
        X[..., t, t] += 1.0
    return X


def block_adjacent_inverse(M):
    """The 7-block approximation C of M^{-1}.  Sec. 2.3, Eqs. (7)-(8).

    Blocks are 16 x 16; kept set B = {(i,i)} U {(i,i-1)}:
        C_ii     = M_ii^{-1}
        C_i,i-1  = -C_ii M_i,i-1 C_i-1,i-1
    all other blocks are zero.
    """
    C = np.zeros_like(M)

    def blk(X, i, j):
        return X[..., i * BS:(i + 1) * BS, j * BS:(j + 1) * BS]

    for i in range(NB):
        C[..., i * BS:(i + 1) * BS, i * BS:(i + 1) * BS] = invert_unit_lower(blk(M, i, i))
    for i in range(1, NB):
        C[..., i * BS:(i + 1) * BS, (i - 1) * BS:i * BS] = \
            -blk(C, i, i) @ blk(M, i, i - 1) @ blk(C, i - 1, i - 1)
    return C


def solve_coefficients(kc, betac, gc, solve: str):
    """C ~ M^{-1}: exact inverse ("exact") or the 7-block form ("blockadj")."""
    M = local_system(kc, betac, gc)
    if solve == "exact":
        return invert_unit_lower(M)
    if solve == "blockadj":
        return block_adjacent_inverse(M)
    raise ValueError(solve)


def intra(kc, vc, betac, gc, solve: str):
    """Local solve of one chunk batch.  Sec. 2.3, Eqs. (5)-(8).

    Returns U = C diag(beta) V, W = C diag(beta * 2^g) K, the weighted
    coefficients Ct = C diag(beta) and Cb = C diag(beta * 2^g), and C.
    """
    C = solve_coefficients(kc, betac, gc, solve)
    Ct = C * betac[..., None, :]
    Cb = C * (betac * np.exp2(gc))[..., None, :]
    return Ct @ vc, Cb @ kc, Ct, Cb, C


def chunk_prefill(q, k, v, a, beta, s0=None, solve: str = "exact", return_all=False):
    """Chunk form of the dense operator.  Sec. 2.1, Eqs. (1)-(4).

    Per chunk c and value head:
        U'      = U - W S_c                                      (1)
        S_{c+1} = 2^gamma S_c + K^T (U' * 2^(gamma - g))         (2)
        O       = d^-1/2 [2^g * (Q S_c) + A U']                  (3)
        A[i,j]  = <q_i,k_j> 2^(g_i - g_j) [j <= i]               (4)
    with U, W from the local solve (exact or block-adjacent).
    """
    q = np.asarray(q, np.float64)
    B, T, Nq, d = q.shape
    Nv = np.asarray(v).shape[2]
    hq = _qk_index(Nq, Nv)
    qc = chunk_view(q, hq)                  # [B, Nv, C, 64, d]
    kc = chunk_view(k, hq)
    vc = chunk_view(v)
    bc = chunk_scalar(beta)
    g, gamma, P = decay_prefix(a)
    C = g.shape[2]
    U, W, Ct, Cb, Cm = intra(kc, vc, bc, g, solve)
    incl = np.tril(np.ones((L, L), bool))
    A = (qc @ np.swapaxes(kc, -1, -2)) * _decay_matrix(g, g, incl)
    dv = vc.shape[-1]
    S = np.zeros((B, Nv, d, dv)) if s0 is None else np.array(s0, np.float64)
    Oc = np.empty((B, Nv, C, L, dv))
    Up = np.empty_like(U)
    states = np.empty((B, Nv, C, d, dv)) if return_all else None
    scale = 1.0 / math.sqrt(d)
    for c in range(C):
        if return_all:
            states[:, :, c] = S
        Upc = U[:, :, c] - W[:, :, c] @ S
        Up[:, :, c] = Upc
        Oc[:, :, c] = scale * (np.exp2(g[:, :, c])[..., None] * (qc[:, :, c] @ S)
                               + A[:, :, c] @ Upc)
        w = np.exp2(gamma[:, :, c][..., None] - g[:, :, c])     # 2^(gamma - g)
        S = np.exp2(gamma[:, :, c])[..., None, None] * S + \
            np.swapaxes(kc[:, :, c], -1, -2) @ (Upc * w[..., None])
    o = Oc.transpose(0, 2, 3, 1, 4).reshape(B, C * L, Nv, dv)[:, :T]
    if return_all:
        return o, S, dict(U=U, W=W, Up=Up, Ct=Ct, Cb=Cb, C=Cm, g=g, gamma=gamma,
                          P=P, states=states, A=A)
    return o, S
