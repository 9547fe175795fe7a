"""SparseGDN selector in fp64: scores, budgets, dynamic tiers, CSR layout.

Test infrastructure only (see the package docstring).

Everything that feeds an integer decision follows the evaluation rules of
``oracle.detfp`` (binary64, fixed summation order, no FMA).  Inputs are the
fp32 selection statistics (the page keeps selection statistics in FP32,
Sec. 3.1): tail scores s [Nv, C], chunk log2 retentions gamma [Nv, C] and gate
energies eta [Nv], for one sequence.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

from .detfp import csum, exp2, powi
from .gdn import L

RATES_PCT = (8, 30, 95)                 # (rho_L, rho_M, rho_H), Sec. 2.4.3, Eq. (13)
DEFAULT_BUDGET_BP = 2900                # the page's default: about 29% of events
MEDIUM_CHOICES = {1: (11, 12, 13), 2: (7, 8, 9), 3: (3, 4, 5), 4: (0,)}   # Sec. 2.4.3 table
HIGH_CHOICES = (1, 2, 3, 4)
FIXED_HIGH, FIXED_MEDIUM = 3, 4   # the fixed 9 Low / 4 Medium / 3 High split of Table 5
LOW, MEDIUM, HIGH = 0, 1, 2


# ---------------------------------------------------------------------------
# statistics
# ---------------------------------------------------------------------------

def tail_score(U, tail: int = 16):
    """s_{c,h} = ||U_{c,h}[64-tail:64, :]||_F.  Sec. 2.4, Eq. (9).

    U: [..., C, 64, dv] (the transformed values before the state correction).
    """
    U = np.asarray(U, np.float64)
    return np.sqrt(np.sum(U[..., L - tail:, :] ** 2, axis=(-1, -2)))


def gate_energy(z, norm_weight=None):
    """eta_h: mean square of w_v * SiLU(z) at sampled gate positions.

    Sec. 2.4, Eq. (11): in every chunk c the gate is sampled at positions
    8, 24, 40, 56 (a = 0..3), each sample reading the single coordinate
    v = 73 (4c + a) mod dv; SiLU(x) = x / (1 + e^-x); w is the learned
    RMSNorm scale (ones when not given).  The mean runs over the 4C samples.
    Positions past T (padded chunk) read z = 0.
    z: [B, T, Nv, dv] -> eta [B, Nv].
    """
    z = np.asarray(z, np.float64)
    B, T, Nv, dv = z.shape
    C = -(-T // L)
    w = np.ones(dv) if norm_weight is None else np.asarray(norm_weight, np.float64)
    cc, aa = np.meshgrid(np.arange(C), np.arange(4), indexing="ij")
    pos = (L * cc + 8 + 16 * aa).ravel()
    coord = ((73 * (4 * cc + aa)) % dv).ravel()
    valid = pos < T
    zs = np.zeros((B, pos.size, Nv))
    zs[:, valid, :] = z[:, pos[valid], :, coord[valid]].transpose(1, 0, 2)
    silu = zs / (1.0 + np.exp(-zs))
    vals = w[coord][None, :, None] * silu
    return np.mean(vals ** 2, axis=1)


# ---------------------------------------------------------------------------
# budgets
# ---------------------------------------------------------------------------

def budget_bp(keep_budget: float) -> int:
    """Keep budget in basis points: floor(b * 10000 + 0.5) in binary64, with b
    first rounded to binary32 (the precision in which a caller hands it over)."""
    return int(math.floor(float(np.float32(keep_budget)) * 10000.0 + 0.5))


def tier_counts(C: int, keep_budget: float = 0.29, tier_rate=None):
    """(k_L, k_M, k_H) = clip(round(rho_l C), 2, C).  Sec. 2.4.3, Eq. (13).

    round() is half away from zero on the exact rational rho_l * C.  At the
    default budget (0.29) rho = (0.08, 0.30, 0.95).  Other budgets re-scale the
    rates (the page re-selects tiers per budget point without giving the map;
    reading used here): b <= 0.29: rho(b) = rho * b / 0.29;
    b > 0.29: rho(b) = 1 - (1 - rho)(1 - b) / 0.71.  C = 1 keeps the only chunk.

    tier_rate = (rho_L, rho_M, rho_H) overrides the budget's rates; each is
    taken in basis points (floor(rho * 10000 + 0.5)), must lie in (0, 1] and
    must not decrease from Low to High.
    """
    if tier_rate is not None:
        rbp = [budget_bp(r) for r in tier_rate]
        if len(rbp) != 3 or not all(1 <= r <= 10000 and 0.0 < float(x) <= 1.0
                                    for r, x in zip(rbp, tier_rate)):
            raise ValueError("tier rates must lie in (0, 1]")
        if not rbp[0] <= rbp[1] <= rbp[2]:
            raise ValueError("tier rates must not decrease from Low to High")
        if C == 1:
            return (1, 1, 1)
        out = []
        for r in rbp:
            x = Fraction(r * C, 10000)
            k = math.floor(x + Fraction(1, 2))
            out.append(min(max(k, 2), C))
        return tuple(out)
    bp = budget_bp(keep_budget)
    if not 1 <= bp <= 10000:
        raise ValueError("keep budget must lie in (0, 1]")
    if C == 1:
        return (1, 1, 1)
    out = []
    for pct in RATES_PCT:
        if bp <= DEFAULT_BUDGET_BP:
            num, den = pct * bp * C, 100 * DEFAULT_BUDGET_BP
        else:
            num = C * (710000 - (100 - pct) * (10000 - bp))
            den = 710000
        k = (2 * num + den) // (2 * den)
        out.append(min(max(k, 2), C))
    return tuple(out)


def nominal_keep(n_high: int, n_medium: int, n_pairs: int = 16) -> float:
    """Nominal event keep of a tier split at the default rates."""
    n_low = n_pairs - n_high - n_medium
    return (n_high * 0.95 + n_medium * 0.30 + n_low * 0.08) / n_pairs


# ---------------------------------------------------------------------------
# the selector
# ---------------------------------------------------------------------------

def split_score(xs, k: int) -> float:
    """B(x, k) = k (n-k) / n * (mean(x[:k]) - mean(x[k:]))^2.  Sec. 2.4.3, Eq. (14).

    xs is sorted in descending order.  k = 0 or k = n gives 0.
    """
    n = len(xs)
    if k <= 0 or k >= n:
        return 0.0
    m1 = csum(xs[:k]) / k
    m2 = csum(xs[k:]) / (n - k)
    f = float(k * (n - k)) / n
    dm = m1 - m2
    return f * (dm * dm)


def lifetime(r: float, C: int) -> float:
    """L_h = sum_{j=1}^{C-2} r^j.  Sec. 2.4, Eq. (11).

    Evaluated in closed form r (1 - r^n) / (1 - r) with n = C - 2 (r^n by
    ``powi``); r = 1 gives n; C <= 2 gives 0.
    """
    n = C - 2
    if n <= 0:
        return 0.0
    if r == 1.0:
        return float(n)
    return r * (1.0 - powi(r, n)) / (1.0 - r)


def _ord(x: float) -> float:
    """Ordering key of a binary64 value: NaN counts as -infinity (a reading:
    the page's orderings assume finite statistics; this keeps every ranking a
    total order when a non-finite input reaches them)."""
    return -math.inf if x != x else x


def _argmax_first(values):
    best, bi = None, 0
    for i, x in enumerate(values):
        if best is None or x > best:
            best, bi = x, i
    return bi


def _normalise(d):
    mu = csum(d) / len(d)
    return [x / mu if mu > 0.0 else 0.0 for x in d]


def select(score, gamma, eta, keep_budget: float = 0.29, window: int = 16,
           fixed_tiers: bool = False, unit_visibility: bool = False, rank_key=None,
           tier_rate=None):
    """Dynamic event selection for one sequence.  Sec. 2.4, Eqs. (10)-(14).

    score, gamma: [Nv, C] (fp32 values); eta: [Nv].  Nv = 32 (16 head pairs;
    the tier table is written for 16 pairs).  Returns a dict with
    mask [16, C] (uint8), tier [16] (0 Low, 1 Medium, 2 High), k (k_L, k_M, k_H),
    n_high, n_medium, rank [16, C] (-1 for anchors), and the intermediate
    statistics (norms, r, L, G, gains, x).

    Selector ablations (Sec. 3.5, Table 5; the speed side of each):
      fixed_tiers      3 High / 4 Medium / 9 Low pairs in every layer instead of
                       the split-score counts of Eqs. (13)-(14); which pairs get
                       which tier still follows x_H, then x_M.
      unit_visibility  G_h = 1 for every head (the gate energy is ignored).
      rank_key [16, C] the non-anchor chunks kept in each pair are the ones with
                       the largest keys (ties: lower chunk first) instead of the
                       largest q_c; the tiers and the keep counts are still the
                       adaptive ones (random keys give the random selection at
                       matched budget).
    tier_rate          (rho_L, rho_M, rho_H) in place of the budget's rates
                       (see tier_counts).
    """
    s = np.asarray(score, np.float32).astype(np.float64)
    gm = np.asarray(gamma, np.float32).astype(np.float64)
    et = np.asarray(eta, np.float32).astype(np.float64)
    Nv, C = s.shape
    if Nv != 32:
        raise ValueError("the tier table is defined for 16 head pairs (Nv = 32)")
    Np = Nv // 2
    kL, kM, kH = tier_counts(C, keep_budget, tier_rate)

    # Eq. (10): per-head chunk norm and within-pair rank key.
    norms = [math.sqrt(csum([x * x for x in s[h].tolist()])) for h in range(Nv)]
    rank = np.full((Np, C), -1, dtype=np.int64)
    for p in range(Np):
        h0, h1 = 2 * p, 2 * p + 1
        qv = []
        for c in range(C):
            t0 = s[h0, c] / norms[h0] if norms[h0] > 0.0 else 0.0
            t1 = s[h1, c] / norms[h1] if norms[h1] > 0.0 else 0.0
            qv.append(_ord(0.5 * (t0 + t1)))
        cand = sorted(range(1, C - 1), key=lambda c: (-qv[c], c))
        for r, c in enumerate(cand):
            rank[p, c] = r

    # Eq. (11): memory lifetime and output visibility.
    lo = max(0, C - window)
    r_h = [csum([exp2(gm[h, c]) for c in range(lo, C)]) / (C - lo) for h in range(Nv)]
    L_h = [lifetime(r, C) for r in r_h]
    eta_bar = csum(et.tolist()) / Nv
    G_h = [math.sqrt(et[h] / eta_bar) if eta_bar > 0.0 else 1.0 for h in range(Nv)]
    if unit_visibility:
        G_h = [1.0] * Nv

    # Eq. (12): upgrade gains L->M and M->H, unnormalised s.
    def band_sum(h, p, lo_k, hi_k):
        return csum([s[h, c] if (lo_k - 2 <= rank[p, c] < hi_k - 2) else 0.0
                     for c in range(C)])

    gain_lm, gain_mh = [], []
    for p in range(Np):
        h0, h1 = 2 * p, 2 * p + 1
        gain_lm.append((L_h[h0] * G_h[h0]) * band_sum(h0, p, kL, kM)
                       + (L_h[h1] * G_h[h1]) * band_sum(h1, p, kL, kM))
        gain_mh.append((L_h[h0] * G_h[h0]) * band_sum(h0, p, kM, kH)
                       + (L_h[h1] * G_h[h1]) * band_sum(h1, p, kM, kH))

    # Eqs. (13)-(14): normalised gains, High count first, then Medium.
    xM = [_ord(x) for x in _normalise(gain_lm)]
    xH = [_ord(x) for x in _normalise(gain_mh)]
    order_h = sorted(range(Np), key=lambda p: (-xH[p], p))
    vals_h = [xH[p] for p in order_h]
    if fixed_tiers:
        n_high = FIXED_HIGH
    else:
        n_high = HIGH_CHOICES[_argmax_first([split_score(vals_h, k) for k in HIGH_CHOICES])]
    high = set(order_h[:n_high])
    rest = [p for p in range(Np) if p not in high]
    order_m = sorted(rest, key=lambda p: (-xM[p], p))
    vals_m = [xM[p] for p in order_m]
    if fixed_tiers:
        n_medium = FIXED_MEDIUM
    else:
        choices = MEDIUM_CHOICES[n_high]
        n_medium = choices[_argmax_first([split_score(vals_m, k) for k in choices])]
    medium = set(order_m[:n_medium])

    tier = np.array([HIGH if p in high else MEDIUM if p in medium else LOW
                     for p in range(Np)], dtype=np.uint8)
    kk = {LOW: kL, MEDIUM: kM, HIGH: kH}
    keep_rank = rank
    if rank_key is not None:
        key = np.asarray(rank_key, np.float32).astype(np.float64)
        keep_rank = np.full((Np, C), -1, dtype=np.int64)
        for p in range(Np):
            cand = sorted(range(1, C - 1), key=lambda c: (-_ord(key[p, c]), c))
            for r, c in enumerate(cand):
                keep_rank[p, c] = r
    mask = np.zeros((Np, C), dtype=np.uint8)
    for p in range(Np):
        k = kk[int(tier[p])]
        for c in range(C):
            if c == 0 or c == C - 1 or (0 <= keep_rank[p, c] < k - 2):
                mask[p, c] = 1
    return dict(mask=mask, tier=tier, k=(kL, kM, kH), n_high=n_high,
                n_medium=n_medium, rank=rank, norms=norms, r=r_h, L=L_h, G=G_h,
                gain_lm=gain_lm, gain_mh=gain_mh, x_m=xM, x_h=xH)


# ---------------------------------------------------------------------------
# CSR event layout
# ---------------------------------------------------------------------------

def event_layout(mask, tier):
    """CSR layout of the kept events of one sequence.  Sec. 2.4.3, Eq. (16).

    Rows are head pairs ordered High, then Medium, then Low (ascending pair
    index within a tier); each row lists its kept chunks in ascending time.
    pred[p, r] is the last kept event of pair p before group r's first chunk
    2r (or -1).  Snapshot slots number the distinct referenced predecessor
    events in (row, chunk) order.  Returns dict(row_pair, row_ptr, col, E,
    pred [16, G], group_slot [16, G], event_slot [E], n_snap).
    """
    mask = np.asarray(mask).astype(bool)
    tier = np.asarray(tier)
    Np, C = mask.shape
    G = (C + 1) // 2
    rows = [p for t in (HIGH, MEDIUM, LOW) for p in range(Np) if int(tier[p]) == t]
    row_ptr = [0]
    col = []
    for p in rows:
        col.extend(c for c in range(C) if mask[p, c])
        row_ptr.append(len(col))
    pred = np.full((Np, G), -1, dtype=np.int64)
    for p in range(Np):
        last = -1
        for r in range(G):
            for e in range(max(0, 2 * r - 2), 2 * r):
                if mask[p, e]:
                    last = e
            pred[p, r] = last
    slot_of = {}
    for p in rows:
        for e in sorted({int(x) for x in pred[p] if x >= 0}):
            slot_of[(p, e)] = len(slot_of)
    group_slot = np.array([[slot_of.get((p, int(pred[p, r])), -1) for r in range(G)]
                           for p in range(Np)], dtype=np.int64)
    event_slot = []
    for i, p in enumerate(rows):
        for j in range(row_ptr[i], row_ptr[i + 1]):
            event_slot.append(slot_of.get((p, col[j]), -1))
    return dict(row_pair=np.array(rows, np.int64), row_ptr=np.array(row_ptr, np.int64),
                col=np.array(col, np.int64), E=len(col), pred=pred,
                group_slot=group_slot, event_slot=np.array(event_slot, np.int64),
                n_snap=len(slot_of))
