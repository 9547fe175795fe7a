"""Pins of the selector oracle (oracle.selector, oracle.detfp).  CPU only."""
import json
import math
import os

import numpy as np
import pytest

from oracle import detfp, selector

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "printed_values.json")))


# ---------------------------------------------------------------- detfp

def test_csum_accuracy_and_exact_cases():
    rng = np.random.default_rng(0)
    for n in (1, 5, 63, 64, 65, 1000, 2048):
        xs = rng.standard_normal(n).tolist()
        ref = math.fsum(xs)
        assert abs(detfp.csum(xs) - ref) <= 1e-14 * max(1.0, sum(abs(x) for x in xs))
    ints = [float(i) for i in range(-500, 700)]
    assert detfp.csum(ints) == sum(ints)
    assert detfp.csum([]) == 0.0


def test_exp2_matches_libm():
    rng = np.random.default_rng(1)
    xs = np.concatenate([rng.uniform(-1100, 60, 4000), rng.uniform(-2, 2, 2000),
                         np.arange(-1070, 60, dtype=float)])
    for x in xs:
        r = detfp.exp2(float(x))
        ref = 2.0 ** float(x)
        if ref == 0.0 or ref < 2.2250738585072014e-308:
            assert abs(r - ref) <= 2 * 5e-324
        else:
            assert abs(r - ref) <= 4.5e-16 * ref, (x, r, ref)
    for n in range(-1074, 1001, 7):
        assert detfp.exp2(float(n)) == math.ldexp(1.0, n)
    assert detfp.exp2(-3.0e38) == 0.0


def test_powi_matches_pow():
    for r in (0.0, 0.5, 0.9, 0.999, 1.0, 1e-3):
        for n in (0, 1, 2, 3, 7, 62, 510, 2046):
            ref = r ** n
            got = detfp.powi(r, n)
            assert got == ref or abs(got - ref) <= 1e-13 * abs(ref)


# ---------------------------------------------------------------- budgets

def test_rates_and_table_match_page():
    assert [p / 100 for p in selector.RATES_PCT] == GOLD["tier_rates"]["rho"]
    table = {int(k): tuple(v) for k, v in GOLD["tier_table"]["medium_choices"].items()}
    assert table == selector.MEDIUM_CHOICES


@pytest.mark.parametrize("C,expect", [
    (1, (1, 1, 1)), (2, (2, 2, 2)), (4, (2, 2, 4)), (35, (3, 11, 33)),
    (64, (5, 19, 61)), (512, (41, 154, 486)), (2048, (164, 614, 1946))])
def test_tier_counts_default(C, expect):
    """k = clip(round(rho C), 2, C), round half away from zero on exact decimals
    (C = 35: 0.30 * 35 = 10.5 -> 11)."""
    assert selector.tier_counts(C) == expect


def test_tier_counts_other_budgets():
    assert selector.tier_counts(512, 1.0) == (512, 512, 512)
    # b = 0.15 <= 0.29: rho * 15/29; 0.08*512*15/29 = 21.19 -> 21, 0.30 -> 79.4 -> 79, 0.95 -> 251.6 -> 252
    assert selector.tier_counts(512, 0.15) == (21, 79, 252)
    # b = 0.5: 1 - (1 - rho) * 0.5 / 0.71: 0.08 -> 0.3521*512 = 180.3 -> 180
    assert selector.tier_counts(512, 0.5) == (180, 260, 494)
    with pytest.raises(ValueError):
        selector.tier_counts(512, 0.0)


@pytest.mark.parametrize("C", [1, 2, 4, 35, 64, 512, 2048])
def test_tier_rate_override_at_page_rates_is_default(C):
    """Overriding with the page's own rates (0.08, 0.30, 0.95) gives the
    default budget's counts (Sec. 2.4.3, Eq. (13))."""
    assert selector.tier_counts(C, 0.5, tier_rate=(0.08, 0.30, 0.95)) == selector.tier_counts(C)


def test_tier_rate_override_hand_values():
    # 0.1 * 35 = 3.5 -> 4, 0.25 * 35 = 8.75 -> 9, 0.5 * 35 = 17.5 -> 18 (halves up)
    assert selector.tier_counts(35, tier_rate=(0.1, 0.25, 0.5)) == (4, 9, 18)
    assert selector.tier_counts(100, tier_rate=(0.1, 0.25, 0.5)) == (10, 25, 50)
    # 0.01 * 64 = 0.64 -> 1, clipped to the two anchors
    assert selector.tier_counts(64, tier_rate=(0.01, 0.01, 1.0)) == (2, 2, 64)
    # the keep budget is not used once rates are given
    assert selector.tier_counts(100, 1.0, tier_rate=(0.1, 0.25, 0.5)) == (10, 25, 50)
    for bad in [(0.3, 0.2, 0.9), (0.0, 0.3, 0.9), (0.1, 0.3, 1.5), (float("nan"), 0.3, 0.9),
                (-0.1, 0.3, 0.9)]:
        with pytest.raises(ValueError):
            selector.tier_counts(64, tier_rate=bad)


def test_select_with_tier_rate_keeps_k_per_tier():
    """With overridden rates every pair keeps exactly k of its tier, anchors
    included (Sec. 2.4.3, Eqs. (13)-(14))."""
    rng = np.random.default_rng(5)
    C = 96
    score = rng.gamma(2.0, 1.0, (32, C)).astype(np.float32)
    gamma = (-rng.uniform(0.1, 3.0, (32, 1)) * np.ones((1, C))).astype(np.float32)
    eta = rng.uniform(0.5, 2.0, 32).astype(np.float32)
    rates = (0.05, 0.2, 0.6)
    out = selector.select(score, gamma, eta, tier_rate=rates)
    k = selector.tier_counts(C, tier_rate=rates)
    assert out["k"] == k
    for p in range(16):
        assert int(out["mask"][p].sum()) == k[int(out["tier"][p])]
        assert out["mask"][p, 0] == 1 and out["mask"][p, C - 1] == 1


def test_nominal_keep_range_matches_page():
    """The candidate table bounds the nominal mean keep to 28.44%-31.31%."""
    vals = [selector.nominal_keep(h, m) for h, ms in selector.MEDIUM_CHOICES.items() for m in ms]
    g = GOLD["nominal_keep_range"]
    assert round(100 * min(vals), 2) == g["low_percent"]
    assert round(100 * max(vals), 2) == g["high_percent"]
    assert min(vals) == pytest.approx(0.284375, abs=1e-15)
    assert max(vals) == pytest.approx(0.313125, abs=1e-15)


# ---------------------------------------------------------------- statistics

def test_split_score_is_between_group_sum_of_squares():
    rng = np.random.default_rng(2)
    for _ in range(50):
        n = int(rng.integers(2, 17))
        x = sorted(rng.uniform(0, 3, n).tolist(), reverse=True)
        for k in range(0, n + 1):
            a, b = x[:k], x[k:]
            tot = sum((t - np.mean(x)) ** 2 for t in x)
            within = (sum((t - np.mean(a)) ** 2 for t in a) if a else 0.0) + \
                     (sum((t - np.mean(b)) ** 2 for t in b) if b else 0.0)
            assert selector.split_score(x, k) == pytest.approx(tot - within, abs=1e-10)


def test_lifetime_equals_geometric_sum():
    for C in (1, 2, 3, 4, 64, 512, 2048):
        for r in (0.0, 1e-20, 0.3, 0.9, 0.99999, 1.0):
            ref = math.fsum(r ** j for j in range(1, C - 1))
            got = selector.lifetime(r, C)
            assert got == pytest.approx(ref, rel=1e-9, abs=1e-300)


def test_tail_score_reads_only_the_last_16_rows():
    U = np.zeros((3, 64, 128))
    U[1, 50, 3] = -2.5
    U[1, 47, :] = 100.0          # row 47 is outside the tail window
    U[2, 48:64, 0] = 1.0          # 16 ones -> sqrt(16) = 4
    s = selector.tail_score(U)
    np.testing.assert_array_equal(s, [0.0, 2.5, 4.0])


@pytest.mark.parametrize("tail", [8, 16, 32, 64])
def test_tail_score_windows(tail):
    """Tail-8/32/64 ablation windows (Fig. 10): row r of the chunk holds r + 1
    in one column, so the score is sqrt(sum of (r + 1)^2 over the last rows)."""
    U = np.zeros((1, 64, 128))
    U[0, :, 5] = np.arange(1, 65)
    expect = math.sqrt(sum((r + 1) ** 2 for r in range(64 - tail, 64)))
    assert selector.tail_score(U, tail)[0] == pytest.approx(expect, rel=1e-15)


def _silu(x):
    return x / (1 + math.exp(-x))


def test_gate_energy_samples_fixed_positions_and_rotating_coordinate():
    gold = GOLD["gate_samples"]
    T, Nv, dv = 64 * 3, 2, 128
    z = np.zeros((1, T, Nv, dv))
    # chunk 1, sample a = 2: position 64 + 40, coordinate 73 * 6 mod 128 = 54
    z[0, 64 + gold["positions"][2], 0, (gold["stride"] * 6) % dv] = 3.0
    # a value next to it (not sampled) changes nothing
    z[0, 64 + 41, 0, 54] = 50.0
    z[0, 64 + 40, 0, 55] = 50.0
    eta = selector.gate_energy(z)
    assert eta[0, 0] == pytest.approx(_silu(3.0) ** 2 / 12, rel=1e-14)
    assert eta[0, 1] == 0.0


def test_gate_energy_visits_every_coordinate_once_per_32_chunks():
    """gcd(73, 128) = 1: 128 consecutive samples read each coordinate once, so a
    gate constant over time gives eta = mean_v (w_v SiLU(f_v))^2."""
    T, dv = 64 * 32, 128
    f = np.linspace(-3, 3, dv)
    w = np.linspace(0.5, 1.5, dv)
    z = np.broadcast_to(f, (1, T, 1, dv)).copy()
    eta = selector.gate_energy(z, w)
    expect = np.mean([(w[v] * _silu(f[v])) ** 2 for v in range(dv)])
    assert eta[0, 0] == pytest.approx(expect, rel=1e-13)


# ---------------------------------------------------------------- selector

def _crafted(C=64):
    """Pair profiles with hand-derivable decisions.

    Every head's score is A_p on chunks [0, k_M - 1) and B_p after, A_p > B_p,
    so ranks follow time, the L->M band lies in the A region and the M->H band
    in the B region: gain_LM ~ A_p, gain_MH ~ B_p.
    B = [3, 3, 3, 1 x 13]: B(x, k) over k = 1..4 is (2.82, 6.04, 9.75, 6.75)
    times a constant -> n_H = 3, High = {0, 1, 2}.
    A over the remaining 13 pairs = [20 x 4, 2 x 9]: k = 3, 4, 5 give
    (605.6, 897.2, 638.0) times a constant -> n_M = 4, Medium = {3, 4, 5, 6}.
    """
    kL, kM, kH = selector.tier_counts(C)
    A = [4.0] * 3 + [20.0] * 4 + [2.0] * 9
    Bv = [3.0] * 3 + [1.0] * 13
    s = np.zeros((32, C), np.float32)
    for p in range(16):
        for h in (2 * p, 2 * p + 1):
            s[h, :kM - 1] = A[p]
            s[h, kM - 1:] = Bv[p]
    gamma = np.full((32, C), -1.0, np.float32)
    eta = np.ones(32, np.float32)
    return s, gamma, eta, (kL, kM, kH)


def test_selector_crafted_decisions():
    s, gamma, eta, (kL, kM, kH) = _crafted()
    out = selector.select(s, gamma, eta)
    assert out["n_high"] == 3 and out["n_medium"] == 4
    assert out["tier"].tolist() == [2, 2, 2, 1, 1, 1, 1] + [0] * 9
    C = s.shape[1]
    for p in range(16):
        k = {2: kH, 1: kM, 0: kL}[int(out["tier"][p])]
        # ties in q everywhere within a region, earlier chunks rank first
        expect = np.zeros(C, np.uint8)
        expect[:k - 1] = 1
        expect[C - 1] = 1
        assert out["mask"][p].tolist() == expect.tolist()


def test_selector_prefers_high_score_chunks():
    """Within a pair, the kept non-anchor chunks are the top-q ones."""
    C = 64
    rng = np.random.default_rng(7)
    s = rng.uniform(0.5, 2.0, (32, C)).astype(np.float32)
    gamma = rng.uniform(-3, -0.1, (32, C)).astype(np.float32)
    eta = rng.uniform(0.5, 2, 32).astype(np.float32)
    out = selector.select(s, gamma, eta)
    s64 = s.astype(np.float64)
    for p in range(16):
        n0 = np.sqrt(np.sum(s64[2 * p] ** 2)); n1 = np.sqrt(np.sum(s64[2 * p + 1] ** 2))
        q = 0.5 * (s64[2 * p] / n0 + s64[2 * p + 1] / n1)
        kept = [c for c in range(1, C - 1) if out["mask"][p, c]]
        dropped = [c for c in range(1, C - 1) if not out["mask"][p, c]]
        assert min(q[kept]) > max(q[dropped])


@pytest.mark.parametrize("C", [1, 2, 3, 4, 17, 64, 512])
def test_selector_structure(C):
    rng = np.random.default_rng(C)
    s = rng.gamma(2.0, 1.0, (32, C)).astype(np.float32)
    gamma = (-rng.uniform(0.5, 300, (32, 1)) * np.ones((1, C))).astype(np.float32)
    gamma[:4] /= 200.0                      # a few long-memory heads
    eta = rng.uniform(0.1, 3, 32).astype(np.float32)
    out = selector.select(s, gamma, eta)
    kL, kM, kH = out["k"]
    nH, nM = out["n_high"], out["n_medium"]
    assert nH in (1, 2, 3, 4) and nM in selector.MEDIUM_CHOICES[nH]
    tiers = out["tier"].tolist()
    assert tiers.count(2) == nH and tiers.count(1) == nM
    counts = out["mask"].sum(axis=1)
    for p in range(16):
        assert counts[p] == {2: kH, 1: kM, 0: kL}[tiers[p]]
        assert out["mask"][p, 0] == 1 and out["mask"][p, C - 1] == 1
    E = int(counts.sum())
    assert E == nH * kH + nM * kM + (16 - nH - nM) * kL
    assert E <= 16 * kH
    # nested candidate sets: the same ranking drives all three tiers
    rank = out["rank"]
    for p in range(16):
        for lo, hi in ((kL, kM), (kM, kH)):
            small = {c for c in range(C) if c in (0, C - 1) or 0 <= rank[p, c] < lo - 2}
            big = {c for c in range(C) if c in (0, C - 1) or 0 <= rank[p, c] < hi - 2}
            assert small <= big
    if C == 512:
        assert 0.28442 <= E / (16 * C) <= 0.31372


@pytest.mark.parametrize("case", ["nan_score_head", "nan_everywhere", "inf_score", "nan_eta",
                                  "nan_gamma", "nan_rank_key"])
def test_selector_total_orders_with_non_finite_statistics(case):
    """Non-finite statistics (inputs outside the operator's domain) still give
    a valid selection: ranks are a permutation of the inner chunks, each tier
    keeps exactly k_l chunks, n_H and n_M come from the table, and E <= 16 k_H
    (the capacity the CSR arrays are sized to).  NaN orders as -infinity."""
    C = 40
    rng = np.random.default_rng(5)
    s = rng.gamma(2.0, 1.0, (32, C)).astype(np.float32)
    gamma = (-rng.uniform(0.5, 30, (32, 1)) * np.ones((1, C))).astype(np.float32)
    eta = rng.uniform(0.1, 3, 32).astype(np.float32)
    key = None
    if case == "nan_score_head":
        s[5, 7] = np.nan
    elif case == "nan_everywhere":
        s[:, ::3] = np.nan
    elif case == "inf_score":
        s[9, 3] = np.inf
    elif case == "nan_eta":
        eta[4] = np.nan
    elif case == "nan_gamma":
        gamma[2, 10] = np.nan
    else:
        key = rng.uniform(size=(16, C)).astype(np.float32)
        key[:, 5:9] = np.nan
    out = selector.select(s, gamma, eta, rank_key=key)
    kL, kM, kH = out["k"]
    nH, nM = out["n_high"], out["n_medium"]
    assert nH in (1, 2, 3, 4) and nM in selector.MEDIUM_CHOICES[nH]
    for p in range(16):
        assert sorted(out["rank"][p, 1:C - 1].tolist()) == list(range(C - 2))
        assert out["mask"][p].sum() == {2: kH, 1: kM, 0: kL}[int(out["tier"][p])]
    assert out["mask"].sum() <= 16 * kH
    if case == "nan_rank_key":
        # chunks whose key is NaN rank after every chunk with a finite key
        for p in range(16):
            k = {2: kH, 1: kM, 0: kL}[int(out["tier"][p])]
            if k - 2 <= C - 2 - 4:
                assert not out["mask"][p, 5:9].any()


def test_high_tier_takes_largest_gains():
    rng = np.random.default_rng(11)
    C = 64
    s = rng.gamma(2.0, 1.0, (32, C)).astype(np.float32)
    gamma = (-rng.uniform(0.05, 5, (32, 1)) * np.ones((1, C))).astype(np.float32)
    eta = rng.uniform(0.1, 3, 32).astype(np.float32)
    out = selector.select(s, gamma, eta)
    xh = np.array(out["x_h"])
    high = np.flatnonzero(out["tier"] == 2)
    others = np.flatnonzero(out["tier"] != 2)
    assert xh[high].min() >= xh[others].max()
    xm = np.array(out["x_m"])
    med = np.flatnonzero(out["tier"] == 1)
    low = np.flatnonzero(out["tier"] == 0)
    if len(med) and len(low):
        assert xm[med].min() >= xm[low].max()


# ---------------------------------------------------------- selector ablations

def _single_high(C=64):
    """Like the crafted case, but one pair's M->H gain stands far above the
    rest, so the split score picks n_H = 1 (the dynamic count differs from
    the fixed 3 / 4 / 9 split).  Gains: x_H order 0, then 1, 2, 3 (B = 2.0,
    1.9, 1.8), the rest tied; x_M order 4, 5, 6, 7 (A = 9, 8, 7, 6) after the
    High pairs."""
    kL, kM, kH = selector.tier_counts(C)
    A = [1.0] * 4 + [9.0, 8.0, 7.0, 6.0] + [1.0] * 8
    Bv = [40.0, 2.0, 1.9, 1.8] + [0.5] * 12
    s = np.zeros((32, C), np.float32)
    for p in range(16):
        for h in (2 * p, 2 * p + 1):
            s[h, :kM - 1] = max(A[p], Bv[p] + 1.0)
            s[h, kM - 1:] = Bv[p]
    return s, np.full((32, C), -1.0, np.float32), np.ones(32, np.float32), (kL, kM, kH)


def test_fixed_tiers_assign_3_high_4_medium_9_low():
    s, gamma, eta, (kL, kM, kH) = _single_high()
    dyn = selector.select(s, gamma, eta)
    assert dyn["n_high"] == 1                       # the dynamic count differs
    out = selector.select(s, gamma, eta, fixed_tiers=True)
    assert out["n_high"] == 3 and out["n_medium"] == 4
    tiers = out["tier"]
    xh, xm = np.array(out["x_h"]), np.array(out["x_m"])
    high = np.flatnonzero(tiers == 2)
    assert sorted(high.tolist()) == sorted(np.argsort(-xh, kind="stable")[:3].tolist())
    rest = [p for p in range(16) if p not in high]
    med = sorted(rest, key=lambda p: (-xm[p], p))[:4]
    assert sorted(np.flatnonzero(tiers == 1).tolist()) == sorted(med)
    counts = out["mask"].sum(axis=1)
    for p in range(16):
        assert counts[p] == {2: kH, 1: kM, 0: kL}[int(tiers[p])]
    # the same ranking as the dynamic selector (only the counts are fixed)
    assert np.array_equal(out["rank"], dyn["rank"])


def test_unit_visibility_equals_equal_gate_energies():
    """G_h = sqrt(eta_h / mean eta) is 1 for equal energies, so G = 1 is the
    selector run with every eta equal; skewed energies do change it."""
    rng = np.random.default_rng(31)
    C = 96
    s = rng.gamma(2.0, 1.0, (32, C)).astype(np.float32)
    gamma = (-rng.uniform(0.05, 5, (32, 1)) * np.ones((1, C))).astype(np.float32)
    eta = np.exp(rng.uniform(-4, 4, 32)).astype(np.float32)
    a = selector.select(s, gamma, eta, unit_visibility=True)
    b = selector.select(s, gamma, np.full(32, 0.7, np.float32))
    c = selector.select(s, gamma, eta)
    assert np.array_equal(a["mask"], b["mask"]) and np.array_equal(a["tier"], b["tier"])
    assert a["G"] == [1.0] * 32
    assert not (np.array_equal(a["mask"], c["mask"]) and np.array_equal(a["tier"], c["tier"]))


def test_rank_key_of_eq10_reproduces_the_selector():
    """Keys equal to the Eq. (10) rank key q_c (formed here from the scores)
    give the default mask; any keys keep the adaptive tiers, the keep counts
    and the anchors, and keep the chunks with the largest keys."""
    rng = np.random.default_rng(33)
    C = 80
    s = rng.gamma(2.0, 1.0, (32, C)).astype(np.float32)
    gamma = (-rng.uniform(0.05, 5, (32, 1)) * np.ones((1, C))).astype(np.float32)
    eta = rng.uniform(0.5, 2, 32).astype(np.float32)
    ref = selector.select(s, gamma, eta)
    s64 = s.astype(np.float64)
    q = np.empty((16, C))
    for p in range(16):
        n0 = math.sqrt(math.fsum(s64[2 * p] ** 2)); n1 = math.sqrt(math.fsum(s64[2 * p + 1] ** 2))
        q[p] = 0.5 * (s64[2 * p] / n0 + s64[2 * p + 1] / n1)
    q32 = q.astype(np.float32)
    for p in range(16):         # fp32 keys keep this draw's order of q exactly
        assert (sorted(range(1, C - 1), key=lambda c: (-q32[p, c], c))
                == sorted(range(1, C - 1), key=lambda c: (-q[p, c], c)))
    same = selector.select(s, gamma, eta, rank_key=q32)
    assert np.array_equal(same["tier"], ref["tier"])
    assert np.array_equal(same["mask"], ref["mask"])
    key = rng.uniform(size=(16, C)).astype(np.float32)
    rnd = selector.select(s, gamma, eta, rank_key=key)
    assert np.array_equal(rnd["tier"], ref["tier"])
    assert np.array_equal(rnd["mask"].sum(axis=1), ref["mask"].sum(axis=1))
    assert np.all(rnd["mask"][:, 0] == 1) and np.all(rnd["mask"][:, C - 1] == 1)
    for p in range(16):
        kept = [c for c in range(1, C - 1) if rnd["mask"][p, c]]
        dropped = [c for c in range(1, C - 1) if not rnd["mask"][p, c]]
        if kept and dropped:
            assert key[p, kept].min() > key[p, dropped].max()
    assert not np.array_equal(rnd["mask"], ref["mask"])


# ---------------------------------------------------------------- CSR layout

def test_event_layout_small_case():
    C = 7
    mask = np.zeros((16, C), np.uint8)
    mask[:, 0] = mask[:, C - 1] = 1
    mask[3, [2, 3]] = 1            # pair 3: events 0, 2, 3, 6
    mask[5, 4] = 1                 # pair 5: events 0, 4, 6
    tier = np.zeros(16, np.uint8)
    tier[5] = 2
    tier[3] = 1
    lay = selector.event_layout(mask, tier)
    assert lay["row_pair"].tolist()[:3] == [5, 3, 0]
    assert lay["row_ptr"].tolist()[:4] == [0, 3, 7, 9]
    assert lay["col"].tolist()[:9] == [0, 4, 6, 0, 2, 3, 6, 0, 6]
    assert lay["E"] == 3 + 4 + 14 * 2
    # groups r = 0..3 start at chunks 0, 2, 4, 6
    assert lay["pred"][3].tolist() == [-1, 0, 3, 3]
    assert lay["pred"][5].tolist() == [-1, 0, 0, 4]
    assert lay["pred"][0].tolist() == [-1, 0, 0, 0]
    # slots: row 0 (pair 5): events 0, 4; row 1 (pair 3): 0, 3; then pairs 0,1,2,4,6..15: 0
    assert lay["group_slot"][5].tolist() == [-1, 0, 0, 1]
    assert lay["group_slot"][3].tolist() == [-1, 2, 3, 3]
    assert lay["group_slot"][0].tolist() == [-1, 4, 4, 4]
    assert lay["n_snap"] == 4 + 14
    assert lay["event_slot"].tolist()[:9] == [0, 1, -1, 2, -1, 3, -1, 4, -1]
