"""Pins of the sparse oracle (oracle.sparse): fixed points, the gap restore of
Eq. (21), the group/chunk identity of Eq. (25) and the page's worked case.
CPU only."""
import math

import numpy as np
import pytest

from oracle import gdn, selector, sparse

from test_oracle_dense import rand_inputs, relerr


def _mask(seed, C, keep=0.4):
    rng = np.random.default_rng(seed)
    m = (rng.uniform(size=(1, 16, C)) < keep).astype(np.uint8)
    m[..., 0] = m[..., -1] = 1
    return m


def test_all_events_kept_exact_equals_dense_and_recurrence():
    q, k, v, a, beta = rand_inputs(40, 1, 320, 16, 32, 16, 16, slow=True)
    mask = np.ones((1, 16, 5), np.uint8)
    o, S = sparse.sparse_prefill(q, k, v, a, beta, mask=mask, solve="exact")
    o_ref, S_ref = gdn.recurrence(q, k, v, a, beta)
    assert relerr(o, o_ref) < 1e-12
    assert relerr(S, S_ref) < 1e-12


def test_budget_one_keeps_everything_blockadj_equals_dense_blockadj():
    q, k, v, a, beta = rand_inputs(41, 1, 448, 16, 32, 16, 16, slow=True)
    z = np.random.default_rng(1).standard_normal((1, 448, 32, 16))
    o, S, info = sparse.sparse_prefill(q, k, v, a, beta, z=z, keep_budget=1.0,
                                       solve="blockadj", return_all=True)
    assert info["mask"].all()
    o_ref, S_ref = gdn.chunk_prefill(q, k, v, a, beta, None, "blockadj")
    assert relerr(o, o_ref) < 1e-12
    assert relerr(S, S_ref) < 1e-12


def test_beta_zero_is_pure_decay_with_skips():
    q, k, v, a, beta = rand_inputs(42, 1, 300, 16, 32, 8, 8, slow=True)
    beta[:] = 0
    s0 = np.random.default_rng(3).standard_normal((1, 32, 8, 8))
    o, S = sparse.sparse_prefill(q, k, v, a, beta, mask=_mask(1, 5), s0=s0)
    cum = np.cumsum(a, axis=1)
    hq = np.arange(32) // 2
    expect_o = np.einsum("bthd,bhde->bthe", q[:, :, hq], s0) * np.exp2(cum)[..., None] / math.sqrt(8)
    assert relerr(o, expect_o) < 1e-12
    assert relerr(S, s0 * np.exp2(cum[:, -1])[..., None, None]) < 1e-12


def test_gap_restore_equals_chunk_by_chunk_decay():
    """Eq. (21): between consecutive kept events e < c the state entering c is
    2^(P_c - P_e+1) times the state after e; adjacent kept events give 1."""
    q, k, v, a, beta = rand_inputs(43, 1, 64 * 9, 16, 32, 8, 8, slow=True)
    mask = _mask(2, 9)
    _, _, info = sparse.sparse_prefill(q, k, v, a, beta, mask=mask, return_all=True)
    S_in, P = info["S_in"], info["P"]
    for p in range(16):
        kept = np.flatnonzero(mask[0, p])
        for e, c in zip(kept[:-1], kept[1:]):
            for h in (2 * p, 2 * p + 1):
                after_e = S_in[0, h, e + 1]
                fac = 2.0 ** (P[0, h, c] - P[0, h, e + 1])
                if c == e + 1:
                    assert fac == 1.0
                np.testing.assert_allclose(S_in[0, h, c], fac * after_e, rtol=1e-13, atol=1e-300)


def _chunk_form_output(info, q, c, d):
    """Eq. (3) per chunk with the sparse states: the O^chunk of Eq. (25)."""
    g = info["g"][0]
    qc, kc = info["qc"][0], info["kc"][0]
    tri = np.tril(np.ones((64, 64), bool))
    D = np.where(tri, np.exp2(np.where(tri, g[:, c, :, None] - g[:, c, None, :], 0)), 0)
    A = (qc[:, c] @ np.swapaxes(kc[:, c], -1, -2)) * D
    return (np.exp2(g[:, c])[..., None] * (qc[:, c] @ info["S_in"][0, :, c])
            + A @ info["Up"][0, :, c]) / math.sqrt(d)


def test_group_output_difference_identity():
    """Eq. (25): O_c+1 - O^chunk_c+1 = (1 - z_c) / sqrt(d) * A_c+1,c U'_c, and
    even chunks agree with Eq. (3) exactly."""
    d = 8
    q, k, v, a, beta = rand_inputs(44, 1, 64 * 8, 16, 32, d, d, slow=True)
    mask = _mask(3, 8, keep=0.5)
    o, _, info = sparse.sparse_prefill(q, k, v, a, beta, mask=mask, return_all=True)
    oc = o[0].reshape(8, 64, 32, d).transpose(2, 0, 1, 3)      # [Nv, C, 64, d]
    g, gamma = info["g"][0], info["gamma"][0]
    qc, kc = info["qc"][0], info["kc"][0]
    zh = np.repeat(mask[0], 2, axis=0)
    checked_skip = 0
    for c in range(0, 8, 2):
        np.testing.assert_allclose(oc[:, c], _chunk_form_output(info, q, c, d), rtol=0, atol=1e-12)
        gx = g[:, c + 1] + gamma[:, c][:, None]
        A10 = (qc[:, c + 1] @ np.swapaxes(kc[:, c], -1, -2)) * np.exp2(gx[:, :, None] - g[:, c][:, None, :])
        diff = oc[:, c + 1] - _chunk_form_output(info, q, c + 1, d)
        expect = (1 - zh[:, c])[:, None, None] / math.sqrt(d) * (A10 @ info["Up"][0, :, c])
        np.testing.assert_allclose(diff, expect, rtol=0, atol=1e-12)
        checked_skip += int((zh[:, c] == 0).sum())
    assert checked_skip > 0


def test_worked_case_skip_chunk4_keep_chunk5():
    """Sec. 2.7 example: chunk 4 skipped, chunk 5 kept.  S_5 = 2^gamma_4 S_4,
    U'_5 = U_5 - W_5 S_5, and O_5 still carries A_5,4 U_4 / sqrt(d)."""
    d = 8
    q, k, v, a, beta = rand_inputs(45, 1, 64 * 6, 16, 32, d, d, slow=True)
    mask = np.ones((1, 16, 6), np.uint8)
    mask[0, :, 4] = 0
    o, _, info = sparse.sparse_prefill(q, k, v, a, beta, mask=mask, return_all=True)
    S_in, gamma, U, Up = info["S_in"][0], info["gamma"][0], info["U"][0], info["Up"][0]
    np.testing.assert_allclose(S_in[:, 5], np.exp2(gamma[:, 4])[:, None, None] * S_in[:, 4], rtol=1e-13)
    np.testing.assert_array_equal(Up[:, 4], U[:, 4])
    W5 = sparse.deferred_w(info["Cb"][0, :, 5], info["kc"][0, :, 5])
    np.testing.assert_allclose(Up[:, 5], U[:, 5] - W5 @ S_in[:, 5], rtol=0, atol=1e-12)
    g = info["g"][0]
    gx = g[:, 5] + gamma[:, 4][:, None]
    A54 = (info["qc"][0, :, 5] @ np.swapaxes(info["kc"][0, :, 4], -1, -2)) * \
        np.exp2(gx[:, :, None] - g[:, 4][:, None, :])
    o5 = o[0, 320:384].transpose(1, 0, 2)
    np.testing.assert_allclose(o5 - _chunk_form_output(info, q, 5, d), A54 @ U[:, 4] / math.sqrt(d),
                               rtol=0, atol=1e-12)


def test_deferred_w_equals_full_product_for_blockadj():
    q, k, v, a, beta = rand_inputs(46, 1, 128, 1, 2, 16, 16, slow=True)
    kc = gdn.chunk_view(k, np.array([0, 0]))
    g, _, _ = gdn.decay_prefix(a)
    U, W, Ct, Cb, C = gdn.intra(kc, gdn.chunk_view(v), gdn.chunk_scalar(beta), g, "blockadj")
    np.testing.assert_allclose(sparse.deferred_w(Cb, kc, "blockadj"), W, rtol=0, atol=1e-13)
    U, W, Ct, Cb, C = gdn.intra(kc, gdn.chunk_view(v), gdn.chunk_scalar(beta), g, "exact")
    np.testing.assert_allclose(sparse.deferred_w(Cb, kc, "exact"), W, rtol=0, atol=1e-13)


@pytest.mark.parametrize("T", [64 * 7, 64 * 16 + 20])
def test_end_to_end_sparse_structure(T):
    """Selector-driven run: realised keep within the tier-table bounds at the
    default budget, masks shared per pair, outputs finite."""
    q, k, v, a, beta = rand_inputs(47, 1, T, 16, 32, 16, 16)
    z = np.random.default_rng(5).standard_normal((1, T, 32, 16))
    o, S, info = sparse.sparse_prefill(q, k, v, a, beta, z=z, return_all=True)
    C = -(-T // 64)
    sel = info["sel"][0]
    kL, kM, kH = selector.tier_counts(C)
    assert info["mask"].sum() == sel["n_high"] * kH + sel["n_medium"] * kM + \
        (16 - sel["n_high"] - sel["n_medium"]) * kL
    assert np.isfinite(o).all() and np.isfinite(S).all()
    assert o.shape == (1, T, 32, 16)
