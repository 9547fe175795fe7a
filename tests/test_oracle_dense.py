"""Pins of the dense oracle (oracle.gdn) against closed forms, library routines,
special cases and printed counts.  CPU only."""
import json
import math
import os

import numpy as np
import pytest
import scipy.linalg

from oracle import gdn

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "printed_values.json")))


def rand_inputs(seed, B, T, Nq, Nv, d=16, dv=16, slow=False):
    """Small fp64 inputs drawn like the workload (normalised q, k; sigmoid beta)."""
    g = np.random.default_rng(seed)
    q = g.standard_normal((B, T, Nq, d)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = g.standard_normal((B, T, Nq, d)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = g.standard_normal((B, T, Nv, dv))
    beta = 1 / (1 + np.exp(-g.standard_normal((B, T, Nv))))
    u = g.uniform(0, math.log(4), Nv)
    a = -np.logaddexp(0, g.standard_normal((B, T, Nv))) * np.exp(u) / math.log(2)
    if slow:
        a = a / 64
    return q, k, v, a, beta


def relerr(x, ref):
    return np.max(np.abs(x - ref)) / np.sqrt(np.mean(ref ** 2))


# ---------------------------------------------------------------- recurrence

def test_beta_zero_is_pure_decay():
    """beta = 0 gives M = I, U = W = 0: S_T = 2^(sum a) s0 and
    o_t = 2^(sum_{t'<=t} a) s0^T q_t / sqrt(d)."""
    B, T, Nq, Nv, d = 1, 150, 2, 4, 16
    q, k, v, a, beta = rand_inputs(1, B, T, Nq, Nv, d, d, slow=True)
    beta[:] = 0
    s0 = np.random.default_rng(2).standard_normal((B, Nv, d, d))
    cum = np.cumsum(a, axis=1)                               # [B, T, Nv]
    hq = np.arange(Nv) // 2
    expect_o = np.einsum("bthd,bhde->bthe", q[:, :, hq], s0) * np.exp2(cum)[..., None] / math.sqrt(d)
    expect_S = s0 * np.exp2(cum[:, -1])[..., None, None]
    for fn in (lambda: gdn.recurrence(q, k, v, a, beta, s0),
               lambda: gdn.chunk_prefill(q, k, v, a, beta, s0, "exact"),
               lambda: gdn.chunk_prefill(q, k, v, a, beta, s0, "blockadj")):
        o, S = fn()
        assert relerr(o, expect_o) < 1e-12
        assert relerr(S, expect_S) < 1e-12


def test_orthonormal_keys_store_and_overwrite():
    """a = 0, beta = 1, one-hot keys: the delta rule stores v under its key,
    reads it back exactly, and a repeated key overwrites the old value."""
    d = dv = 8
    T = 8
    keys = [0, 1, 2, 3, 4, 2, 6, 7]           # token 5 re-uses key e_2
    queries = [0, 1, 2, 3, 4, 2, 2, 1]        # token 6 reads key e_2 back, token 7 e_1
    q = np.zeros((1, T, 1, d)); k = np.zeros((1, T, 1, d))
    for t in range(T):
        k[0, t, 0, keys[t]] = 1.0
        q[0, t, 0, queries[t]] = 1.0
    v = np.random.default_rng(3).standard_normal((1, T, 2, dv))
    a = np.zeros((1, T, 2)); beta = np.ones((1, T, 2))
    o, S = gdn.recurrence(q, k, v, a, beta)
    s = math.sqrt(d)
    for t in range(6):
        np.testing.assert_allclose(o[0, t], v[0, t] / s, atol=1e-14)
    np.testing.assert_allclose(o[0, 6], v[0, 5] / s, atol=1e-14)   # overwritten value
    np.testing.assert_allclose(o[0, 7], v[0, 1] / s, atol=1e-14)
    np.testing.assert_allclose(S[0, :, 2, :], v[0, 5], atol=1e-14)
    assert np.abs(S[0, :, 5, :]).max() == 0.0                     # never written


def test_decode_step_reads_back_and_leaves_the_complement():
    """One decode step with a unit key and beta = 1 stores v exactly under k
    whatever the decay and old state: S'^T k = v, so q = k reads v / sqrt(d);
    every direction x orthogonal to k only decays: S'^T x = 2^a S^T x."""
    g = np.random.default_rng(21)
    B, Nq, Nv, d = 2, 2, 4, 16
    k = g.standard_normal((B, Nq, d)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = g.standard_normal((B, Nv, d))
    a = -g.uniform(0.1, 3.0, (B, Nv))
    s = g.standard_normal((B, Nv, d, d))
    o, S = gdn.decode_step(k, k, v, a, np.ones((B, Nv)), s)
    hq = np.arange(Nv) // (Nv // Nq)
    kh = k[:, hq]                                            # [B, Nv, d]
    np.testing.assert_allclose(np.einsum("bhd,bhde->bhe", kh, S), v, atol=1e-12)
    np.testing.assert_allclose(o, v / math.sqrt(d), atol=1e-12)
    x = g.standard_normal((B, Nv, d))
    x -= np.sum(x * kh, axis=-1, keepdims=True) * kh         # x orthogonal to k
    np.testing.assert_allclose(np.einsum("bhd,bhde->bhe", x, S),
                               np.exp2(a)[..., None] * np.einsum("bhd,bhde->bhe", x, s),
                               atol=1e-12)


def test_decode_step_continues_a_chunk_prefill():
    """Chunk prefill of T tokens then one decode step equals the token
    recurrence over T + 1 tokens (last output and final state)."""
    q, k, v, a, beta = rand_inputs(22, 1, 131, 2, 4, 16, 16)
    o_ref, S_ref = gdn.recurrence(q, k, v, a, beta)
    _, S = gdn.chunk_prefill(q[:, :-1], k[:, :-1], v[:, :-1], a[:, :-1], beta[:, :-1], None,
                             "exact")
    o, S2 = gdn.decode_step(q[:, -1], k[:, -1], v[:, -1], a[:, -1], beta[:, -1], S)
    assert relerr(o, o_ref[:, -1]) < 1e-11
    assert relerr(S2, S_ref) < 1e-11


def test_value_columns_are_independent():
    """Permuting the value columns (and s0's) permutes O and S the same way."""
    q, k, v, a, beta = rand_inputs(4, 1, 100, 1, 2, 16, 16)
    s0 = np.random.default_rng(5).standard_normal((1, 2, 16, 16))
    perm = np.random.default_rng(6).permutation(16)
    o, S = gdn.chunk_prefill(q, k, v, a, beta, s0, "exact")
    o2, S2 = gdn.chunk_prefill(q, k, v[..., perm], a, beta, s0[..., perm], "exact")
    np.testing.assert_allclose(o2, o[..., perm], rtol=0, atol=1e-13)
    np.testing.assert_allclose(S2, S[..., perm], rtol=0, atol=1e-13)


@pytest.mark.parametrize("T", [64, 128, 256, 200, 37])
@pytest.mark.parametrize("slow", [False, True])
def test_chunk_form_equals_recurrence(T, slow):
    """Eqs. (1)-(6) with the exact local solve reproduce the token recurrence,
    including a ragged final chunk (zero-padded, U4 reading)."""
    q, k, v, a, beta = rand_inputs(10 + T, 2, T, 2, 4, 16, 16, slow=slow)
    s0 = np.random.default_rng(T).standard_normal((2, 4, 16, 16)) * 0.3
    o_ref, S_ref = gdn.recurrence(q, k, v, a, beta, s0)
    o, S = gdn.chunk_prefill(q, k, v, a, beta, s0, "exact")
    assert o.shape == o_ref.shape
    assert relerr(o, o_ref) < 1e-12
    assert relerr(S, S_ref) < 1e-12


def test_chained_prefill():
    """Prefill(T1) then prefill(T2, s0 = S_final) equals prefill(T1 + T2)."""
    q, k, v, a, beta = rand_inputs(20, 1, 192, 2, 4, 16, 16, slow=True)
    o, S = gdn.chunk_prefill(q, k, v, a, beta, None, "blockadj")
    o1, S1 = gdn.chunk_prefill(q[:, :128], k[:, :128], v[:, :128], a[:, :128], beta[:, :128], None, "blockadj")
    o2, S2 = gdn.chunk_prefill(q[:, 128:], k[:, 128:], v[:, 128:], a[:, 128:], beta[:, 128:], S1, "blockadj")
    assert relerr(np.concatenate([o1, o2], 1), o) < 1e-12
    assert relerr(S2, S) < 1e-12


def test_decay_prefix_closed_form():
    """a = -1 everywhere: g[c, i] = -(i + 1), gamma = -64, P_c = -64 c."""
    a = -np.ones((1, 64 * 3, 2))
    g, gamma, P = gdn.decay_prefix(a)
    np.testing.assert_array_equal(g[0, 0, 1], -(np.arange(64) + 1.0))
    np.testing.assert_array_equal(gamma[0, 1], [-64.0] * 3)
    np.testing.assert_array_equal(P[0, 0], [0.0, -64.0, -128.0, -192.0])


# ---------------------------------------------------------------- local solve

def _random_system(seed, n=6):
    q, k, v, a, beta = rand_inputs(seed, 1, 64 * n, 1, 2, 32, 32)
    kc = gdn.chunk_view(k, np.array([0, 0]))
    vc = gdn.chunk_view(v)
    bc = gdn.chunk_scalar(beta)
    g, _, _ = gdn.decay_prefix(a)
    # fast decay leaves M nearly the identity; a slow variant exercises the
    # far blocks, so test both
    g_slow, _, _ = gdn.decay_prefix(a / 64)
    return kc, vc, bc, g, g_slow


def test_local_solve_matches_library_triangular_solve():
    kc, vc, bc, g, g_slow = _random_system(30)
    for gg in (g, g_slow):
        M = gdn.local_system(kc, bc, gg)
        assert np.all(np.triu(M, 1) == 0) and np.all(np.diagonal(M, axis1=-2, axis2=-1) == 1)
        X = gdn.invert_unit_lower(M)
        M2 = M.reshape(-1, 64, 64)
        ref = np.stack([scipy.linalg.solve_triangular(m, np.eye(64), lower=True, unit_diagonal=True)
                        for m in M2]).reshape(M.shape)
        assert np.max(np.abs(X - ref)) < 1e-12
        U, W, Ct, Cb, C = gdn.intra(kc, vc, bc, gg, "exact")
        # M U = diag(beta) V and M W = diag(beta 2^g) K  (Eq. (6))
        assert np.max(np.abs(M @ U - bc[..., None] * vc)) < 1e-12
        assert np.max(np.abs(M @ W - (bc * np.exp2(gg))[..., None] * kc)) < 1e-12


def test_block_adjacent_equals_masked_dense_inverse():
    """Eq. (8) blocks equal the matching blocks of M^{-1}; the approximation is
    M^{-1} with blocks (2,0), (3,0), (3,1) set to zero."""
    kc, vc, bc, g, g_slow = _random_system(31)
    M = gdn.local_system(kc, bc, g_slow)
    inv = np.linalg.inv(M)
    Cba = gdn.block_adjacent_inverse(M)
    masked = inv.copy()
    for (i, j) in [(2, 0), (3, 0), (3, 1)]:
        masked[..., 16 * i:16 * (i + 1), 16 * j:16 * (j + 1)] = 0
    assert np.max(np.abs(Cba - masked)) < 1e-12
    # the dropped blocks are really non-zero in the exact inverse here
    assert np.abs(inv[..., 32:48, 0:16]).max() > 1e-6


def test_block_adjacent_support_count():
    """1,248 of the 2,016 strictly lower entries are kept (61.9%)."""
    gold = GOLD["block_adjacent_support"]
    kc, vc, bc, g, g_slow = _random_system(32, n=1)
    C = gdn.block_adjacent_inverse(gdn.local_system(kc, bc, g_slow))[0, 0, 0]
    strict = np.tril(np.ones((64, 64), bool), -1)
    kept = int(np.count_nonzero(C[strict]))
    assert kept == gold["kept_strict_lower"]
    assert int(strict.sum()) == gold["total_strict_lower"]
    assert round(100 * kept / strict.sum(), 1) == gold["percent"]
    assert int(np.count_nonzero(C)) == kept + 64


def test_blockadj_dense_prefill_matches_explicit_masked_inverse():
    """Dense prefill with the 7-block solve equals the chunk recurrence driven
    by an explicitly masked numpy inverse."""
    q, k, v, a, beta = rand_inputs(33, 1, 256, 2, 4, 16, 16, slow=True)
    o, S = gdn.chunk_prefill(q, k, v, a, beta, None, "blockadj")
    # reference: same chunk algebra with C from np.linalg.inv, blocks zeroed
    hq = np.arange(4) // 2
    kc = gdn.chunk_view(k, hq); vc = gdn.chunk_view(v); qc = gdn.chunk_view(q, hq)
    bc = gdn.chunk_scalar(beta)
    g, gamma, _ = gdn.decay_prefix(a)
    inv = np.linalg.inv(gdn.local_system(kc, bc, g))
    for (i, j) in [(2, 0), (3, 0), (3, 1)]:
        inv[..., 16 * i:16 * (i + 1), 16 * j:16 * (j + 1)] = 0
    U = (inv * bc[..., None, :]) @ vc
    W = (inv * (bc * np.exp2(g))[..., None, :]) @ kc
    S_ = np.zeros((1, 4, 16, 16)); outs = []
    tri = np.tril(np.ones((64, 64), bool))
    for c in range(4):
        Up = U[:, :, c] - W[:, :, c] @ S_
        D = np.where(tri, np.exp2(np.where(tri, g[:, :, c, :, None] - g[:, :, c, None, :], 0)), 0)
        A = (qc[:, :, c] @ np.swapaxes(kc[:, :, c], -1, -2)) * D
        outs.append((np.exp2(g[:, :, c])[..., None] * (qc[:, :, c] @ S_) + A @ Up) / 4.0)
        S_ = np.exp2(gamma[:, :, c])[..., None, None] * S_ + \
            np.swapaxes(kc[:, :, c], -1, -2) @ (Up * np.exp2(gamma[:, :, c][..., None] - g[:, :, c])[..., None])
    o_ref = np.stack(outs, 2).transpose(0, 2, 3, 1, 4).reshape(1, 256, 4, 16)
    assert relerr(o, o_ref) < 1e-12
    assert relerr(S, S_) < 1e-12
