"""The selector's bit-reproducibility rests on correctly rounded binary64
division and square root on the device (SparseGDN reading notes, Sec. 2.4,
Eqs. (10)-(14) are evaluated with them; see the selector source).  The
library's own compiled forms of both operations (sgdn_fp64_selftest, built
with the selector's flags) are compared bit for bit with the host's IEEE
operations on about 10^7 operands drawn from the ranges the selector meets
and from half the exponent range (normal-number quotients)."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

N = 10_000_000


def _operands(seed):
    g = np.random.default_rng(seed)
    n4 = N // 4
    parts_x, parts_y = [], []
    # fp32-valued statistics over their norms, means and sample counts
    parts_x.append(g.gamma(2.0, 1.0, n4).astype(np.float32).astype(np.float64))
    parts_y.append(np.sqrt(g.uniform(1.0, 4096.0, n4)) * g.uniform(0.5, 3.0, n4))
    # sums of squares and gains: wide positive magnitudes
    parts_x.append(np.exp(g.uniform(-200, 200, n4)))
    parts_y.append(np.exp(g.uniform(-200, 200, n4)))
    # full 53-bit significands, random signs, exponents over half the range
    # (quotients stay normal numbers)
    m = g.uniform(1.0, 2.0, (2, n4))
    e = g.integers(-500, 500, (2, n4))
    parts_x.append(np.abs(np.ldexp(m[0], e[0])))
    parts_y.append(np.ldexp(m[1], e[1]) * np.where(g.uniform(size=n4) < 0.5, -1, 1))
    # integers and small rationals (k (n - k) / n, C - 2, 1 - r)
    k = g.integers(1, 4096, N - 3 * n4).astype(np.float64)
    parts_x.append(k * g.integers(1, 4096, N - 3 * n4))
    parts_y.append(np.maximum(1.0 - g.uniform(0.0, 1.0, N - 3 * n4), 2.0 ** -60))
    return np.concatenate(parts_x), np.concatenate(parts_y)


def test_fp64_division_and_sqrt_round_correctly():
    import torch
    from gated_deltanet_prefill_chunkwise_amd import ops
    x, y = _operands(20261202)
    assert x.size == N and np.all(x >= 0) and np.all(y != 0)
    q, r = ops.fp64_selftest(torch.from_numpy(x).cuda(), torch.from_numpy(y).cuda())
    torch.cuda.synchronize()
    qh, rh = x / y, np.sqrt(x)
    qd, rd = q.cpu().numpy(), r.cpu().numpy()
    bad_q = np.flatnonzero(qd.view(np.uint64) != qh.view(np.uint64))
    bad_r = np.flatnonzero(rd.view(np.uint64) != rh.view(np.uint64))
    print(f"{N} operands: division mismatches {bad_q.size}, sqrt mismatches {bad_r.size}")
    assert bad_q.size == 0, [(x[i], y[i], qd[i], qh[i]) for i in bad_q[:5]]
    assert bad_r.size == 0, [(x[i], rd[i], rh[i]) for i in bad_r[:5]]
