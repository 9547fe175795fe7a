"""Parity over the keep-budget and batch sweep: one layer, bf16, T = 32768,
Nq = 16, Nv = 32, batch 2 / 4 / 8, keep budget 0.15 / 0.29 / 0.5 / 1.0, and
the wide spread of per-head decay scales (u_h ~ U(0, ln 16)).  The pages
time this sweep (batch scaling and the keep-budget trade-off, Sec. 3); here
it is a parity case at its full size, in one launch per stage as a batch
runs; the single 32768-token layer (keep 0.29, u_h ~ U(0, ln 4)) runs beside
it.

For every (batch, budget): the selector of every sequence is bit-exact
against the oracle selector on the GPU's own fp32 statistics, the event
count per sequence matches the mask, and in the last sequence the pair with
the most events has O and S_final within the bar given the GPU's mask.  The
single 32768-token layer checks O and S_final of all 16 head pairs.
"""
import functools
import math
import types

import numpy as np
import pytest

from gated_deltanet_prefill_chunkwise_amd import synth
from oracle import selector, sparse

from helpers import TOL, host, rel_max_err

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]

T = 32768
NQ, NV = 16, 32


@functools.lru_cache(maxsize=1)
def _inputs(B, u_max):
    return synth.torch_inputs(synth.seed_for(4 if B > 1 else 2, 0) + B, B, T, NQ, NV, dtype="bf16",
                              with_z=True, u_max=u_max, device="cuda")


# the sweep, then the single 32768-token layer at the default budget and the
# default decay spread (one sequence: CSR rows 0-3 and 4-15 on two streams)
CASES = [(B, keep, math.log(16.0)) for keep in (0.15, 0.29, 0.5, 1.0) for B in (2, 4, 8)] + \
        [(1, 0.29, math.log(4.0))]


@pytest.mark.parametrize("B,keep,u_max", CASES)
def test_sweep_selector_and_pair(B, keep, u_max):
    import torch
    from gated_deltanet_prefill_chunkwise_amd import ops
    d = _inputs(B, u_max)
    C = T // 64
    score = torch.empty((B, NV, C), device="cuda")
    gam = torch.empty((B, NV, C), device="cuda")
    eta = torch.empty((B, NV), device="cuda")
    mask = torch.empty((B, NV // 2, C), dtype=torch.uint8, device="cuda")
    tier = torch.empty((B, NV // 2), dtype=torch.uint8, device="cuda")
    dbg = ops.debug_struct(score=score, gamma=gam, eta=eta, mask=mask, tier=tier)
    o, S, st = ops.prefill_sparse(d["q"], d["k"], d["v"], d["a"], d["beta"], z=d["z"],
                                  keep_budget=keep, solve="blockadj", debug=dbg,
                                  out_dtype=torch.float16)
    torch.cuda.synchronize()
    sc, gm, et = score.cpu().numpy(), gam.cpu().numpy(), eta.cpu().numpy()
    m_gpu, t_gpu, st = mask.cpu().numpy(), tier.cpu().numpy(), st.cpu().numpy()
    for b in range(B):
        ref = selector.select(sc[b], gm[b], et[b], keep_budget=keep)
        assert np.array_equal(m_gpu[b], ref["mask"]), f"mask of sequence {b}"
        assert np.array_equal(t_gpu[b], ref["tier"]), f"tiers of sequence {b}"
        assert int(st[b, 0]) == int(m_gpu[b].sum())
    b = B - 1
    # one sequence: every pair; batches: the pair with the most events of the
    # last sequence
    pairs = list(range(NV // 2)) if B == 1 else [int(np.argmax(m_gpu[b].sum(axis=1)))]
    p0, p1 = pairs[0], pairs[-1] + 1
    f = lambda t: t[b:b + 1].float().cpu().numpy().astype(np.float64)
    x = types.SimpleNamespace(q=f(d["q"][:, :, p0:p1]), k=f(d["k"][:, :, p0:p1]),
                              v=f(d["v"][:, :, 2 * p0:2 * p1]), a=f(d["a"][:, :, 2 * p0:2 * p1]),
                              beta=f(d["beta"][:, :, 2 * p0:2 * p1]))
    o_ref, S_ref = sparse.sparse_prefill(x.q, x.k, x.v, x.a, x.beta, solve="blockadj",
                                         mask=m_gpu[b:b + 1, p0:p1])
    eo = rel_max_err(host(o[b:b + 1, :, 2 * p0:2 * p1]), o_ref)
    es = rel_max_err(host(S[b:b + 1, 2 * p0:2 * p1]), S_ref)
    keep_meas = float(m_gpu.mean())
    print(f"B {B} keep {keep}: measured keep {keep_meas:.4f}; pairs {p0}..{p1 - 1} of sequence "
          f"{b} ({int(m_gpu[b, p0:p1].sum())} events): err O {eo:.3e} S {es:.3e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]
