"""Parity at the benchmark's full size.

One layer of the benchmark workload (T = 131072, bf16, B = 1, Nq = 16, Nv = 32,
the benchmark's seed for layer 0, inputs drawn on the device) runs on the GPU
for all 32 heads, as the benchmark launches it.  The fp64 oracle then checks:

* dense: one head pair over the whole sequence (O at every token and S_final);
  pairs are independent, so the pair's oracle run is the full problem
  restricted to those heads;
* sparse: the selector from the GPU's own fp32 statistics (score, gamma, eta),
  mask and tiers bit-exact, and the pairs with the most and the fewest events
  over the whole sequence given the GPU's mask (pairs are independent once
  the mask is fixed).

Each oracle pass takes tens of seconds on the host.
"""
import types

import numpy as np
import pytest

from gated_deltanet_prefill_chunkwise_amd import synth
from oracle import gdn, selector, sparse

from helpers import TOL, host, rel_max_err

pytestmark = pytest.mark.gpu

T = 131072
NQ, NV = 16, 32


def _device_inputs():
    return synth.torch_inputs(synth.seed_for(3, 0), 1, T, NQ, NV, dtype="bf16", with_z=True,
                              device="cuda")


def _pair_inputs(d, p):
    """Host fp64 copies of head pair p's inputs (bf16 values are exact)."""
    f = lambda t: t.float().cpu().numpy().astype(np.float64)
    return types.SimpleNamespace(q=f(d["q"][:, :, p:p + 1]), k=f(d["k"][:, :, p:p + 1]),
                                 v=f(d["v"][:, :, 2 * p:2 * p + 2]), a=f(d["a"][:, :, 2 * p:2 * p + 2]),
                                 beta=f(d["beta"][:, :, 2 * p:2 * p + 2]))


def test_full_size_dense_pair():
    import torch
    from gated_deltanet_prefill_chunkwise_amd import ops
    d = _device_inputs()
    o, S = ops.prefill_dense(d["q"], d["k"], d["v"], d["a"], d["beta"], solve="exact")
    torch.cuda.synchronize()
    p = 11
    x = _pair_inputs(d, p)
    o_ref, S_ref = gdn.chunk_prefill(x.q, x.k, x.v, x.a, x.beta, None, "exact")
    eo = rel_max_err(host(o[:, :, 2 * p:2 * p + 2]), o_ref)
    es = rel_max_err(host(S[:, 2 * p:2 * p + 2]), S_ref)
    print(f"pair {p}: err O {eo:.3e}  S {es:.3e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


def test_full_size_sparse_selector_and_pair():
    import torch
    from gated_deltanet_prefill_chunkwise_amd import ops
    d = _device_inputs()
    C = T // 64
    score = torch.empty((1, NV, C), device="cuda")
    gam = torch.empty((1, NV, C), device="cuda")
    eta = torch.empty((1, NV), device="cuda")
    mask = torch.empty((1, NV // 2, C), dtype=torch.uint8, device="cuda")
    tier = torch.empty((1, NV // 2), dtype=torch.uint8, device="cuda")
    dbg = ops.debug_struct(score=score, gamma=gam, eta=eta, mask=mask, tier=tier)
    o, S, st = ops.prefill_sparse(d["q"], d["k"], d["v"], d["a"], d["beta"], z=d["z"],
                                  keep_budget=0.29, solve="blockadj", debug=dbg)
    torch.cuda.synchronize()
    m_gpu = mask.cpu().numpy()[0]
    # selector: identical fp32 statistics give identical integers
    ref = selector.select(score.cpu().numpy()[0], gam.cpu().numpy()[0], eta.cpu().numpy()[0],
                          keep_budget=0.29)
    assert np.array_equal(m_gpu, ref["mask"]), "mask"
    assert np.array_equal(tier.cpu().numpy()[0], ref["tier"]), "tier"
    assert int(st.cpu().numpy()[0, 0]) == int(m_gpu.sum())
    # the pair with the most events (a High-tier pair: its CSR row is among
    # rows 0-3, whose H scan and O run on the caller's stream) and the pair
    # with the fewest (a Low-tier pair: CSR rows 4-15, on the library's second
    # stream), each given the GPU's mask
    counts = m_gpu.sum(axis=1)
    for p in (int(np.argmax(counts)), int(np.argmin(counts))):
        x = _pair_inputs(d, p)
        o_ref, S_ref = sparse.sparse_prefill(x.q, x.k, x.v, x.a, x.beta, solve="blockadj",
                                             mask=m_gpu[None, p:p + 1])
        eo = rel_max_err(host(o[:, :, 2 * p:2 * p + 2]), o_ref)
        es = rel_max_err(host(S[:, 2 * p:2 * p + 2]), S_ref)
        print(f"pair {p} ({int(counts[p])} events): err O {eo:.3e}  S {es:.3e}")
        assert eo <= TOL["bf16"] and es <= TOL["bf16"]
