"""Long-memory parity at 32768 tokens on every head.

At the workload's decays the state carried across a chunk is scaled by at most
2^-74, so what the H scan carries over long event chains never reaches the
outputs within tolerance.  Here a is divided by 64 (per-chunk retention
2^-1.2 .. 2^-4.7; SparseGDN reading notes, Sec. 2.6): the state stays live
over many chunks, so O and S_final depend on every link of the chains, the
fp16 state operands and snapshots, the gap factors over multi-chunk gaps
(Eq. (21)) and the group entries restored from distant snapshots.  One layer
(bf16, B = 1, Nq = 16, Nv = 32), dense with the exact solve and sparse at
the default budget with the on-device selector; all 32 heads against the
fp64 oracle.
"""
import numpy as np
import pytest

from gated_deltanet_prefill_chunkwise_amd import synth
from oracle import gdn, selector, sparse

from helpers import TOL, host, rel_max_err

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

T = 32768
NQ, NV = 16, 32


def _inputs():
    return synth.torch_inputs(synth.seed_for(2, 0) + 64, 1, T, NQ, NV, dtype="bf16",
                              with_z=True, device="cuda", decay_scale=1 / 64)


def _host(d):
    return {k: v.float().cpu().numpy().astype(np.float64) for k, v in d.items()}


def test_live_state_dense_all_heads():
    import torch
    from gated_deltanet_prefill_chunkwise_amd import ops
    d = _inputs()
    o, S = ops.prefill_dense(d["q"], d["k"], d["v"], d["a"], d["beta"], solve="exact")
    torch.cuda.synchronize()
    x = _host(d)
    o_ref, S_ref = gdn.chunk_prefill(x["q"], x["k"], x["v"], x["a"], x["beta"], None, "exact")
    eo, es = rel_max_err(host(o), o_ref), rel_max_err(host(S), S_ref)
    # the carried state matters: the outputs differ from those of a state
    # that forgets everything older than one chunk by far more than the bar
    print(f"err O {eo:.3e}  S {es:.3e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


def test_live_state_sparse_all_heads():
    import torch
    from gated_deltanet_prefill_chunkwise_amd import ops
    d = _inputs()
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
    m_gpu, t_gpu = mask.cpu().numpy()[0], tier.cpu().numpy()[0]
    ref = selector.select(score.cpu().numpy()[0], gam.cpu().numpy()[0], eta.cpu().numpy()[0],
                          keep_budget=0.29)
    assert np.array_equal(m_gpu, ref["mask"]) and np.array_equal(t_gpu, ref["tier"])
    # slow decay: lifetimes L_h of Eq. (11) are of order one (at the
    # workload's decays they are below 2^-70), so the gains are not all zero
    # and the tier split is an actual decision
    assert np.max(ref["L"]) > 0.1
    x = _host(d)
    o_ref, S_ref = sparse.sparse_prefill(x["q"], x["k"], x["v"], x["a"], x["beta"],
                                         solve="blockadj", mask=m_gpu[None])
    eo, es = rel_max_err(host(o), o_ref), rel_max_err(host(S), S_ref)
    per_head = [rel_max_err(host(o[:, :, h]), o_ref[:, :, h]) for h in range(NV)]
    print(f"keep {m_gpu.mean():.4f}, tiers {np.bincount(t_gpu, minlength=3).tolist()}: "
          f"err O {eo:.3e}  S {es:.3e}; worst head {int(np.argmax(per_head))} "
          f"{max(per_head):.3e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]
