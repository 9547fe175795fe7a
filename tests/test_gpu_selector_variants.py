"""Selector ablations on the GPU (Sec. 3.5, Table 5, Fig. 10): fixed 3/4/9
tiers, G_h = 1, caller rank keys (random selection at matched budget) and
the Tail-8/32/64 score windows; and the caller's tier rates in place of the
budget's (Eq. (13) with rho given).

* sgdn_select with each switch: mask, tiers, CSR rows, predecessors and
  snapshot slots bit-exact against the oracle selector with the same switch
  on the same fp32 statistics;
* sgdn_prefill_sparse end to end: the device's own statistics (tail score of
  the chosen window) within tolerance of the oracle's, the device mask equal
  to the oracle selector's on those statistics, and O / S_final within the
  bar given that mask.
"""
import numpy as np
import pytest

from gated_deltanet_prefill_chunkwise_amd import synth
from oracle import selector, sparse

from helpers import TOL, host, rel_max_err, to_device

pytestmark = pytest.mark.gpu

VARIANTS = [dict(fixed_tiers=True), dict(unit_visibility=True), dict(rank_key="random"),
            dict(fixed_tiers=True, unit_visibility=True, rank_key="random"),
            dict(tier_rate=(0.05, 0.2, 0.6)), dict(tier_rate=(0.5, 0.5, 1.0), rank_key="random")]


def _keys(seed, B, C):
    return np.random.default_rng(seed).uniform(size=(B, 16, C)).astype(np.float32)


@pytest.mark.parametrize("C", [3, 64, 200])
@pytest.mark.parametrize("vi", range(len(VARIANTS)))
def test_select_variants_bit_exact(C, vi):
    import torch
    from gated_deltanet_prefill_chunkwise_amd import ops
    var = dict(VARIANTS[vi])
    B = 2
    score, gamma, eta = synth.selector_stats(2000 + C + vi, B, C)
    key = _keys(2100 + C, B, C) if var.get("rank_key") else None
    var["rank_key"] = None if key is None else torch.from_numpy(key).cuda()
    out = ops.select(torch.from_numpy(score).cuda(), torch.from_numpy(gamma).cuda(),
                     torch.from_numpy(eta).cuda(), keep_budget=0.29, **var)
    torch.cuda.synchronize()
    out = {k: v.cpu().numpy() for k, v in out.items()}
    for b in range(B):
        ref = selector.select(score[b], gamma[b], eta[b], keep_budget=0.29,
                              fixed_tiers=var.get("fixed_tiers", False),
                              unit_visibility=var.get("unit_visibility", False),
                              rank_key=None if key is None else key[b],
                              tier_rate=var.get("tier_rate"))
        lay = selector.event_layout(ref["mask"], ref["tier"])
        assert np.array_equal(out["mask"][b], ref["mask"]), "mask"
        assert np.array_equal(out["tier"][b], ref["tier"]), "tier"
        assert np.array_equal(out["row_pair"][b], lay["row_pair"])
        assert np.array_equal(out["row_ptr"][b], lay["row_ptr"])
        assert np.array_equal(out["col"][b, :lay["E"]], lay["col"])
        assert np.array_equal(out["pred"][b], lay["pred"])
        assert np.array_equal(out["group_slot"][b], lay["group_slot"])
        if var.get("fixed_tiers") and C > 2:
            assert (out["tier"][b] == 2).sum() == 3 and (out["tier"][b] == 1).sum() == 4


def _end_to_end(T, tail=16, **var):
    import torch
    from gated_deltanet_prefill_chunkwise_amd import ops
    inp = synth.numpy_inputs(synth.seed_for(4) + T + tail, 1, T, 16, 32, dtype="bf16",
                             with_z=True, decay_scale=1 / 16)
    C = -(-T // 64)
    key = _keys(2200 + T, 1, C) if var.get("rank_key") else None
    d = to_device(inp)
    score = torch.empty((1, 32, C), device="cuda")
    gam = torch.empty((1, 32, C), device="cuda")
    eta = torch.empty((1, 32), device="cuda")
    mask = torch.empty((1, 16, C), dtype=torch.uint8, device="cuda")
    tier = torch.empty((1, 16), dtype=torch.uint8, device="cuda")
    dbg = ops.debug_struct(score=score, gamma=gam, eta=eta, mask=mask, tier=tier)
    o, S, st = ops.prefill_sparse(d["q"], d["k"], d["v"], d["a"], d["beta"], z=d["z"],
                                  keep_budget=0.29, solve="blockadj", debug=dbg, tail=tail,
                                  fixed_tiers=var.get("fixed_tiers", False),
                                  unit_visibility=var.get("unit_visibility", False),
                                  rank_key=None if key is None else torch.from_numpy(key).cuda(),
                                  tier_rate=var.get("tier_rate"))
    torch.cuda.synchronize()
    o, S = host(o), host(S)
    _, _, info = sparse.sparse_prefill(inp.q, inp.k, inp.v, inp.a, inp.beta, z=inp.z,
                                       solve="blockadj", tail=tail, return_all=True)
    s_gpu = host(score)[0]
    s_ref = info["score"][0].astype(np.float64)
    assert np.max(np.abs(s_gpu - s_ref) / np.maximum(s_ref, 1e-6)) < 2e-2, "tail score"
    ref = selector.select(score.cpu().numpy()[0], gam.cpu().numpy()[0], eta.cpu().numpy()[0],
                          keep_budget=0.29, fixed_tiers=var.get("fixed_tiers", False),
                          unit_visibility=var.get("unit_visibility", False),
                          rank_key=None if key is None else key[0],
                          tier_rate=var.get("tier_rate"))
    assert np.array_equal(mask.cpu().numpy()[0], ref["mask"]), "mask"
    assert np.array_equal(tier.cpu().numpy()[0], ref["tier"]), "tier"
    o_ref, S_ref = sparse.sparse_prefill(inp.q, inp.k, inp.v, inp.a, inp.beta, solve="blockadj",
                                         mask=ref["mask"][None])
    eo, es = rel_max_err(o, o_ref), rel_max_err(S, S_ref)
    print(f"tail {tail} {var}: E {int(st.cpu()[0, 0])}  err O {eo:.3e} S {es:.3e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


@pytest.mark.parametrize("tail", [8, 16, 32, 64])
def test_tail_windows_end_to_end(tail):
    _end_to_end(64 * 9 + 5, tail=tail)


@pytest.mark.parametrize("vi", range(len(VARIANTS)))
def test_selector_variants_end_to_end(vi):
    _end_to_end(64 * 12 + 33, **VARIANTS[vi])


@pytest.mark.parametrize("T", [1, 37, 64, 65, 130])
def test_tiny_sequences_end_to_end(T):
    """One sequence of one to three chunks (ragged or whole) through the
    single-sequence schedule (CSR rows 0-3 and 4-15 on two streams): the
    first and last chunk are the same or adjacent anchors, every pair keeps
    them, and the tail window may lie wholly in the zero padding."""
    _end_to_end(T)
