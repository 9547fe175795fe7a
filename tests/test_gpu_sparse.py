"""GPU parity of the SparseGDN path against the fp64 oracle.

* sgdn_select: bit-exact mask, tiers, CSR rows, predecessors and snapshot slots
  on identical seeded fp32 statistics.
* sgdn_prefill_sparse with a given event mask (the oracle's own selection):
  O and S_final within 2e-2 (bf16) / 1e-4 (fp32) of max error over RMS.
* end to end with the on-device selector: the device statistics (score,
  gamma, eta) within tolerance of the oracle's, the oracle selector on the
  device's own fp32 statistics bit-exact with the device mask and tiers, and
  O, S_final against the oracle given that mask.
"""
import numpy as np
import pytest

from gated_deltanet_prefill_chunkwise_amd import synth
from oracle import gdn, selector, sparse

from helpers import TOL, host, rel_max_err, to_device

pytestmark = pytest.mark.gpu


def _t(x, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    return t if dtype is None else t.to(dtype)


# ------------------------------------------------------------------ selector

def compare_select(score, gamma, eta, budget):
    import torch
    from gated_deltanet_prefill_chunkwise_amd import ops
    out = ops.select(_t(score), _t(gamma), _t(eta), keep_budget=budget)
    torch.cuda.synchronize()
    out = {k: v.cpu().numpy() for k, v in out.items()}
    B = score.shape[0]
    for b in range(B):
        ref = selector.select(score[b], gamma[b], eta[b], keep_budget=budget)
        lay = selector.event_layout(ref["mask"], ref["tier"])
        assert np.array_equal(out["mask"][b], ref["mask"]), "mask"
        assert np.array_equal(out["tier"][b], ref["tier"]), "tier"
        assert np.array_equal(out["row_pair"][b], lay["row_pair"]), "row_pair"
        assert np.array_equal(out["row_ptr"][b], lay["row_ptr"]), "row_ptr"
        E = lay["E"]
        assert np.array_equal(out["col"][b, :E], lay["col"]), "col"
        assert np.array_equal(out["pred"][b], lay["pred"]), "pred"
        assert np.array_equal(out["group_slot"][b], lay["group_slot"]), "group_slot"
        st = out["stats"][b]
        kL, kM, kH = ref["k"]
        nt = [int((ref["tier"] == t).sum()) for t in (0, 1, 2)]
        assert st.tolist() == [E, 16 * kH, *nt, kL, kM, kH, lay["n_snap"], 0, 0], st


@pytest.mark.parametrize("C", [1, 2, 3, 4, 5, 33, 64, 200, 512])
@pytest.mark.parametrize("ties", [False, True])
def test_select_bit_exact(C, ties):
    score, gamma, eta = synth.selector_stats(1000 + C + 7 * ties, 2, C, ties=ties)
    compare_select(score, gamma, eta, 0.29)


@pytest.mark.parametrize("budget", [0.15, 0.5, 1.0])
def test_select_bit_exact_budgets(budget):
    score, gamma, eta = synth.selector_stats(77, 2, 300)
    compare_select(score, gamma, eta, budget)


def test_select_bit_exact_full_length():
    """C = 2048 (T = 128K)."""
    score, gamma, eta = synth.selector_stats(2048, 1, 2048)
    compare_select(score, gamma, eta, 0.29)


@pytest.mark.parametrize("case", ["nan_scores", "inf_score", "nan_eta", "nan_gamma"])
def test_select_bit_exact_non_finite(case):
    """Non-finite statistics (what inputs outside the operator's domain give):
    both sides order NaN as -infinity, so the selection stays a valid one and
    bit-exact."""
    score, gamma, eta = synth.selector_stats(4242, 2, 96)
    if case == "nan_scores":
        score[0, 3, ::5] = np.nan
        score[1, :, 7] = np.nan
    elif case == "inf_score":
        score[1, 8, 40] = np.inf
    elif case == "nan_eta":
        eta[0, 11] = np.nan
    else:
        gamma[1, 20, 90] = np.nan
    compare_select(score, gamma, eta, 0.29)


def test_select_crafted_decisions():
    """Hand-derived case of the oracle pins: n_H = 3, n_M = 4."""
    from test_oracle_selector import _crafted
    s, gamma, eta, _ = _crafted()
    compare_select(s[None], gamma[None], eta[None], 0.29)


# ------------------------------------------------------------------ prefill

def oracle_sparse(inp, budget=0.29, solve="blockadj", mask=None, s0=None):
    return sparse.sparse_prefill(inp.q, inp.k, inp.v, inp.a, inp.beta, z=inp.z, keep_budget=budget,
                                 solve=solve, mask=mask, s0=s0, return_all=True)


def run_sparse(inp, budget=0.29, solve="blockadj", mask=None, s0=None, debug=None, out_dtype=None):
    import torch
    from gated_deltanet_prefill_chunkwise_amd import ops
    d = to_device(inp)
    m = None if mask is None else _t(mask.astype(np.uint8))
    s0d = None if s0 is None else _t(s0.astype(np.float32))
    o, S, st = ops.prefill_sparse(d["q"], d["k"], d["v"], d["a"], d["beta"], z=d["z"],
                                  keep_budget=budget, solve=solve, mask_override=m, s0=s0d,
                                  debug=debug, out_dtype=out_dtype)
    if out_dtype is not None:
        assert o.dtype == out_dtype
    torch.cuda.synchronize()
    return host(o), host(S), st.cpu().numpy()


@pytest.mark.parametrize("dtype,T,decay", [("f32", 64 * 5 + 9, 1 / 32), ("bf16", 64 * 9 + 5, 1.0),
                                           ("bf16", 64 * 9 + 5, 1 / 64), ("bf16", 64 * 2, 1 / 16)])
def test_sparse_given_mask(dtype, T, decay):
    """The oracle selects its own mask; the GPU runs H and O with that mask."""
    inp = synth.numpy_inputs(300 + T, 1, T, 16, 32, dtype=dtype, with_z=True, decay_scale=decay)
    o_ref, S_ref, info = oracle_sparse(inp)
    o, S, st = run_sparse(inp, mask=info["mask"])
    eo, es = rel_max_err(o, o_ref), rel_max_err(S, S_ref)
    print(f"err O {eo:.3e} S {es:.3e}  E {st[0, 0]}")
    assert eo <= TOL[dtype] and es <= TOL[dtype]
    assert st[0, 0] == int(info["mask"].sum())


@pytest.mark.parametrize("solve", ["exact", "blockadj"])
def test_sparse_fp16_output(solve):
    """O in fp16 (the benchmark's output type) on the sparse path, both
    streams of the single-sequence schedule: the plain bar."""
    import torch
    T = 64 * 30 + 21
    inp = synth.numpy_inputs(synth.seed_for(2) + 12, 1, T, 16, 32, dtype="bf16", with_z=True,
                             decay_scale=1 / 16)
    _, _, info = oracle_sparse(inp, solve=solve)
    o, S, st = run_sparse(inp, solve=solve, mask=info["mask"], out_dtype=torch.float16)
    o_ref, S_ref = sparse.sparse_prefill(inp.q, inp.k, inp.v, inp.a, inp.beta, solve=solve,
                                         mask=info["mask"])
    eo, es = rel_max_err(o, o_ref), rel_max_err(S, S_ref)
    print(f"fp16 o: err O {eo:.3e} S {es:.3e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


@pytest.mark.parametrize("solve", ["exact", "blockadj"])
def test_sparse_bf16_output(solve):
    """O in bf16 on the sparse path (the O kernel's bf16-output instance on
    both streams of the single-sequence schedule): the bar is the fp32-output
    bar plus the output's own rounding (at most 2^-8 of the element)."""
    import torch
    T = 64 * 30 + 21
    inp = synth.numpy_inputs(synth.seed_for(2) + 11, 1, T, 16, 32, dtype="bf16", with_z=True,
                             decay_scale=1 / 16)
    _, _, info = oracle_sparse(inp, solve=solve)
    o, S, _ = run_sparse(inp, solve=solve, mask=info["mask"], out_dtype=torch.bfloat16)
    o_ref, S_ref = sparse.sparse_prefill(inp.q, inp.k, inp.v, inp.a, inp.beta, solve=solve,
                                         mask=info["mask"])
    rms = np.sqrt(np.mean(o_ref ** 2))
    excess = np.abs(o - o_ref) - 2.0 ** -8 * np.abs(o_ref)
    print(f"max excess over the output rounding {excess.max() / rms:.3e}; err S {rel_max_err(S, S_ref):.3e}")
    assert excess.max() <= TOL["bf16"] * rms
    assert rel_max_err(S, S_ref) <= TOL["bf16"]


def test_sparse_random_mask_with_initial_state():
    T = 64 * 7 + 30
    inp = synth.numpy_inputs(5, 2, T, 16, 32, dtype="bf16", decay_scale=1 / 64)
    rng = np.random.default_rng(9)
    mask = (rng.uniform(size=(2, 16, 8)) < 0.35).astype(np.uint8)
    mask[:, 3] = 0            # a pair without any event
    s0 = (rng.standard_normal((2, 32, 128, 128)) * 0.05).astype(np.float32).astype(np.float64)
    o_ref, S_ref, _ = oracle_sparse(inp, mask=mask, s0=s0)
    o, S, _ = run_sparse(inp, mask=mask, s0=s0)
    eo, es = rel_max_err(o, o_ref), rel_max_err(S, S_ref)
    print(f"err O {eo:.3e} S {es:.3e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_all_events_exact_equals_dense(dtype):
    """All-ones mask with the exact solve reproduces the dense operator."""
    T = 64 * 6 + 17
    inp = synth.numpy_inputs(21, 1, T, 16, 32, dtype=dtype, decay_scale=1 / 64)
    mask = np.ones((1, 16, 7), np.uint8)
    o, S, _ = run_sparse(inp, solve="exact", mask=mask)
    o_ref, S_ref = gdn.chunk_prefill(inp.q, inp.k, inp.v, inp.a, inp.beta, None, "exact")
    assert rel_max_err(o, o_ref) <= TOL[dtype] and rel_max_err(S, S_ref) <= TOL[dtype]


def test_budget_one_equals_dense_blockadj():
    T = 64 * 10
    inp = synth.numpy_inputs(22, 1, T, 16, 32, dtype="bf16", with_z=True, decay_scale=1 / 32)
    o, S, st = run_sparse(inp, budget=1.0)
    assert st[0, 0] == 16 * 10
    o_ref, S_ref = gdn.chunk_prefill(inp.q, inp.k, inp.v, inp.a, inp.beta, None, "blockadj")
    assert rel_max_err(o, o_ref) <= TOL["bf16"] and rel_max_err(S, S_ref) <= TOL["bf16"]


def _mask_valid(mask, tier, C, budget=0.29):
    kL, kM, kH = selector.tier_counts(C, budget)
    k = {0: kL, 1: kM, 2: kH}
    for p in range(16):
        assert mask[p, 0] == 1 and mask[p, C - 1] == 1
        assert mask[p].sum() == k[int(tier[p])]
    nH = int((tier == 2).sum()); nM = int((tier == 1).sum())
    assert nH in (1, 2, 3, 4) and nM in selector.MEDIUM_CHOICES[nH]


@pytest.mark.parametrize("T,decay", [(4096, 1.0), (4096, 1 / 64), (64 * 37 + 19, 1 / 16)])
def test_selector_end_to_end(T, decay):
    """The whole sparse path with the on-device selector (gate energy, tail
    scores, ranking, tiers, CSR), checked in three parts:
    * the device statistics against the oracle's own (tolerance: they come
      from different arithmetic);
    * the oracle selector run on the device's fp32 statistics reproduces the
      device's mask and tiers bit for bit (identical inputs, identical
      integers);
    * O and S_final against the oracle prefill given the device's mask.
    The agreement of the device mask with the oracle's own selection (from
    the oracle's fp64 statistics) is printed as information only: near-ties
    of the rank key may flip at the top-k boundary."""
    import torch
    from gated_deltanet_prefill_chunkwise_amd import ops
    inp = synth.numpy_inputs(synth.seed_for(2) + T, 1, T, 16, 32, dtype="bf16", with_z=True,
                             decay_scale=decay)
    C = -(-T // 64)
    score = torch.empty((1, 32, C), device="cuda")
    gam = torch.empty((1, 32, C), device="cuda")
    eta = torch.empty((1, 32), device="cuda")
    mask = torch.empty((1, 16, C), dtype=torch.uint8, device="cuda")
    tier = torch.empty((1, 16), dtype=torch.uint8, device="cuda")
    dbg = ops.debug_struct(score=score, gamma=gam, eta=eta, mask=mask, tier=tier)
    o, S, st = run_sparse(inp, debug=dbg)
    o_own, S_own, info = oracle_sparse(inp)
    s_gpu, s_ref = host(score)[0], info["score"][0].astype(np.float64)
    assert np.max(np.abs(s_gpu - s_ref) / np.maximum(s_ref, 1e-6)) < 2e-2
    assert np.max(np.abs(host(eta)[0] - info["eta"][0]) / info["eta"][0]) < 1e-3
    m_gpu, t_gpu = mask.cpu().numpy()[0], tier.cpu().numpy()[0]
    ref = selector.select(score.cpu().numpy()[0], gam.cpu().numpy()[0], eta.cpu().numpy()[0],
                          keep_budget=0.29)
    assert np.array_equal(m_gpu, ref["mask"]), "mask"
    assert np.array_equal(t_gpu, ref["tier"]), "tier"
    _mask_valid(m_gpu, t_gpu, C)
    assert st[0, 0] == int(m_gpu.sum()) and st[0, 9] == 0 and st[0, 10] == 0
    o_ref, S_ref = sparse.sparse_prefill(inp.q, inp.k, inp.v, inp.a, inp.beta, solve="blockadj",
                                         mask=m_gpu[None])
    eo, es = rel_max_err(o, o_ref), rel_max_err(S, S_ref)
    flips = int((m_gpu != info["mask"][0]).sum())
    print(f"err O {eo:.3e} S {es:.3e}; mask entries differing from the oracle's own selection "
          f"(information only): {flips} of {m_gpu.size}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


def test_sparse_deterministic():
    inp = synth.numpy_inputs(31, 1, 64 * 20, 16, 32, dtype="bf16", with_z=True)
    a = run_sparse(inp)
    b = run_sparse(inp)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))


@pytest.mark.parametrize("B,T,budget", [(1, 64 * 71 + 3, 0.29), (3, 64 * 66 + 5, 0.29),
                                         (2, 64 * 67 + 1, 1.0), (1, 64 * 23 + 3, 0.29)])
def test_one_stream_schedule_equals_two_streams(B, T, budget):
    """Without a second stream every kernel runs on the caller's stream: the
    same products in the same order per head, so bit-identical outputs (one
    sequence and batches longer than 64 chunks, whose rows 4-15 are forked per
    sequence; keep 1.0 and sequences of at most 64 chunks keep one launch per
    stage)."""
    import torch
    from gated_deltanet_prefill_chunkwise_amd import ops
    inp = synth.numpy_inputs(33 + B, B, T, 16, 32, dtype="bf16", with_z=True,
                             decay_scale=1 / 16)
    d = to_device(inp)
    outs = []
    for aux in (True, False):
        o, S, st = ops.prefill_sparse(d["q"], d["k"], d["v"], d["a"], d["beta"], z=d["z"],
                                      keep_budget=budget, solve="blockadj", aux=aux)
        torch.cuda.synchronize()
        outs.append((o.cpu(), S.cpu(), st.cpu()))
    assert all(torch.equal(x, y) for x, y in zip(*outs))
