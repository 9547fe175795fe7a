"""sgdn_select_noalloc: the selector with its scratch in the library's static
device array (no workspace argument) gives exactly sgdn_select's results.
Two calls in a row, the second with a smaller input (fewer sequences and
chunks, so the scratch holds the first call's larger contents), each
compared with sgdn_select on the same statistics; then the oracle selector
on the same inputs (bit-exact, as for sgdn_select).  A problem beyond the
scratch's capacity is refused before anything is enqueued."""
import numpy as np
import pytest

from gated_deltanet_prefill_chunkwise_amd import synth
from oracle import selector

pytestmark = pytest.mark.gpu


def _run(seed, B, C, budget, key=False):
    import torch
    from gated_deltanet_prefill_chunkwise_amd import ops
    score, gamma, eta = synth.selector_stats(seed, B, C)
    t = lambda x: torch.from_numpy(x).cuda()
    rk = None
    if key:
        rk = t(np.random.default_rng(seed).uniform(size=(B, 16, C)).astype(np.float32))
    ref = ops.select(t(score), t(gamma), t(eta), keep_budget=budget, rank_key=rk)
    got = ops.select(t(score), t(gamma), t(eta), keep_budget=budget, rank_key=rk, noalloc=True)
    torch.cuda.synchronize()
    for name in ref:
        assert torch.equal(ref[name], got[name]), name
    got = {k: v.cpu().numpy() for k, v in got.items()}
    for b in range(B):
        o = selector.select(score[b], gamma[b], eta[b], keep_budget=budget,
                            rank_key=None if rk is None else rk[b].cpu().numpy())
        assert np.array_equal(got["mask"][b], o["mask"]) and np.array_equal(got["tier"][b], o["tier"])
    return got


def test_noalloc_select_matches_workspace_select_twice():
    a = _run(611, 8, 2048, 0.29)       # the largest: 8 sequences of 131072 tokens
    b = _run(612, 2, 300, 0.5)         # then smaller, over the first call's contents
    assert a["stats"][:, 0].min() > 0 and b["stats"][:, 0].min() > 0
    _run(613, 3, 77, 0.15, key=True)   # the caller-key ranking (second rank table)


def test_noalloc_select_refuses_beyond_scratch():
    import torch
    from gated_deltanet_prefill_chunkwise_amd import ops
    B, C = 16, 2048                    # 32768 sequence-chunks: beyond the 4 MiB scratch
    z = torch.zeros((B, 32, C), device="cuda")
    with pytest.raises(ops.SgdnError) as e:
        ops.select(z, z, torch.ones((B, 32), device="cuda"), noalloc=True,
                   rank_key=torch.zeros((B, 16, C), device="cuda"))
    assert e.value.status == -3
