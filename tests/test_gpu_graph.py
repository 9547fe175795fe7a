"""HIP-graph capture of the prefill calls: a captured call (the sparse one
with and without the caller's second stream, which it forks to and joins
back from) replays to the eager result, several times, with eager work and
synchronisation between replays.  The library holds no stream of its own,
so the first call can itself be captured.
"""
import numpy as np
import pytest

from gated_deltanet_prefill_chunkwise_amd import synth

from helpers import to_device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("mode", ["sparse", "sparse_one_stream", "dense"])
def test_prefill_graph_replay_matches_eager(mode):
    import torch
    from gated_deltanet_prefill_chunkwise_amd import ops
    inp = synth.numpy_inputs(4100, 1, 64 * 9 + 5, 16, 32, dtype="bf16", with_z=True,
                             decay_scale=1 / 16)
    d = to_device(inp)
    prob = ops.problem(d["q"], d["v"], "blockadj", torch.float32)
    sp = mode.startswith("sparse")
    nbytes = ops.workspace_bytes(prob, sp, ops.sparse_params() if sp else None)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    o = torch.empty(d["v"].shape, dtype=torch.float32, device="cuda")
    S = torch.empty((1, 32, 128, 128), dtype=torch.float32, device="cuda")
    st = torch.zeros((1, ops.STATS_INTS), dtype=torch.int32, device="cuda")

    def call():
        if sp:
            ops.prefill_sparse(d["q"], d["k"], d["v"], d["a"], d["beta"], z=d["z"], keep_budget=0.29,
                               solve="blockadj", o=o, s_final=S, stats=st, workspace=ws,
                               aux=mode == "sparse")
        else:
            ops.prefill_dense(d["q"], d["k"], d["v"], d["a"], d["beta"], solve="blockadj", o=o,
                              s_final=S, stats=st, workspace=ws)

    call()                                   # eager
    torch.cuda.synchronize()
    o_ref, S_ref, st_ref = o.clone(), S.clone(), st.clone()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for _ in range(3):
        o.zero_()
        S.zero_()
        st.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(S, S_ref)
        assert torch.equal(st, st_ref)
    assert np.isfinite(o_ref.cpu().numpy()).all()
