"""Workspace bounds: the library touches only the bytes sgdn_workspace_bytes
reports.  The workspace is handed over as the head of a larger buffer whose
tail is filled with a guard pattern; after dense and sparse calls on ragged
multi-chunk inputs (several of each kernel's tiles) the guard must be intact,
and the outputs must equal those computed with a workspace of exactly the
reported size.
"""
import numpy as np
import pytest

from gated_deltanet_prefill_chunkwise_amd import synth

pytestmark = pytest.mark.gpu

GUARD = 1 << 20


def _guarded(nbytes):
    import torch
    buf = torch.full((nbytes + GUARD,), 0xA5, dtype=torch.uint8, device="cuda")
    return buf, buf[:nbytes]


@pytest.mark.parametrize("mode", ["dense", "sparse"])
@pytest.mark.parametrize("T", [64 * 9 + 21, 4096 + 37])
def test_workspace_guard(mode, T):
    import torch
    from gated_deltanet_prefill_chunkwise_amd import ops
    d = synth.torch_inputs(synth.seed_for(11, T), 1, T, 16, 32, dtype="bf16", with_z=True)
    prob = ops.problem(d["q"], d["v"], "blockadj", torch.float32)
    sparse = mode == "sparse"
    nbytes = ops.workspace_bytes(prob, sparse, ops.sparse_params() if sparse else None)
    assert nbytes > 0
    buf, ws = _guarded(nbytes)

    def run(workspace):
        if sparse:
            o, s, _ = ops.prefill_sparse(d["q"], d["k"], d["v"], d["a"], d["beta"], z=d["z"],
                                         keep_budget=0.29, solve="blockadj", workspace=workspace)
        else:
            o, s = ops.prefill_dense(d["q"], d["k"], d["v"], d["a"], d["beta"], solve="blockadj",
                                     workspace=workspace)
        torch.cuda.synchronize()
        return o.cpu(), s.cpu()

    o1, s1 = run(ws)
    tail = buf[nbytes:].cpu().numpy()
    assert np.all(tail == 0xA5), f"{mode}: {int(np.sum(tail != 0xA5))} guard bytes overwritten"
    exact = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    o2, s2 = run(exact)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
