"""Device-side statistics of inputs outside the operator's domain.

The operator's domain (SparseGDN reading notes, Sec. 2.1): finite inputs,
log2 retention a <= 0.  The kernels flag violations in
sgdn_stats.nonfinite_input (which input) and non-finite results in
nonfinite_output (with finite inputs: an fp16 intermediate beyond 65504).
Every case here runs the kernels on ordinary (if out-of-range) numbers; the
selector orders NaN as -infinity, so its rankings stay permutations.
"""
import numpy as np
import pytest

from gated_deltanet_prefill_chunkwise_amd import synth

from helpers import to_device

pytestmark = pytest.mark.gpu

T = 64 * 6 + 9
NF_IN = {"q": 1, "k": 2, "v": 4, "a": 8, "beta": 16, "z": 32, "s0": 64}
NF_O, NF_S = 1, 2


def _inputs(seed=77):
    return synth.numpy_inputs(seed, 2, T, 16, 32, dtype="bf16", with_z=True, decay_scale=1 / 16)


def _run(mode, d, s0=None, out_dtype=None):
    import torch
    from gated_deltanet_prefill_chunkwise_amd import ops
    st = torch.full((2, ops.STATS_INTS), -7, dtype=torch.int32, device="cuda")
    if mode == "dense":
        o, S = ops.prefill_dense(d["q"], d["k"], d["v"], d["a"], d["beta"], s0=s0, solve="exact",
                                 stats=st, out_dtype=out_dtype)
    else:
        o, S, _ = ops.prefill_sparse(d["q"], d["k"], d["v"], d["a"], d["beta"], z=d["z"], s0=s0,
                                     keep_budget=0.29, solve="blockadj", stats=st,
                                     out_dtype=out_dtype)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), S.cpu().numpy(), st.cpu().numpy()


@pytest.mark.parametrize("mode", ["dense", "sparse"])
def test_clean_call_has_no_flags(mode):
    o, S, st = _run(mode, to_device(_inputs()))
    assert (st[:, 9:] == 0).all(), st
    assert np.isfinite(o).all() and np.isfinite(S).all()
    C = -(-T // 64)
    if mode == "dense":
        # every chunk of every pair an event, Nv (G - 1) group-entry states
        G = (C + 1) // 2
        assert st[:, :9].tolist() == [[16 * C, 16 * C, 0, 0, 0, 0, 0, 0, 32 * (G - 1)]] * 2


@pytest.mark.parametrize("mode", ["dense", "sparse"])
@pytest.mark.parametrize("what", ["q", "k", "v", "beta", "a_nan", "a_positive", "z", "s0"])
def test_input_flag(mode, what):
    """A NaN (or a positive decay) in one sequence's input sets that input's
    bit in that sequence's statistics only."""
    import torch
    if mode == "dense" and what == "z":
        pytest.skip("the dense path reads no gate")
    inp = _inputs(78)
    d = to_device(inp)
    s0 = None
    t, h = 200, 5
    if what in ("q", "k"):
        d[what][1, t, h // 2, 17] = float("nan")
    elif what in ("v", "z"):
        d[what][1, t, h, 3] = float("nan")
    elif what == "beta":
        d["beta"][1, t, h] = float("nan")
    elif what == "a_nan":
        d["a"][1, t, h] = float("nan")
    elif what == "a_positive":
        d["a"][1, t, h] = 0.25          # finite, but outside the domain
    elif what == "z":
        pass
    else:
        s0 = torch.zeros((2, 32, 128, 128), device="cuda")
        s0[1, h, 7, 9] = float("nan")
    if what == "z":
        # a position the gate energy samples: 64 c + 8 + 16 a, coordinate 73 (4c + a) mod 128
        c, a = 3, 1
        d["z"][1, 64 * c + 8 + 16 * a, h, (73 * (4 * c + a)) % 128] = float("nan")
    o, S, st = _run(mode, d, s0)
    bit = NF_IN[what.split("_")[0]]
    assert st[1, 9] & bit, (what, st[1])
    assert st[0, 9] == 0 and st[0, 10] == 0, st[0]           # the other sequence is clean
    assert np.isfinite(o[0]).all() and np.isfinite(S[0]).all()
    if what in ("q", "k", "v", "beta", "a_nan", "s0"):
        # a NaN reaches this sequence's outputs, and they are flagged
        assert not np.isfinite(o[1]).all() or not np.isfinite(S[1]).all()
        assert st[1, 10] != 0
    if mode == "sparse":
        E = st[:, 0]
        assert (E > 0).all() and (E <= st[:, 1]).all()       # a valid selection


@pytest.mark.parametrize("mode", ["dense", "sparse"])
def test_fp16_range_overflow_is_flagged(mode):
    """Finite inputs whose intermediates exceed the fp16 range (|v| ~ 1e5 with
    beta near 1) give non-finite outputs, flagged as such; the inputs are not."""
    inp = _inputs(79)
    d = to_device(inp)
    d["v"][0] = d["v"][0] * 1e5
    o, S, st = _run(mode, d)
    assert st[0, 9] == 0 and st[1, 9] == 0
    assert st[0, 10] & NF_O
    assert not np.isfinite(o[0]).all()
    assert st[1, 10] == 0 and np.isfinite(o[1]).all()


@pytest.mark.parametrize("mode", ["dense", "sparse"])
def test_fp16_output_overflow_is_flagged(mode):
    """fp32 inputs (fp32 intermediates) with |v| ~ 1e7: every intermediate and
    the fp32 output are finite, but an fp16 o cannot hold the outputs; the
    fp16 call flags nonfinite_output, the fp32 call does not."""
    import torch
    inp = synth.numpy_inputs(80, 2, T, 16, 32, dtype="f32", with_z=True, decay_scale=1 / 16)
    d = to_device(inp)
    d["v"][0] = d["v"][0] * 1e7
    o, S, st = _run(mode, d)
    assert (st[:, 9:] == 0).all(), st
    assert np.isfinite(o).all() and np.abs(o[0]).max() > 1e5
    o, S, st = _run(mode, d, out_dtype=torch.float16)
    assert st[0, 9] == 0 and st[1, 9] == 0
    assert st[0, 10] == NF_O and not np.isfinite(o[0]).all()
    assert st[1, 10] == 0 and np.isfinite(o[1]).all()
