"""GPU parity of the dense prefill (sgdn_prefill_dense) against the fp64 oracle.

Bar: max |O_gpu - O_ref| / rms(O_ref) <= 2e-2 for bf16 inputs, 1e-4 for fp32
(same for the final state)."""
import numpy as np
import pytest

from gated_deltanet_prefill_chunkwise_amd import synth
from oracle import gdn

from helpers import TOL, host, rel_max_err, to_device

pytestmark = pytest.mark.gpu


def run_dense(inp, solve, s0=None, debug=None):
    import torch
    from gated_deltanet_prefill_chunkwise_amd import ops
    d = to_device(inp)
    s0d = None if s0 is None else torch.from_numpy(s0.astype(np.float32)).cuda()
    o, S = ops.prefill_dense(d["q"], d["k"], d["v"], d["a"], d["beta"], s0=s0d, solve=solve,
                             debug=debug)
    torch.cuda.synchronize()
    return host(o), host(S)


def check(inp, solve, s0=None, ref="chunk"):
    o, S = run_dense(inp, solve, s0)
    if ref == "recurrence":
        o_ref, S_ref = gdn.recurrence(inp.q, inp.k, inp.v, inp.a, inp.beta, s0)
    else:
        o_ref, S_ref = gdn.chunk_prefill(inp.q, inp.k, inp.v, inp.a, inp.beta, s0, solve)
    eo, es = rel_max_err(o, o_ref), rel_max_err(S, S_ref)
    print(f"err O {eo:.3e}  S {es:.3e}")
    tol = TOL[inp.dtype]
    assert eo <= tol and es <= tol, (eo, es)
    return eo, es


def test_config0_fp32_exact_matches_recurrence():
    """B1, T256, one q/k head with 2 value heads, fp32, exact solve."""
    inp = synth.numpy_inputs(synth.seed_for(0), 1, 256, 1, 2, dtype="f32")
    check(inp, "exact", ref="recurrence")


@pytest.mark.parametrize("T", [1, 37, 64, 65, 200, 64 * 5 + 37])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("solve", ["exact", "blockadj"])
def test_ragged_lengths(T, dtype, solve):
    inp = synth.numpy_inputs(100 + T, 1, T, 2, 4, dtype=dtype)
    check(inp, solve)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("solve", ["exact", "blockadj"])
def test_slow_decay_with_initial_state(dtype, solve):
    """a / 64 keeps the state alive across chunks so H and the snapshots matter."""
    inp = synth.numpy_inputs(7, 2, 64 * 9 + 11, 2, 4, dtype=dtype, decay_scale=1 / 64)
    s0 = np.random.default_rng(3).standard_normal((2, 4, 128, 128)) * 0.05
    check(inp, solve, s0=s0.astype(np.float32).astype(np.float64))


@pytest.mark.parametrize("solve", ["exact", "blockadj"])
def test_config1_full_layer(solve):
    """B1, T4096, Nq16 / Nv32, bf16 (exact and block-adjacent)."""
    inp = synth.numpy_inputs(synth.seed_for(1), 1, 4096, 16, 32, dtype="bf16")
    check(inp, solve)


def test_config1_slow_decay():
    inp = synth.numpy_inputs(synth.seed_for(1) + 1, 1, 4096, 16, 32, dtype="bf16", decay_scale=1 / 64)
    check(inp, "exact")


def test_debug_stage_outputs():
    import torch
    from gated_deltanet_prefill_chunkwise_amd import ops
    inp = synth.numpy_inputs(11, 1, 64 * 3 + 5, 2, 4, dtype="f32", decay_scale=1 / 8)
    B, T, Nq, Nv = 1, inp.q.shape[1], 2, 4
    C = -(-T // 64)
    g = torch.empty((B, Nv, C, 64), device="cuda")
    gam = torch.empty((B, Nv, C), device="cuda")
    pre = torch.empty((B, Nv, C + 1), dtype=torch.float64, device="cuda")
    U = torch.empty((B, Nv, C, 64, 128), device="cuda")
    dbg = ops.debug_struct(g=g, gamma=gam, prefix=pre, U=U)
    run_dense(inp, "exact", debug=dbg)
    g_ref, gam_ref, P_ref = gdn.decay_prefix(inp.a)
    np.testing.assert_allclose(host(g), g_ref, rtol=1e-5, atol=1e-4)
    np.testing.assert_allclose(host(gam), gam_ref, rtol=1e-5, atol=1e-4)
    np.testing.assert_allclose(host(pre), P_ref, rtol=1e-5, atol=1e-4)
    hq = np.arange(Nv) // 2
    U_ref = gdn.intra(gdn.chunk_view(inp.k, hq), gdn.chunk_view(inp.v), gdn.chunk_scalar(inp.beta),
                      g_ref, "exact")[0]
    assert rel_max_err(host(U), U_ref) <= 1e-4


def test_deterministic():
    inp = synth.numpy_inputs(12, 1, 1000, 4, 8, dtype="bf16", decay_scale=1 / 16)
    o1, S1 = run_dense(inp, "exact")
    o2, S2 = run_dense(inp, "exact")
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)


@pytest.mark.parametrize("solve", ["exact", "blockadj"])
def test_fp16_output(solve):
    """o in fp16 (the benchmark's output type): the plain bf16-input bar, with
    the output's own rounding (at most 2^-11 of the element) inside it."""
    import torch
    from gated_deltanet_prefill_chunkwise_amd import ops
    inp = synth.numpy_inputs(synth.seed_for(1) + 8, 1, 2048 + 40, 16, 32, dtype="bf16")
    d = to_device(inp)
    o, S = ops.prefill_dense(d["q"], d["k"], d["v"], d["a"], d["beta"], solve=solve,
                             out_dtype=torch.float16)
    torch.cuda.synchronize()
    assert o.dtype == torch.float16
    o_ref, S_ref = gdn.chunk_prefill(inp.q, inp.k, inp.v, inp.a, inp.beta, None, solve)
    eo, es = rel_max_err(host(o), o_ref), rel_max_err(host(S), S_ref)
    print(f"fp16 o: err O {eo:.3e} S {es:.3e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


@pytest.mark.parametrize("solve", ["exact", "blockadj"])
def test_bf16_output(solve):
    """o in bf16: the bar is the fp32 bar plus the output's own rounding
    (half a bf16 ulp, at most 2^-8 of the element)."""
    import torch
    from gated_deltanet_prefill_chunkwise_amd import ops
    inp = synth.numpy_inputs(synth.seed_for(1) + 7, 1, 2048 + 40, 16, 32, dtype="bf16")
    d = to_device(inp)
    o, S = ops.prefill_dense(d["q"], d["k"], d["v"], d["a"], d["beta"], solve=solve,
                             out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert o.dtype == torch.bfloat16
    o_ref, S_ref = gdn.chunk_prefill(inp.q, inp.k, inp.v, inp.a, inp.beta, None, solve)
    rms = np.sqrt(np.mean(o_ref ** 2))
    excess = np.abs(host(o) - o_ref) - 2.0 ** -8 * np.abs(o_ref)
    print(f"max excess over the output rounding {excess.max() / rms:.3e}")
    assert excess.max() <= TOL["bf16"] * rms
