"""GPU parity of the single-token decode step (sgdn_decode_step) against the
fp64 oracle's decode step, on its own and continuing a GPU prefill.

Bar: max |x_gpu - x_ref| / rms(x_ref) <= 2e-2 for bf16 inputs, 1e-4 for fp32,
for the output and the new state; a bf16 output adds its own rounding.
"""
import numpy as np
import pytest

from gated_deltanet_prefill_chunkwise_amd import synth
from oracle import gdn

from helpers import TOL, host, rel_max_err

pytestmark = pytest.mark.gpu


def _token(seed, B, Nq, Nv, dtype):
    """One token per sequence: the prefill recipe at T = 1, token axis dropped."""
    inp = synth.numpy_inputs(seed, B, 1, Nq, Nv, dtype=dtype)
    return {n: getattr(inp, n)[:, 0] for n in ("q", "k", "v", "a", "beta")}


def _state(seed, B, Nv, scale=0.3):
    s = np.random.default_rng(seed).standard_normal((B, Nv, 128, 128)) * scale
    return s.astype(np.float32).astype(np.float64)


def _dev(x, dtype):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    return t.to(torch.bfloat16 if dtype == "bf16" else torch.float32)


def _run(tok, s, dtype, inplace=False, out_dtype=None):
    import torch
    from gated_deltanet_prefill_chunkwise_amd import ops
    d = {n: _dev(tok[n], dtype) for n in ("q", "k", "v", "beta")}
    a = torch.from_numpy(np.ascontiguousarray(tok["a"], np.float32)).cuda()
    st = torch.from_numpy(s.astype(np.float32)).cuda()
    o, S = ops.decode_step(d["q"], d["k"], d["v"], a, d["beta"], st,
                           s_out=st if inplace else None, out_dtype=out_dtype)
    torch.cuda.synchronize()
    if inplace:
        assert S.data_ptr() == st.data_ptr()
    return host(o), host(S)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,Nq,Nv", [(1, 16, 32), (3, 16, 32), (2, 4, 16), (2, 8, 8)])
def test_decode_step_matches_oracle(dtype, B, Nq, Nv):
    tok = _token(900 + B + Nv, B, Nq, Nv, dtype)
    s = _state(901 + B, B, Nv)
    o, S = _run(tok, s, dtype)
    o_ref, S_ref = gdn.decode_step(tok["q"], tok["k"], tok["v"], tok["a"], tok["beta"], s)
    eo, es = rel_max_err(o, o_ref), rel_max_err(S, S_ref)
    print(f"err O {eo:.3e}  S {es:.3e}")
    assert eo <= TOL[dtype] and es <= TOL[dtype]


def test_decode_step_in_place_is_identical():
    tok = _token(910, 2, 16, 32, "bf16")
    s = _state(911, 2, 32)
    o1, S1 = _run(tok, s, "bf16")
    o2, S2 = _run(tok, s, "bf16", inplace=True)
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)


def test_decode_step_bf16_output():
    import torch
    tok = _token(920, 2, 16, 32, "bf16")
    s = _state(921, 2, 32)
    o, _ = _run(tok, s, "bf16", out_dtype=torch.bfloat16)
    o_ref, _ = gdn.decode_step(tok["q"], tok["k"], tok["v"], tok["a"], tok["beta"], s)
    rms = np.sqrt(np.mean(o_ref ** 2))
    assert np.all(np.abs(o - o_ref) <= TOL["bf16"] * rms + 2.0 ** -8 * np.abs(o_ref))


def test_decode_step_fp16_output():
    import torch
    tok = _token(922, 2, 16, 32, "bf16")
    s = _state(923, 2, 32)
    o, _ = _run(tok, s, "bf16", out_dtype=torch.float16)
    o_ref, _ = gdn.decode_step(tok["q"], tok["k"], tok["v"], tok["a"], tok["beta"], s)
    assert rel_max_err(o, o_ref) <= TOL["bf16"]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_continues_gpu_prefill(dtype):
    """GPU dense prefill over T tokens, then three GPU decode steps from its
    final state, against the oracle recurrence over all T + 3 tokens."""
    import torch
    from gated_deltanet_prefill_chunkwise_amd import ops
    T, n = 64 * 3 + 17, 3
    inp = synth.numpy_inputs(930, 2, T + n, 2, 4, dtype=dtype, decay_scale=1 / 16)
    dev = lambda x: _dev(x, dtype)
    a = torch.from_numpy(np.ascontiguousarray(inp.a)).cuda()
    _, S = ops.prefill_dense(dev(inp.q[:, :T]), dev(inp.k[:, :T]), dev(inp.v[:, :T]),
                             a[:, :T].contiguous(), dev(inp.beta[:, :T]), solve="exact")
    outs = []
    for t in range(T, T + n):
        o, S = ops.decode_step(dev(inp.q[:, t]), dev(inp.k[:, t]), dev(inp.v[:, t]),
                               a[:, t].contiguous(), dev(inp.beta[:, t]), S, s_out=S)
        outs.append(host(o))
    torch.cuda.synchronize()
    o_ref, S_ref = gdn.recurrence(inp.q, inp.k, inp.v, inp.a, inp.beta)
    for i, o in enumerate(outs):
        e = rel_max_err(o, o_ref[:, T + i])
        print(f"decode {i}: err O {e:.3e}")
        assert e <= TOL[dtype]
    es = rel_max_err(host(S), S_ref)
    print(f"err S {es:.3e}")
    assert es <= TOL[dtype]


def test_decode_step_large_batch_sampled():
    """B = 128 sequences x 32 heads (4096 heads, 16384 workgroups); the oracle
    checks a sample of 24 heads."""
    B, Nq, Nv = 128, 16, 32
    tok = _token(940, B, Nq, Nv, "bf16")
    s = np.random.default_rng(941).standard_normal((B, Nv, 128, 128)).astype(np.float32) * 0.3
    o, S = _run(tok, s, "bf16")
    rng = np.random.default_rng(942)
    for bh in rng.choice(B * Nv, 24, replace=False):
        b, h = divmod(int(bh), Nv)
        hq = h // (Nv // Nq)
        o_ref, S_ref = gdn.decode_step(tok["q"][b:b + 1, hq:hq + 1], tok["k"][b:b + 1, hq:hq + 1],
                                       tok["v"][b:b + 1, h:h + 1], tok["a"][b:b + 1, h:h + 1],
                                       tok["beta"][b:b + 1, h:h + 1],
                                       s[b:b + 1, h:h + 1].astype(np.float64))
        assert rel_max_err(o[b, h], o_ref[0, 0]) <= TOL["bf16"]
        assert rel_max_err(S[b, h], S_ref[0, 0]) <= TOL["bf16"]
