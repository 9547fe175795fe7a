"""Packed variable-length batches (sgdn_problem.cu_seqlens).

Every sequence of a packed call must give what the oracle gives for that
sequence alone (its own chunks, its own s0 / final state and, in the sparse
path, its own valid chunks for the selector).  A packed call of equal-length
sequences must also reproduce the dense-layout call bit for bit.
Lengths cover the edge cases: empty, 1, exactly one chunk, one chunk plus a
token, ragged tails, and sequences much shorter than the longest.
"""
import numpy as np
import pytest

from gated_deltanet_prefill_chunkwise_amd import synth
from oracle import gdn, selector, sparse

from helpers import TOL, host, rel_max_err

pytestmark = pytest.mark.gpu


def _seq_inputs(seed, lens, Nq, Nv, dtype, with_z=False, decay=1.0):
    """One synthetic draw per sequence (the prefill recipe), cut to its length."""
    out = []
    for i, n in enumerate(lens):
        x = synth.numpy_inputs(seed + 17 * i, 1, max(n, 1), Nq, Nv, dtype=dtype, with_z=with_z,
                               decay_scale=decay)
        out.append({f: None if getattr(x, f) is None else getattr(x, f)[:, :n]
                    for f in ("q", "k", "v", "a", "beta", "z")})
    return out


def _packed(seqs, dtype):
    """Concatenate along the token axis: [1, N_tok, ...] device tensors."""
    import torch
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    d = {}
    for f in ("q", "k", "v", "beta", "z", "a"):
        if seqs[0][f] is None:
            d[f] = None
            continue
        x = np.concatenate([s[f] for s in seqs], axis=1)
        t = torch.from_numpy(np.ascontiguousarray(x)).cuda()
        d[f] = t.float() if f == "a" else t.to(tdt)
    return d


def _cu(lens):
    import torch
    return torch.tensor(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32), device="cuda")


def _rows(o, lens, i):
    cu = np.concatenate([[0], np.cumsum(lens)])
    return o[:, cu[i]:cu[i + 1]]


LENS = [1, 64, 65, 200, 0, 131, 7, 64 * 4 + 63]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("solve", ["exact", "blockadj"])
def test_dense_varlen_matches_each_sequence(dtype, solve):
    import torch
    from gated_deltanet_prefill_chunkwise_amd import ops
    seqs = _seq_inputs(500, LENS, 2, 4, dtype, decay=1 / 16)
    d = _packed(seqs, dtype)
    B = len(LENS)
    s0 = (np.random.default_rng(501).standard_normal((B, 4, 128, 128)) * 0.05).astype(np.float32)
    o, S = ops.prefill_dense(d["q"], d["k"], d["v"], d["a"], d["beta"], solve=solve,
                             s0=torch.from_numpy(s0).cuda(), cu_seqlens=_cu(LENS))
    torch.cuda.synchronize()
    o, S = host(o), host(S)
    assert o.shape[1] == sum(LENS)
    for i, (n, x) in enumerate(zip(LENS, seqs)):
        s0i = s0[i:i + 1].astype(np.float64)
        if n == 0:
            assert np.array_equal(S[i:i + 1], s0i), "empty sequence keeps its state"
            continue
        o_ref, S_ref = gdn.chunk_prefill(x["q"], x["k"], x["v"], x["a"], x["beta"], s0i, solve)
        eo, es = rel_max_err(_rows(o, LENS, i), o_ref), rel_max_err(S[i:i + 1], S_ref)
        print(f"seq {i} (T={n}): err O {eo:.3e} S {es:.3e}")
        assert eo <= TOL[dtype] and es <= TOL[dtype]


@pytest.mark.parametrize("mode", ["dense", "sparse"])
def test_equal_lengths_packed_is_bitwise_dense_layout(mode):
    import torch
    from gated_deltanet_prefill_chunkwise_amd import ops
    B, T = 3, 64 * 5 + 9
    x = synth.numpy_inputs(510, B, T, 16, 32, dtype="bf16", with_z=True, decay_scale=1 / 16)
    tdt = torch.bfloat16
    dev = {f: torch.from_numpy(np.ascontiguousarray(getattr(x, f))).cuda().to(tdt)
           for f in ("q", "k", "v", "beta", "z")}
    dev["a"] = torch.from_numpy(np.ascontiguousarray(x.a)).cuda()
    flat = {f: t.reshape(1, B * T, *t.shape[2:]) for f, t in dev.items()}
    cu = _cu([T] * B)
    if mode == "dense":
        run = lambda d, **kw: ops.prefill_dense(d["q"], d["k"], d["v"], d["a"], d["beta"],
                                                solve="exact", **kw)
    else:
        run = lambda d, **kw: ops.prefill_sparse(d["q"], d["k"], d["v"], d["a"], d["beta"],
                                                 z=d["z"], keep_budget=0.29, **kw)
    r1 = run(dev)
    r2 = run(flat, cu_seqlens=cu, max_seqlen=T)
    torch.cuda.synchronize()
    assert torch.equal(r1[0].reshape(1, B * T, 32, 128), r2[0])
    assert torch.equal(r1[1], r2[1])
    if mode == "sparse":
        assert torch.equal(r1[2], r2[2])


SPARSE_LENS = [64 * 6 + 5, 64 * 13, 1, 0, 64 * 3 + 40, 64, 64 * 2 + 1]


def test_select_varlen_bit_exact():
    """sgdn_select with per-sequence valid chunks: every sequence equals the
    oracle's selection on its own chunks; chunks and groups past its end are
    empty."""
    import torch
    from gated_deltanet_prefill_chunkwise_amd import ops
    C = 40
    lens = [64 * 40, 64 * 7 + 3, 1, 0, 64 * 2, 64 * 25 + 60]
    B = len(lens)
    score, gamma, eta = synth.selector_stats(520, B, C)
    out = ops.select(torch.from_numpy(score).cuda(), torch.from_numpy(gamma).cuda(),
                     torch.from_numpy(eta).cuda(), keep_budget=0.29, cu_seqlens=_cu(lens))
    torch.cuda.synchronize()
    out = {k: v.cpu().numpy() for k, v in out.items()}
    for b, n in enumerate(lens):
        Cb = -(-n // 64)
        Gb = (Cb + 1) // 2
        assert not out["mask"][b, :, Cb:].any()
        assert np.all(out["pred"][b, :, Gb:] == -1) and np.all(out["group_slot"][b, :, Gb:] == -1)
        if Cb == 0:
            assert out["row_ptr"][b, -1] == 0 and out["stats"][b, 0] == 0
            continue
        ref = selector.select(score[b, :, :Cb], gamma[b, :, :Cb], eta[b], keep_budget=0.29)
        lay = selector.event_layout(ref["mask"], ref["tier"])
        assert np.array_equal(out["mask"][b, :, :Cb], ref["mask"]), b
        assert np.array_equal(out["tier"][b], ref["tier"]), b
        assert np.array_equal(out["row_pair"][b], lay["row_pair"]), b
        assert np.array_equal(out["row_ptr"][b], lay["row_ptr"]), b
        assert np.array_equal(out["col"][b, :lay["E"]], lay["col"]), b
        assert np.array_equal(out["pred"][b, :, :Gb], lay["pred"]), b
        assert np.array_equal(out["group_slot"][b, :, :Gb], lay["group_slot"]), b
        kL, kM, kH = ref["k"]
        assert out["stats"][b, 5:8].tolist() == [kL, kM, kH], b


@pytest.mark.parametrize("with_s0", [False, True])
def test_sparse_varlen_matches_each_sequence(with_s0):
    """End to end with the on-device selector: each sequence's mask is the
    oracle selector's on the GPU's own fp32 statistics for that sequence, and
    O and the final state match the oracle given that mask; with an initial
    state per sequence, an empty sequence hands its s0 back unchanged."""
    import torch
    from gated_deltanet_prefill_chunkwise_amd import ops
    lens = SPARSE_LENS
    B = len(lens)
    seqs = _seq_inputs(530, lens, 16, 32, "bf16", with_z=True, decay=1 / 16)
    d = _packed(seqs, "bf16")
    T = max(lens)
    C = -(-T // 64)
    score = torch.empty((B, 32, C), device="cuda")
    gam = torch.empty((B, 32, C), device="cuda")
    eta = torch.empty((B, 32), device="cuda")
    mask = torch.empty((B, 16, C), dtype=torch.uint8, device="cuda")
    tier = torch.empty((B, 16), dtype=torch.uint8, device="cuda")
    dbg = ops.debug_struct(score=score, gamma=gam, eta=eta, mask=mask, tier=tier)
    s0 = (np.random.default_rng(531).standard_normal((B, 32, 128, 128)) * 0.05).astype(np.float32) \
        if with_s0 else None
    o, S, st = ops.prefill_sparse(d["q"], d["k"], d["v"], d["a"], d["beta"], z=d["z"],
                                  keep_budget=0.29, solve="blockadj", debug=dbg,
                                  s0=None if s0 is None else torch.from_numpy(s0).cuda(),
                                  cu_seqlens=_cu(lens))
    torch.cuda.synchronize()
    o, S, st = host(o), host(S), st.cpu().numpy()
    sc, gm, et = score.cpu().numpy(), gam.cpu().numpy(), eta.cpu().numpy()
    m_gpu, t_gpu = mask.cpu().numpy(), tier.cpu().numpy()
    for i, (n, x) in enumerate(zip(lens, seqs)):
        Cb = -(-n // 64)
        assert not m_gpu[i, :, Cb:].any()
        if n == 0:
            assert st[i, 0] == 0
            assert np.array_equal(S[i], s0[i]) if with_s0 else not S[i].any()
            continue
        ref = selector.select(sc[i, :, :Cb], gm[i, :, :Cb], et[i], keep_budget=0.29)
        assert np.array_equal(m_gpu[i, :, :Cb], ref["mask"]), i
        assert np.array_equal(t_gpu[i], ref["tier"]), i
        assert st[i, 0] == int(ref["mask"].sum())
        o_ref, S_ref = sparse.sparse_prefill(x["q"], x["k"], x["v"], x["a"], x["beta"],
                                             solve="blockadj", mask=ref["mask"][None],
                                             s0=None if s0 is None else s0[i:i + 1].astype(np.float64))
        eo, es = rel_max_err(_rows(o, lens, i), o_ref), rel_max_err(S[i:i + 1], S_ref)
        print(f"seq {i} (T={n}, {st[i, 0]} events): err O {eo:.3e} S {es:.3e}")
        assert eo <= TOL["bf16"] and es <= TOL["bf16"]


def test_sparse_varlen_one_stream_equals_two_streams():
    """The forked schedule (CSR rows 4-15 of every packed sequence on the
    second stream) computes the same products in the same order per head as
    the one-stream schedule: bit-identical outputs and statistics (the longest
    sequence has more than 64 chunks, so the fork applies)."""
    import torch
    from gated_deltanet_prefill_chunkwise_amd import ops
    lens = [64 * 80 + 5, 64 * 13, 1, 0, 64 * 70 + 40, 64, 64 * 2 + 1]
    d = _packed(_seq_inputs(540, lens, 16, 32, "bf16", with_z=True, decay=1 / 16), "bf16")
    outs = []
    for aux in (True, False):
        r = ops.prefill_sparse(d["q"], d["k"], d["v"], d["a"], d["beta"], z=d["z"],
                               keep_budget=0.29, solve="blockadj", cu_seqlens=_cu(lens), aux=aux)
        torch.cuda.synchronize()
        outs.append([t.cpu() for t in r])
    assert all(torch.equal(x, y) for x, y in zip(*outs))
