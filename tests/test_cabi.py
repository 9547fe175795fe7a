"""The C ABI: libsgdn.so loads, exports every function include/sgdn.h declares,
and rejects bad arguments before enqueuing anything.  CPU only (no compute)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sgdn.h")


@pytest.fixture(scope="module")
def L():
    from gated_deltanet_prefill_chunkwise_amd import build, ops
    if not os.path.exists(ops.LIB_PATH):
        build.build()
    return ops.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sgdn_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(
        ["sgdn_workspace_bytes", "sgdn_event_capacity", "sgdn_prefill_dense", "sgdn_select",
         "sgdn_prefill_sparse", "sgdn_status_string", "sgdn_decode_step", "sgdn_fp64_selftest",
         "sgdn_select_noalloc"])


def test_struct_layouts_match_header(tmp_path):
    """The binding's ctypes mirrors of the header's structs have the sizes and
    field offsets a C compiler gives them (stats: 11 int32 words)."""
    from gated_deltanet_prefill_chunkwise_amd import ops
    assert ops.STATS_INTS == 11 and len(ops.STAT_FIELDS) == ops.STATS_INTS
    structs = {"sgdn_problem": ops.Problem, "sgdn_sparse_params": ops.SparseParams,
               "sgdn_stats": ops.Stats, "sgdn_debug": ops.Debug}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "sgdn.h"', "int main(void) {"]
    for cname, py in structs.items():
        lines.append(f'printf("{cname} %zu\\n", sizeof({cname}));')
        for f, _ in py._fields_:
            lines.append(f'printf("{cname}.{f} %zu\\n", offsetof({cname}, {f}));')
    lines.append("return 0; }")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    got = dict(line.split() for line in subprocess.run([str(exe)], capture_output=True,
                                                        text=True, check=True).stdout.splitlines())
    for cname, py in structs.items():
        assert int(got[cname]) == ctypes.sizeof(py), cname
        for f, _ in py._fields_:
            assert int(got[f"{cname}.{f}"]) == getattr(py, f).offset, f"{cname}.{f}"


def test_library_exports_every_declared_symbol(L):
    from gated_deltanet_prefill_chunkwise_amd import ops
    out = subprocess.run(["nm", "-D", "--defined-only", ops.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(L, name)


def _prob(**kw):
    from gated_deltanet_prefill_chunkwise_amd import ops
    base = dict(batch=1, seqlen=4096, n_qk=16, n_v=32, d_k=128, d_v=128, dtype=1, solve=0,
                o_dtype=0, cu_seqlens=None)
    base.update(kw)
    return ops.Problem(*[base[n] for n, _ in ops.Problem._fields_])


def test_workspace_bytes(L):
    from gated_deltanet_prefill_chunkwise_amd import ops
    p = _prob()
    dense = ops.workspace_bytes(p, False)
    sp = ops.workspace_bytes(p, True, ops.sparse_params())
    assert dense > 0 and sp > 0 and dense % 256 == 0
    # U alone: B * Nv * C * 64 * 128 bf16
    assert dense >= 32 * 64 * 64 * 128 * 2
    assert ops.workspace_bytes(_prob(d_k=64), False) == 0
    assert ops.workspace_bytes(_prob(n_v=20), False) == 0
    assert ops.workspace_bytes(_prob(n_qk=8, n_v=16), True, ops.sparse_params()) == 0
    assert ops.workspace_bytes(p, True, ops.sparse_params(keep_budget=0.0)) == 0
    assert ops.workspace_bytes(p, True, ops.sparse_params(keep_budget=1.5)) == 0


def test_event_capacity(L):
    """k_l of Eq. (13) and E_max = 16 k_H come from the library (the binding
    does none of that arithmetic); values as the oracle pins them."""
    from gated_deltanet_prefill_chunkwise_amd import ops
    from oracle import selector
    for T, budget in ((4096, 0.29), (32768, 0.29), (131072, 0.29), (64 * 35, 0.29),
                      (32768, 0.15), (32768, 0.5), (32768, 1.0), (64, 0.29), (100, 0.29)):
        k, e_max = ops.event_capacity(_prob(seqlen=T), ops.sparse_params(keep_budget=budget))
        C = -(-T // 64)
        assert k == selector.tier_counts(C, budget), (T, budget)
        assert e_max == 16 * k[2]
    assert ops.event_capacity(_prob(seqlen=32768), ops.sparse_params())[0] == (41, 154, 486)
    with pytest.raises(ops.SgdnError):
        ops.event_capacity(_prob(n_qk=8, n_v=16), ops.sparse_params())
    with pytest.raises(ops.SgdnError):
        ops.event_capacity(_prob(), ops.sparse_params(keep_budget=0.0))
    # the caller's tier rates replace the budget's (Eq. (13) with rho given)
    for T, rates in ((64 * 35, (0.1, 0.25, 0.5)), (32768, (0.08, 0.30, 0.95)),
                     (131072, (0.05, 0.2, 0.6)), (64, (0.01, 0.01, 1.0))):
        k, e_max = ops.event_capacity(_prob(seqlen=T), ops.sparse_params(0.5, tier_rate=rates))
        assert k == selector.tier_counts(-(-T // 64), tier_rate=rates), (T, rates)
        assert e_max == 16 * k[2]
    for bad in ((0.3, 0.2, 0.9), (0.0, 0.3, 0.9), (0.1, 0.3, 1.5), (float("nan"), 0.3, 0.9),
                (-0.1, 0.3, 0.9), (0.1, 0.3, float("inf"))):
        with pytest.raises(ops.SgdnError):
            ops.event_capacity(_prob(), ops.sparse_params(tier_rate=bad))
    e = ctypes.c_int32()
    assert L.sgdn_event_capacity(ctypes.byref(_prob()), ctypes.byref(ops.sparse_params()), None,
                                 None) == -1
    assert L.sgdn_event_capacity(ctypes.byref(_prob()), ctypes.byref(ops.sparse_params()), None,
                                 ctypes.byref(e)) == 0 and e.value == 16 * 61


def test_fp64_selftest_argument_errors(L):
    assert L.sgdn_fp64_selftest(None, None, None, None, -1, None) == -1
    assert L.sgdn_fp64_selftest(None, FAKE, FAKE, FAKE, 10, None) == -1
    assert L.sgdn_fp64_selftest(None, None, None, None, 0, None) == 0   # nothing to do


def test_status_strings(L):
    from gated_deltanet_prefill_chunkwise_amd import ops
    assert ops.status_string(0) == "ok"
    assert ops.status_string(-3) == "workspace too small"
    assert ops.status_string(-99) == "unknown status"


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation


def test_dense_argument_errors(L):
    def call(p, ws_bytes=1 << 40, q=FAKE, ws=FAKE):
        return L.sgdn_prefill_dense(ctypes.byref(p), q, FAKE, FAKE, FAKE, FAKE, None, FAKE, None,
                                    None, ws, ws_bytes, None, None)
    assert call(_prob(d_k=64)) == -2
    assert call(_prob(n_v=33)) == -2
    assert call(_prob(seqlen=0)) == -1
    assert call(_prob(dtype=7)) == -1
    assert call(_prob(solve=3)) == -1
    assert call(_prob(o_dtype=5)) == -1
    assert call(_prob(), q=None) == -1
    assert call(_prob(), ws=None) == -1
    assert call(_prob(), ws_bytes=1024) == -3
    assert L.sgdn_prefill_dense(None, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, None, FAKE,
                                1, None, None) == -1


def test_sparse_and_select_argument_errors(L):
    from gated_deltanet_prefill_chunkwise_amd import ops

    def sparse(p, params, z=FAKE, mask=None, ws_bytes=1 << 40):
        return L.sgdn_prefill_sparse(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, z,
                                     None if params is None else ctypes.byref(params), mask, None,
                                     FAKE, None, None, FAKE, ws_bytes, None, None)
    good = ops.sparse_params()
    assert sparse(_prob(), None) == -1
    assert sparse(_prob(n_qk=8, n_v=16), good) == -2
    assert sparse(_prob(), ops.sparse_params(keep_budget=0.0)) == -1
    assert sparse(_prob(), ops.sparse_params(tail=12)) == -2
    assert sparse(_prob(), ops.sparse_params(tail=128)) == -2
    bad = ops.sparse_params()
    bad.fixed_tiers = 2
    assert sparse(_prob(), bad) == -1
    bad = ops.sparse_params()
    bad.ablate = 32
    assert sparse(_prob(), bad) == -1
    assert sparse(_prob(cu_seqlens=0x2000), ops.sparse_params(ablate=("csr",))) == -2
    # the packed-W ablation is defined for the dense layout only
    assert sparse(_prob(cu_seqlens=0x2000), ops.sparse_params(ablate=("deferred_w",))) == -2
    assert sparse(_prob(), good, z=None) == -1               # no gate and no mask
    assert sparse(_prob(seqlen=64 * 8193), good) == -2       # C > 8192
    assert sparse(_prob(), good, ws_bytes=4096) == -3
    # a caller's second stream needs its two distinct fork / join events
    aux = ops.sparse_params()
    aux.aux_stream = 0x3000
    assert sparse(_prob(), aux) == -1
    aux.aux_events[0] = 0x4000
    assert sparse(_prob(), aux) == -1
    aux.aux_events[1] = 0x4000
    assert sparse(_prob(), aux) == -1

    def sel(p, params, score=FAKE):
        return L.sgdn_select(ctypes.byref(p), score, FAKE, FAKE, ctypes.byref(params), FAKE, FAKE,
                             FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 40, None)
    assert sel(_prob(), good, score=None) == -1
    assert sel(_prob(n_qk=4, n_v=8), good) == -2
    assert sel(_prob(), ops.sparse_params(r_window=8)) == -2


def test_select_noalloc_argument_errors(L):
    """Validation and the scratch-capacity refusal happen on the host, before
    the scratch is located or anything is enqueued."""
    from gated_deltanet_prefill_chunkwise_amd import ops

    def sel(p, params, score=FAKE):
        return L.sgdn_select_noalloc(ctypes.byref(p), score, FAKE, FAKE, ctypes.byref(params), FAKE,
                                     FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None)
    good = ops.sparse_params()
    assert sel(_prob(), good, score=None) == -1
    assert sel(_prob(n_qk=4, n_v=8), good) == -2
    assert sel(_prob(), ops.sparse_params(r_window=8)) == -2
    # 16 x 131072 tokens with a caller key: 6 MiB of selector scratch > 4 MiB
    keyed = ops.sparse_params()
    keyed.rank_key = 0x5000
    assert sel(_prob(batch=16, seqlen=131072), keyed) == -3
    assert sel(_prob(batch=17, seqlen=131072), good) == -3      # without a key: 4.35 MB
    assert ops.NOALLOC_SCRATCH_BYTES == 4 << 20


def test_decode_argument_errors(L):
    def call(p, s_in=FAKE, s_out=FAKE, q=FAKE):
        return L.sgdn_decode_step(ctypes.byref(p), q, FAKE, FAKE, FAKE, FAKE, s_in, s_out, FAKE,
                                  None)
    one = dict(seqlen=1)
    assert call(_prob(seqlen=2)) == -1                     # one token per sequence
    assert call(_prob(d_k=64, **one)) == -2
    assert call(_prob(n_qk=3, n_v=32, **one)) == -2        # Nv not a multiple of Nq
    assert call(_prob(dtype=4, **one)) == -1
    assert call(_prob(o_dtype=4, **one)) == -1
    assert call(_prob(batch=0, **one)) == -1
    assert call(_prob(**one), q=None) == -1
    assert call(_prob(**one), s_out=None) == -1
    # states that overlap without being the same buffer
    assert call(_prob(**one), s_out=ctypes.c_void_p(0x1000 + 4096)) == -1
    assert call(_prob(**one), s_in=ctypes.c_void_p(0x1004), s_out=ctypes.c_void_p(0x1004)) == -1
    assert L.sgdn_decode_step(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == -1
    assert call(_prob(cu_seqlens=0x2000, **one)) == -1      # packed offsets do not apply
