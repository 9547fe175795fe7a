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
        ["sgdn_workspace_bytes", "sgdn_prefill_dense", "sgdn_select", "sgdn_prefill_sparse",
         "sgdn_status_string", "sgdn_decode_step"])


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


def test_status_strings(L):
    from gated_deltanet_prefill_chunkwise_amd import ops
    assert ops.status_string(0) == "ok"
    assert ops.status_string(-3) == "workspace too small"
    assert ops.status_string(-99) == "unknown status"


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation


def test_dense_argument_errors(L):
    def call(p, ws_bytes=1 << 40, q=FAKE, ws=FAKE):
        return L.sgdn_prefill_dense(ctypes.byref(p), q, FAKE, FAKE, FAKE, FAKE, None, FAKE, None,
                                    ws, ws_bytes, None, None)
    assert call(_prob(d_k=64)) == -2
    assert call(_prob(n_v=33)) == -2
    assert call(_prob(seqlen=0)) == -1
    assert call(_prob(dtype=7)) == -1
    assert call(_prob(solve=3)) == -1
    assert call(_prob(o_dtype=5)) == -1
    assert call(_prob(), q=None) == -1
    assert call(_prob(), ws=None) == -1
    assert call(_prob(), ws_bytes=1024) == -3
    assert L.sgdn_prefill_dense(None, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, FAKE, 1,
                                None, None) == -1


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

    def sel(p, params, score=FAKE):
        return L.sgdn_select(ctypes.byref(p), score, FAKE, FAKE, ctypes.byref(params), FAKE, FAKE,
                             FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 40, None)
    assert sel(_prob(), good, score=None) == -1
    assert sel(_prob(n_qk=4, n_v=8), good) == -2
    assert sel(_prob(), ops.sparse_params(r_window=8)) == -2


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
