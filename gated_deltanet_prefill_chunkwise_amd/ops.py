"""Thin Python binding of libsgdn.so (C ABI in include/sgdn.h).

Argument marshalling only: every step of the prefill runs in the library's HIP
kernels.  Tensors are torch device tensors (torch provides memory and the
stream).  The library is loaded on first use; a missing library raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsgdn.so")

SGDN_F32, SGDN_BF16, SGDN_F16 = 0, 1, 2
SOLVES = {"exact": 0, "blockadj": 1}
EXPORTS = ("sgdn_workspace_bytes", "sgdn_event_capacity", "sgdn_prefill_dense", "sgdn_select",
           "sgdn_prefill_sparse", "sgdn_decode_step", "sgdn_status_string", "sgdn_fp64_selftest",
           "sgdn_select_noalloc")
NOALLOC_SCRATCH_BYTES = 4 << 20   # SGDN_NOALLOC_SCRATCH_BYTES


class Problem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("batch", "seqlen", "n_qk", "n_v", "d_k", "d_v", "dtype", "solve", "o_dtype")] + \
               [("cu_seqlens", ctypes.c_void_p)]


class SparseParams(ctypes.Structure):
    _fields_ = [("keep_budget", ctypes.c_float), ("tier_rate", ctypes.c_float * 3),
                ("tail", ctypes.c_int32),
                ("r_window", ctypes.c_int32), ("norm_weight", ctypes.c_void_p),
                ("fixed_tiers", ctypes.c_int32), ("unit_visibility", ctypes.c_int32),
                ("rank_key", ctypes.c_void_p), ("ablate", ctypes.c_int32),
                ("aux_stream", ctypes.c_void_p), ("aux_events", ctypes.c_void_p * 2)]


ABLATE = {"deferred_w": 1, "compact_states": 2, "csr": 4, "mapped_o": 8,
          "tier_schedule": 16}   # SGDN_ABLATE_* bits


class Stats(ctypes.Structure):
    _fields_ = [("E", ctypes.c_int32), ("E_max", ctypes.c_int32),
                ("n_tier", ctypes.c_int32 * 3), ("k", ctypes.c_int32 * 3),
                ("n_snapshots", ctypes.c_int32), ("nonfinite_input", ctypes.c_int32),
                ("nonfinite_output", ctypes.c_int32)]


# bits of Stats.nonfinite_input / nonfinite_output (SGDN_NF_*)
NF_INPUT = {"q": 1, "k": 2, "v": 4, "a": 8, "beta": 16, "z": 32, "s0": 64}
NF_OUTPUT = {"o": 1, "s_final": 2}
STAT_FIELDS = ("E", "E_max", "n_low", "n_medium", "n_high", "k_low", "k_medium", "k_high",
               "n_snapshots", "nonfinite_input", "nonfinite_output")


class Debug(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("g", "gamma", "prefix", "score", "eta", "U", "mask", "tier")] + \
               [("events", ctypes.POINTER(ctypes.c_void_p)), ("n_events", ctypes.c_int32)]


EV_NAMES = ("start", "intra", "prefix", "gate", "select", "deferred_w", "hscan", "o")


STATS_INTS = ctypes.sizeof(Stats) // 4

_lib = None


class SgdnError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_string(status)} ({status})")
        self.status = status


def lib():
    """Load libsgdn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m gated_deltanet_prefill_chunkwise_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        P = ctypes.POINTER(Problem)
        SP = ctypes.POINTER(SparseParams)
        L.sgdn_workspace_bytes.argtypes = [P, i32, SP]
        L.sgdn_workspace_bytes.restype = sz
        L.sgdn_event_capacity.argtypes = [P, SP, ctypes.POINTER(ctypes.c_int32),
                                          ctypes.POINTER(ctypes.c_int32)]
        L.sgdn_event_capacity.restype = i32
        L.sgdn_fp64_selftest.argtypes = [vp, vp, vp, vp, ctypes.c_int64, vp]
        L.sgdn_fp64_selftest.restype = i32
        L.sgdn_prefill_dense.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp]
        L.sgdn_prefill_dense.restype = i32
        L.sgdn_select.argtypes = [P, vp, vp, vp, SP, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.sgdn_select.restype = i32
        L.sgdn_select_noalloc.argtypes = [P, vp, vp, vp, SP, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.sgdn_select_noalloc.restype = i32
        L.sgdn_prefill_sparse.argtypes = [P, vp, vp, vp, vp, vp, vp, SP, vp, vp, vp, vp, vp, vp,
                                          sz, vp, vp]
        L.sgdn_prefill_sparse.restype = i32
        L.sgdn_decode_step.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.sgdn_decode_step.restype = i32
        L.sgdn_status_string.argtypes = [i32]
        L.sgdn_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().sgdn_status_string(int(status)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _code(dtype):
    """sgdn_dtype of an input tensor dtype (fp32 or bf16)."""
    import torch
    codes = {torch.float32: SGDN_F32, torch.bfloat16: SGDN_BF16}
    if dtype not in codes:
        raise ValueError(f"inputs must be float32 or bfloat16, got {dtype}")
    return codes[dtype]


def _ocode(dtype):
    """sgdn_dtype of the output o (fp32, bf16 or fp16)."""
    import torch
    codes = {torch.float32: SGDN_F32, torch.bfloat16: SGDN_BF16, torch.float16: SGDN_F16}
    if dtype not in codes:
        raise ValueError(f"o must be float32, bfloat16 or float16, got {dtype}")
    return codes[dtype]


def batch_shape(q, cu_seqlens=None, max_seqlen=None):
    """(B, T) of a call.  Packed sequences (``cu_seqlens`` int32 [B + 1] on the
    device, q [1, N_tok, Nq, d]): B = len(cu_seqlens) - 1 and T = the longest
    sequence (read back from the device unless ``max_seqlen`` is given)."""
    if cu_seqlens is None:
        return q.shape[0], q.shape[1]
    import torch
    _check(cu_seqlens, "cu_seqlens", torch.int32)
    if q.shape[0] != 1:
        raise ValueError("packed sequences take q, k, v, a, beta, z of batch 1 [1, N_tok, ...]")
    B = cu_seqlens.numel() - 1
    if B < 1:
        raise ValueError("cu_seqlens needs at least two offsets")
    if max_seqlen is None:
        max_seqlen = int((cu_seqlens[1:] - cu_seqlens[:-1]).max().item())
    return B, max(int(max_seqlen), 1)


def problem(q, v, solve="exact", out_dtype=None, cu_seqlens=None, max_seqlen=None) -> Problem:
    B, T = batch_shape(q, cu_seqlens, max_seqlen)
    Nq, d = q.shape[2], q.shape[3]
    Nv, dv = v.shape[2], v.shape[3]
    od = _ocode(out_dtype) if out_dtype is not None else SGDN_F32
    return Problem(B, T, Nq, Nv, d, dv, _code(q.dtype), SOLVES[solve], od,
                   None if cu_seqlens is None else cu_seqlens.data_ptr())


def sparse_params(keep_budget=0.29, norm_weight=None, tail=16, r_window=16, fixed_tiers=False,
                  unit_visibility=False, rank_key=None, ablate=(), aux=None,
                  tier_rate=None) -> SparseParams:
    """Selector parameters; ``rank_key`` (device fp32 [B, Nv/2, C]) and the
    flags are the selector ablations, ``ablate`` names kernel-pipeline
    ablations (keys of ABLATE), ``tier_rate`` a (rho_L, rho_M, rho_H)
    override of the budget's tier rates, all described in include/sgdn.h.
    ``aux`` is an (aux stream, fork event, join event) triple of torch
    objects, or None for the one-stream schedule."""
    bits = 0
    for name in ablate:
        bits |= ABLATE[name]
    rates = (ctypes.c_float * 3)(*((0.0, 0.0, 0.0) if tier_rate is None else tier_rate))
    p = SparseParams(float(keep_budget), rates, tail, r_window,
                     None if norm_weight is None else norm_weight.data_ptr(),
                     int(bool(fixed_tiers)), int(bool(unit_visibility)),
                     None if rank_key is None else rank_key.data_ptr(), bits)
    if aux is not None:
        stream, ev0, ev1 = aux
        p.aux_stream = stream.cuda_stream
        p.aux_events[0] = ev0.cuda_event
        p.aux_events[1] = ev1.cuda_event
    return p


_aux = {}


def aux_stream(device=None):
    """The binding's second stream and fork / join events for ``device``
    (created once per device and kept; the library itself holds none).  The
    stream has the default priority; the events are recorded once so that
    their handles exist."""
    import torch
    idx = None if device is None else torch.device(device).index
    dev = torch.device("cuda", torch.cuda.current_device() if idx is None else idx)
    if dev not in _aux:
        with torch.cuda.device(dev):
            st = torch.cuda.Stream(device=dev)
            evs = (torch.cuda.Event(enable_timing=False), torch.cuda.Event(enable_timing=False))
            for e in evs:
                e.record(st)
            st.synchronize()
        _aux[dev] = (st, *evs)
    return _aux[dev]


def event_capacity(prob: Problem, params: SparseParams):
    """((k_L, k_M, k_H), E_max per sequence) as the library sizes them."""
    k = (ctypes.c_int32 * 3)()
    e = ctypes.c_int32()
    st = lib().sgdn_event_capacity(ctypes.byref(prob), ctypes.byref(params), k, ctypes.byref(e))
    if st != 0:
        raise SgdnError(st, "sgdn_event_capacity")
    return tuple(k), int(e.value)


def fp64_selftest(x, y, stream=None):
    """Run the selector's compiled binary64 division and square root on device
    fp64 tensors; returns (x / y, sqrt(x)) as device tensors."""
    import torch
    _check(x, "x", torch.float64)
    _check(y, "y", torch.float64)
    if x.shape != y.shape:
        raise ValueError("x and y must have the same shape")
    q = torch.empty_like(x)
    r = torch.empty_like(x)
    st = lib().sgdn_fp64_selftest(_ptr(x), _ptr(y), _ptr(q), _ptr(r), x.numel(), _stream(stream))
    if st != 0:
        raise SgdnError(st, "sgdn_fp64_selftest")
    return q, r


def workspace_bytes(prob: Problem, sparse: bool, params: SparseParams | None = None) -> int:
    return int(lib().sgdn_workspace_bytes(ctypes.byref(prob), int(sparse),
                                          None if params is None else ctypes.byref(params)))


def _check(t, name, dtype=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _stats_check(stats, B):
    import torch
    _check(stats, "stats", torch.int32)
    if stats is not None and tuple(stats.shape) != (B, STATS_INTS):
        raise ValueError(f"stats must be int32 [{B}, {STATS_INTS}]")


def _workspace(nbytes, device, workspace):
    import torch
    if workspace is not None and workspace.numel() * workspace.element_size() >= nbytes:
        return workspace
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def debug_struct(events=None, **bufs) -> Debug:
    """Debug outputs (torch tensors by field name) and optional hipEvent_t handles."""
    d = Debug(*[None if bufs.get(n) is None else bufs[n].data_ptr() for n, _ in Debug._fields_[:8]])
    if events is not None:
        arr = (ctypes.c_void_p * len(events))(*events)
        d.events = ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))
        d.n_events = len(events)
        d._keep = arr
    return d


def prefill_dense(q, k, v, a, beta, s0=None, solve="exact", want_state=True, o=None,
                  s_final=None, workspace=None, debug=None, stream=None, out_dtype=None,
                  cu_seqlens=None, max_seqlen=None, stats=None):
    """Dense GDN-core prefill; returns (o, s_final).

    o is fp32 unless ``out_dtype`` (or a given ``o``) says otherwise.  With
    ``cu_seqlens`` the inputs hold packed sequences (see ``batch_shape``).
    ``stats`` (int32 [B, STATS_INTS] on the device) receives the per-sequence
    statistics, including the non-finite flags.
    """
    import torch
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (beta, "beta")):
        _check(t, n, q.dtype)
    _check(a, "a", torch.float32)
    _check(s0, "s0", torch.float32)
    if o is not None:
        out_dtype = o.dtype
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    _check(o, "o", out_dtype)
    prob = problem(q, v, solve, out_dtype, cu_seqlens, max_seqlen)
    B, Nv, dv = prob.batch, v.shape[2], v.shape[3]
    if o is None:
        o = torch.empty(v.shape, dtype=out_dtype, device=v.device)
    if want_state and s_final is None:
        s_final = torch.empty((B, Nv, q.shape[3], dv), dtype=torch.float32, device=q.device)
    _stats_check(stats, B)
    nbytes = workspace_bytes(prob, False)
    if nbytes == 0:
        raise SgdnError(-2, "sgdn_workspace_bytes")
    ws = _workspace(nbytes, q.device, workspace)
    dbg = None if debug is None else ctypes.byref(debug)
    st = lib().sgdn_prefill_dense(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(a),
                                  _ptr(beta), _ptr(s0), _ptr(o), _ptr(s_final), _ptr(stats),
                                  _ptr(ws), ws.numel(), _stream(stream), dbg)
    if st != 0:
        raise SgdnError(st, "sgdn_prefill_dense")
    return o, s_final


def decode_step(q, k, v, a, beta, state, s_out=None, o=None, out_dtype=None, stream=None):
    """One-token decode step from ``state`` [B, Nv, d, dv] fp32; returns (o, s_out).

    q, k [B, Nq, d], v [B, Nv, dv], a [B, Nv] fp32, beta [B, Nv].  ``s_out``
    may be ``state`` itself (updated in place); by default a new tensor.
    """
    import torch
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (beta, "beta")):
        _check(t, n, q.dtype)
    _check(a, "a", torch.float32)
    _check(state, "state", torch.float32)
    if o is not None:
        out_dtype = o.dtype
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    _check(o, "o", out_dtype)
    B, Nq, d = q.shape
    Nv, dv = v.shape[1], v.shape[2]
    if o is None:
        o = torch.empty(v.shape, dtype=out_dtype, device=v.device)
    if s_out is None:
        s_out = torch.empty_like(state)
    _check(s_out, "s_out", torch.float32)
    for t, shape, n in ((k, (B, Nq, d), "k"), (a, (B, Nv), "a"), (beta, (B, Nv), "beta"),
                        (state, (B, Nv, d, dv), "state"), (s_out, (B, Nv, d, dv), "s_out"),
                        (o, (B, Nv, dv), "o")):
        if tuple(t.shape) != shape:
            raise ValueError(f"{n} must have shape {shape}, got {tuple(t.shape)}")
    prob = Problem(B, 1, Nq, Nv, d, dv, _code(q.dtype), 0, _ocode(out_dtype))
    st = lib().sgdn_decode_step(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(a),
                                _ptr(beta), _ptr(state), _ptr(s_out), _ptr(o), _stream(stream))
    if st != 0:
        raise SgdnError(st, "sgdn_decode_step")
    return o, s_out


def select(score, gamma, eta, keep_budget=0.29, workspace=None, stream=None, cu_seqlens=None,
           fixed_tiers=False, unit_visibility=False, rank_key=None, noalloc=False, out=None,
           tier_rate=None):
    """Selector + CSR layout on fp32 statistics; returns a dict of device tensors.

    With ``cu_seqlens`` (int32 [B + 1] token offsets) sequence b has only its
    ceil(len_b / 64) valid chunks; the arrays keep the stride C.  ``noalloc``
    calls sgdn_select_noalloc (the library's static scratch, no workspace);
    ``out`` reuses a dict of output tensors from an earlier call.
    """
    import torch
    B, Nv, C = score.shape
    for t, n in ((score, "score"), (gamma, "gamma"), (eta, "eta")):
        _check(t, n, torch.float32)
    _check(cu_seqlens, "cu_seqlens", torch.int32)
    _check(rank_key, "rank_key", torch.float32)
    if rank_key is not None and tuple(rank_key.shape) != (B, Nv // 2, C):
        raise ValueError("rank_key must be [B, Nv/2, C]")
    if cu_seqlens is not None and cu_seqlens.numel() != B + 1:
        raise ValueError("cu_seqlens must hold B + 1 offsets")
    T = C * 64
    prob = Problem(B, T, Nv // 2, Nv, 128, 128, SGDN_BF16, 1, SGDN_F32,
                   None if cu_seqlens is None else cu_seqlens.data_ptr())
    params = sparse_params(keep_budget, fixed_tiers=fixed_tiers, unit_visibility=unit_visibility,
                           rank_key=rank_key, tier_rate=tier_rate)
    NP, G = Nv // 2, (C + 1) // 2
    dev = score.device
    _, e_max = event_capacity(prob, params)
    shapes = dict(mask=((B, NP, C), torch.uint8), tier=((B, NP), torch.uint8),
                  row_pair=((B, NP), torch.int32), row_ptr=((B, NP + 1), torch.int32),
                  col=((B, e_max), torch.int32), pred=((B, NP, G), torch.int32),
                  group_slot=((B, NP, G), torch.int32), stats=((B, STATS_INTS), torch.int32))
    if out is not None:
        for name, (shape, dt) in shapes.items():
            _check(out[name], name, dt)
            if tuple(out[name].shape) != shape:
                raise ValueError(f"{name} must have shape {shape}, got {tuple(out[name].shape)}")
    else:
        out = {name: torch.empty(shape, dtype=dt, device=dev) for name, (shape, dt) in shapes.items()}
        out["col"].fill_(-1)
    return _select_call(prob, params, score, gamma, eta, out, workspace, noalloc, stream)


def _select_call(prob, params, score, gamma, eta, out, workspace, noalloc, stream):
    args = (_ptr(out["mask"]), _ptr(out["tier"]), _ptr(out["row_pair"]), _ptr(out["row_ptr"]),
            _ptr(out["col"]), _ptr(out["pred"]), _ptr(out["group_slot"]), _ptr(out["stats"]))
    if noalloc:
        st = lib().sgdn_select_noalloc(ctypes.byref(prob), _ptr(score), _ptr(gamma), _ptr(eta),
                                       ctypes.byref(params), *args, _stream(stream))
        if st != 0:
            raise SgdnError(st, "sgdn_select_noalloc")
        return out
    nbytes = workspace_bytes(prob, True, params)
    if nbytes == 0:
        raise SgdnError(-2, "sgdn_workspace_bytes")
    ws = _workspace(nbytes, score.device, workspace)
    st = lib().sgdn_select(ctypes.byref(prob), _ptr(score), _ptr(gamma), _ptr(eta),
                           ctypes.byref(params), *args, _ptr(ws), ws.numel(), _stream(stream))
    if st != 0:
        raise SgdnError(st, "sgdn_select")
    return out


def prefill_sparse(q, k, v, a, beta, z=None, keep_budget=0.29, solve="blockadj",
                   mask_override=None, s0=None, norm_weight=None, want_state=True, o=None,
                   s_final=None, stats=None, workspace=None, debug=None, stream=None,
                   out_dtype=None, cu_seqlens=None, max_seqlen=None, tail=16, fixed_tiers=False,
                   unit_visibility=False, rank_key=None, ablate=(), aux=True, tier_rate=None):
    """SparseGDN prefill; returns (o, s_final, stats[B, STATS_INTS] int32).

    o is fp32 unless ``out_dtype`` (or a given ``o``) says otherwise.  With
    ``cu_seqlens`` the inputs hold packed sequences (see ``batch_shape``).
    ``aux``: True uses the binding's second stream (``aux_stream``) for the
    H scan and O of the shorter chains (where the library forks: sequences
    longer than 64 chunks, see include/sgdn.h), False runs every kernel on
    ``stream``, or a (stream, event, event) triple of the caller's.
    """
    import torch
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (beta, "beta"), (z, "z")):
        _check(t, n, q.dtype)
    _check(a, "a", torch.float32)
    _check(s0, "s0", torch.float32)
    _check(mask_override, "mask_override", torch.uint8)
    _check(norm_weight, "norm_weight", torch.float32)
    if o is not None:
        out_dtype = o.dtype
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    _check(o, "o", out_dtype)
    prob = problem(q, v, solve, out_dtype, cu_seqlens, max_seqlen)
    _check(rank_key, "rank_key", torch.float32)
    if rank_key is not None and tuple(rank_key.shape) != (prob.batch, v.shape[2] // 2,
                                                         -(-prob.seqlen // 64)):
        raise ValueError("rank_key must be [B, Nv/2, C]")
    if aux is True:
        aux = aux_stream(q.device)
    elif aux is False:
        aux = None
    params = sparse_params(keep_budget, norm_weight, tail=tail, fixed_tiers=fixed_tiers,
                           unit_visibility=unit_visibility, rank_key=rank_key, ablate=ablate,
                           aux=aux, tier_rate=tier_rate)
    B, Nv, dv = prob.batch, v.shape[2], v.shape[3]
    if o is None:
        o = torch.empty(v.shape, dtype=out_dtype, device=v.device)
    if want_state and s_final is None:
        s_final = torch.empty((B, Nv, q.shape[3], dv), dtype=torch.float32, device=q.device)
    if stats is None:
        stats = torch.zeros((B, STATS_INTS), dtype=torch.int32, device=q.device)
    _stats_check(stats, B)
    nbytes = workspace_bytes(prob, True, params)
    if nbytes == 0:
        raise SgdnError(-2, "sgdn_workspace_bytes")
    ws = _workspace(nbytes, q.device, workspace)
    dbg = None if debug is None else ctypes.byref(debug)
    st = lib().sgdn_prefill_sparse(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(a),
                                   _ptr(beta), _ptr(z), ctypes.byref(params), _ptr(mask_override),
                                   _ptr(s0), _ptr(o), _ptr(s_final), _ptr(stats), _ptr(ws),
                                   ws.numel(), _stream(stream), dbg)
    if st != 0:
        raise SgdnError(st, "sgdn_prefill_sparse")
    return o, s_final, stats

