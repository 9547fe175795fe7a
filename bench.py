"""GDN-core prefill benchmark on one MI355X.

Workload: 24 independently seeded GDN layers run back to back, bf16 inputs,
batch 1, T = 131072, Nq = 16, Nv = 32, d = dv = 128 (value heads 2p, 2p+1
share query/key head p), per-value-head output gate z, synthetic inputs drawn
on the device.  One step = one pass of the 24-layer stack through the whole
SparseGDN path at the default keep budget (29% of head-pair x chunk events):
intra (block-adjacent solve, tail score), gate energy, selector and CSR
layout, deferred W, event-sparse H scan with compact snapshots, grouped O.
The dense exact path (intra, H, O) is timed the same way beside it, and so is
the single-token decode step that continues from the final states (a batch
of 128 sequences through the same 24 layers, states updated in place).  A
packed variable-length leg reads the same tokens as 16 sequences of mixed
lengths (cu_seqlens) and times both paths again.  A selector-ablation leg
times the sparse step with each switch of Sec. 3.5 (fixed 3/4/9 tiers,
G_h = 1, random keys at matched budget, Tail-8/32/64 windows), and a
kernel-pipeline ablation leg times it with deferred W, compact states, the
CSR event walk and the two-chunk O mapping undone (Table 6), reporting each
mechanism's speedup over its stages.

Beside the 131072-token stack, the same layers' first 4K ... 64K tokens are
timed in both modes (the length sweep of Sec. 3.2, Table 1; 32K is the other
length the metric names), and the keep-budget x batch grid of Sec. 3.3-3.4
(batch 2 / 4 / 8 of 32768 tokens, keep 0.15 / 0.29 / 0.5 / 1.0, per-head
decay scale u ~ U(0, ln 16)) is timed against the dense path at each batch.

Every timed prefill writes an fp16 O (fp32 a and s_final); an output leg
repeats both modes with an fp32 and a bf16 O.

Prints one JSON line.  value = tokens/s of the 24-layer stack (B*T per step);
each timed configuration reports the mean and the median over its steps.
The headline modes and the length sweep are also timed as replays of the
step captured once as a HIP graph (graph_*), which removes the host's
per-launch cost (it matters at the short lengths, where a layer's kernels
are short).
roofline = the dominant kernel's algorithmic bytes per layer over its mean
time per layer (HIP events recorded by the library on the caller's stream;
in the sparse path the H scan of CSR rows 4-15 runs on a second stream
during the launch for rows 0-3, which the events bracket, so the bytes of
both count over that time; traffic likewise sums both launches).
path_roofline = the whole layer against HBM with the algorithmic bytes of
the I/O streams (bf16 Q, K, V; fp16 O; fp32 a; bf16 beta) plus the compact
snapshots written and read; mfma = the algorithmic flops of the method over
the same time against the dense bf16 matrix-core peak.
snapshot_bytes = the group-entry snapshot memory of one layer: allocated (a
slot for every group boundary of every head) and used (the compact
snapshots the H scan wrote; all of them in the dense path).
cpu_baseline = the fp64 numpy oracle as it stands, one worker process per
host core (up to 16), each on a different layer's first tokens, in both
modes, in the same unit.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 / fp16 matrix cores, published
B, T, NQ, NV, D = 1, 131072, 16, 32, 128
O_DTYPE = "fp16"               # output o of every timed prefill (fp32 and bf16 O: output_leg)
LAYERS = 24
STAGES = ("intra", "prefix", "gate", "select", "deferred_w", "hscan", "o")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--layers", type=int, default=LAYERS)
    ap.add_argument("--seqlen", type=int, default=T)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--mode", choices=("both", "sparse", "dense"), default="both")
    ap.add_argument("--cpu-tokens", type=int, default=2048,
                    help="tokens of one layer each oracle worker processes")
    ap.add_argument("--cpu-workers", type=int, default=16,
                    help="oracle worker processes (at most the host's usable cores)")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the 4K-64K length sweep")
    ap.add_argument("--no-grid", action="store_true",
                    help="skip the keep-budget x batch grid")
    ap.add_argument("--no-varlen", action="store_true",
                    help="skip the packed variable-length leg")
    ap.add_argument("--no-ablations", action="store_true",
                    help="skip the kernel-pipeline ablation leg")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the graph-replay timings (one call per layer and step)")
    ap.add_argument("--no-output-types", action="store_true",
                    help="skip the leg that reruns both modes with an fp32 and a bf16 O")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the selector-ablation leg")
    ap.add_argument("--decode-batch", type=int, default=128,
                    help="sequences of the decode-step leg (0 skips it)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration)")
    return ap.parse_args()


class Hip:
    """Minimal HIP event API through the runtime torch already loaded."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        assert self.lib.hipEventCreateWithFlags(ctypes.byref(e), 0) == 0
        return e.value

    def elapsed_ms(self, a, b):
        f = ctypes.c_float()
        assert self.lib.hipEventElapsedTime(ctypes.byref(f), ctypes.c_void_p(a), ctypes.c_void_p(b)) == 0
        return f.value


def algorithmic_bytes_per_token(stage: str, mode: str, sigma: float, keep: float) -> float:
    """Bytes per token of the I/O streams a stage must move: bf16 Q, K, V, a
    (fp32) and beta, a 2-byte O (the output stream of the problem statement;
    this run writes it as fp16), and the fp16 group snapshots (one 128x128 state
    per head per two chunks, written by the H scan and read by O); pipeline
    intermediates (U, U', W or Cb, K^T tiles) are not counted."""
    k_in = NQ * D * 2           # K (shared by a head pair)
    q_in = NQ * D * 2
    v_in = NV * D * 2
    o_out = NV * D * 2          # O at 2 bytes (fp16 here)
    a_b = NV * 4 + NV * 2       # a (fp32) + beta (bf16)
    snap = NV * D * D * 2 / 128 * (sigma if mode == "sparse" else 1.0)   # one direction
    if stage == "intra":
        return k_in + v_in + a_b
    if stage == "hscan":
        return k_in * (keep if mode == "sparse" else 1.0) + snap
    if stage == "o":
        return q_in + k_in + o_out + snap
    if stage == "path":
        return q_in + k_in + v_in + a_b + o_out + 2 * snap
    return 0.0


def path_bytes_per_token(mode: str, sigma: float, o_bytes: int = 2) -> float:
    """Algorithmic HBM bytes per token of one layer: the I/O streams (bf16 Q,
    K, V, a 2-byte O by default, fp32 a, bf16 beta) plus the fp16 group snapshots,
    one 128x128 state per head per two chunks written once and read once
    (the fraction sigma of them in the sparse path)."""
    io = NQ * D * 2 * 2 + NV * D * 2 + NV * D * o_bytes + NV * 4 + NV * 2
    snap = 2 * NV * D * D * 2 / 128 * (sigma if mode == "sparse" else 1.0)
    return io + snap


def flops_per_token(mode: str, keep: float) -> float:
    """Algorithmic flops per token of one layer (multiply-adds x 2): per chunk
    and value head the Gram and Q K^T products of a pair counted once per
    pair, the causal triangle only, the 7 blocks of the block-adjacent solve,
    and in the sparse path W, W S and K^T U' on the kept events only:
      dense exact: Gram 129,024 + inverse 43,680 + U 266,240 + W 266,240
                   + W S, K^T U', Q S 3 x 1,048,576 + Q K^T 133,120
                   + A U' 266,240 = 4,250,272 MAC;
      sparse:      Gram 79,872 + inverse 15,776 + U 167,936 + Q S 1,048,576
                   + Q K^T 264,192 + A U' 528,384 = 2,104,736 MAC, plus
                   (W 167,936 + W S + K^T U' 2 x 1,048,576) x keep."""
    mac = 4250272.0 if mode == "dense" else 2104736.0 + 2265088.0 * keep
    return mac * 2 * NV / 64


def code_text(path: str) -> str:
    """A HIP source with its comments removed and its whitespace collapsed:
    what the compiler sees of it, so that editing a comment keeps the
    counters taken on the code valid."""
    import re
    src = open(path, encoding="utf-8").read()
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def source_hash(stage: str) -> str:
    f = {"hscan": "hscan.hip", "o": "ochunk.hip", "intra": "intra.hip",
         "decode": "decode.hip"}.get(stage)
    if f is None:
        return ""
    p = os.path.join(ROOT, "gated_deltanet_prefill_chunkwise_amd", "csrc", f)
    return hashlib.sha256(code_text(p).encode()).hexdigest()[:16]


def measured_traffic(stage: str, mode: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
        e = d[f"{mode}:{stage}"]
        if e.get("source_sha256_16") != source_hash(stage):
            return None
        return float(e["bytes_per_launch"])
    except Exception:
        return None


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_worker(path: str, mode: str) -> float:
    """One oracle run (a worker process, one BLAS thread) on a saved layer
    sample; returns its wall time."""
    import numpy as np
    from oracle import gdn, sparse
    x = np.load(path)
    f = {k: x[k].astype(np.float64) for k in x.files}
    t0 = time.perf_counter()
    if mode == "dense":
        gdn.chunk_prefill(f["q"], f["k"], f["v"], f["a"], f["beta"], None, "exact")
    else:
        sparse.sparse_prefill(f["q"], f["k"], f["v"], f["a"], f["beta"], z=f["z"],
                              keep_budget=0.29, solve="blockadj")
    return time.perf_counter() - t0


def _worker_init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass
    # one tiny run of each path, so that lazy imports and first-call costs
    # stay outside the timed region
    import numpy as np
    from oracle import gdn, sparse
    g = np.random.default_rng(0)
    x = {k: g.standard_normal(s) for k, s in (("q", (1, 128, 16, 128)), ("k", (1, 128, 16, 128)),
                                                ("v", (1, 128, 32, 128)), ("z", (1, 128, 32, 128)))}
    a, beta = -np.ones((1, 128, 32)), np.full((1, 128, 32), 0.5)
    gdn.chunk_prefill(x["q"], x["k"], x["v"], a, beta, None, "exact")
    sparse.sparse_prefill(x["q"], x["k"], x["v"], a, beta, z=x["z"])


def _noop(i):
    time.sleep(0.05)
    return i


def cpu_baseline(layers, tokens, workers):
    """The fp64 oracle as it stands, on the host's cores: one worker process
    per core (at most `workers`, at most the cores this process may use), each
    running the whole oracle on the first `tokens` tokens of a different
    layer, all 32 value heads; dense (exact) and sparse (29%, block-adjacent,
    selector included).  Throughput = all workers' tokens over the wall time
    of the pool, in the headline's unit (per 24-layer stack)."""
    import multiprocessing as mp
    import tempfile
    from concurrent.futures import ProcessPoolExecutor
    import numpy as np
    usable = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    n = max(1, min(workers, usable or 1, len(layers)))
    # samples go through memory-backed files (removed below)
    tmp = tempfile.mkdtemp(prefix="sgdn_cpu_", dir="/dev/shm" if os.path.isdir("/dev/shm") else None)
    paths = []
    t0 = time.perf_counter()
    for l in range(n):
        inp = layers[l][0]
        arrs = {k: v[:, :tokens].float().cpu().numpy() for k, v in inp.items()}
        pth = os.path.join(tmp, f"layer{l}.npz")
        np.savez(pth, **arrs)
        paths.append(pth)
    print(f"[bench] cpu baseline: {n} samples of {tokens} tokens staged in "
          f"{time.perf_counter() - t0:.1f} s; {n} workers", file=sys.stderr, flush=True)
    out = {}
    try:
        with ProcessPoolExecutor(max_workers=n, mp_context=mp.get_context("spawn"),
                                 initializer=_worker_init) as ex:
            list(ex.map(_noop, range(4 * n)))      # every worker started and initialised
            for mode in ("dense", "sparse"):
                t0 = time.perf_counter()
                per = list(ex.map(_oracle_worker, paths, [mode] * n))
                wall = time.perf_counter() - t0
                tok_s_layer = n * tokens / wall
                print(f"[bench] cpu baseline {mode}: {wall:.1f} s for {n} x {tokens} tokens",
                      file=sys.stderr, flush=True)
                out[mode] = dict(value=round(tok_s_layer / LAYERS, 2),
                                 per_layer_tok_s=round(tok_s_layer, 1), wall_s=round(wall, 2),
                                 worker_s=[round(t, 2) for t in per])
    finally:
        for pth in paths:
            os.remove(pth)
        os.rmdir(tmp)
    return dict(value=out["sparse"]["value"], unit="tok/s (24-layer GDN-core stack)", cores=n,
                kind="oracle", host_cpus=os.cpu_count(), usable_cpus=usable, cpu_model=_cpu_model(),
                dense=out["dense"], sparse=out["sparse"],
                sample=(f"fp64 numpy oracle as it stands, {n} worker processes (one BLAS thread "
                        f"each) on {n} cores, each on the first {tokens} tokens of a different "
                        f"layer (all 32 value heads): the sparse path (29% budget, block-adjacent "
                        f"solve, selector included; value) and the dense exact path; tokens of all "
                        f"workers over the pool's wall time, divided by 24 for the stack"))


def timed_steps(args, step):
    """args.warmup untimed calls of step(i), then args.steps timed ones, each
    bracketed by events on the current stream; returns (mean ms, median ms)."""
    import statistics
    import torch
    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for i in range(args.steps):
        evs[i][0].record()
        step(i)
        evs[i][1].record()
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in evs]
    return statistics.fmean(ms), statistics.median(ms)


def graph_steps(args, step):
    """The same step captured once as a HIP graph (torch.cuda.CUDAGraph over
    the library's launches on the caller's stream and its second stream),
    then args.steps timed replays after args.warmup untimed ones; returns
    (mean, median) ms per replay."""
    import statistics
    import torch
    cur = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(cur)
    with torch.cuda.stream(side):
        step(None)
    cur.wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(None)
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for i in range(args.steps):
        evs[i][0].record()
        g.replay()
        evs[i][1].record()
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in evs]
    del g
    return statistics.fmean(ms), statistics.median(ms)


def time_stack(args, hip, L, call):
    """Warm-up then args.steps timed passes of call(l, dbg) over L layers;
    returns (ms per step, mean ms per launch of every stage)."""
    import torch
    from gated_deltanet_prefill_chunkwise_amd import ops
    nev = len(STAGES) + 1
    events = [[[hip.event() for _ in range(nev)] for _ in range(L)] for _ in range(args.steps)]
    dbgs = [[ops.debug_struct(events=events[s][l]) for l in range(L)] for s in range(args.steps)]
    for _ in range(args.warmup):
        for l in range(L):
            call(l, None)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for s_ in range(args.steps):
        for l in range(L):
            call(l, dbgs[s_][l])
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    stage = {name: round(sum(hip.elapsed_ms(events[s_][l][i], events[s_][l][i + 1])
                             for s_ in range(args.steps) for l in range(L)) / (args.steps * L), 4)
             for i, name in enumerate(STAGES)}
    return ms, stage


def ablation_leg(args, layers, hip, prob, dev):
    """The sparse step with kernel-pipeline mechanisms undone (Table 6),
    beside the default.  Each row sets one run against its matched
    reference run: speedup = run / reference time over the row's stages."""
    import torch
    from gated_deltanet_prefill_chunkwise_amd import ops
    runs = {"default": (), "deferred_w": ("deferred_w",), "csr": ("csr",),
            "compact_states": ("compact_states",), "tier_schedule": ("tier_schedule",),
            "compact_states+mapped_o": ("compact_states", "mapped_o"), "mapped_o": ("mapped_o",)}
    # (mechanism, run with it undone, reference run, stages).  CSR-off also
    # forms W of every chunk, so it is set against the packed-W run; mapped-O
    # off is set against the run with the same dense group-entry states, so
    # that only O's reads differ; compact+mapped undoes both.  With one
    # sequence the O stage holds the wait for the second stream's H scan and
    # O, so the H-side rows take the H scan and O stages together.
    full = ("intra", "deferred_w", "hscan", "o")
    rows = [("deferred_w", "deferred_w", "default", full),
            ("csr_event_scan", "csr", "deferred_w", ("hscan", "o")),
            ("compact_states", "compact_states", "default", ("hscan", "o")),
            ("tier_schedule", "tier_schedule", "default", ("hscan", "o")),
            ("mapped_o", "compact_states+mapped_o", "compact_states", ("hscan", "o")),
            ("compact_states+mapped_o", "compact_states+mapped_o", "default", full),
            ("mapped_o_over_compact_snapshots", "mapped_o", "default", ("hscan", "o"))]
    out = {"runs": {}, "rows": []}
    for name, ab in runs.items():
        ws = torch.empty(ops.workspace_bytes(prob, True, ops.sparse_params(ablate=ab)),
                         dtype=torch.uint8, device=dev)

        def call(l, dbg, ab=ab, ws=ws):
            inp, o, sf, st = layers[l]
            ops.prefill_sparse(inp["q"], inp["k"], inp["v"], inp["a"], inp["beta"], z=inp["z"],
                               keep_budget=0.29, solve="blockadj", o=o, s_final=sf, stats=st,
                               workspace=ws, debug=dbg, ablate=ab)
        ms, stage = time_stack(args, hip, len(layers), call)
        del ws
        out["runs"][name] = {"undone": list(ab), "ms_per_step": round(ms, 4),
                             "stage_ms_per_launch": stage}
        print(f"[bench] ablation {name}: {ms:.3f} ms per {args.layers}-layer step; stages "
              + ", ".join(f"{k} {v:.3f}" for k, v in stage.items()), file=sys.stderr, flush=True)
    for mech, run, ref, sc in rows:
        st = out["runs"][run]["stage_ms_per_launch"]
        base = out["runs"][ref]["stage_ms_per_launch"]
        out["rows"].append({"mechanism": mech, "run": run, "reference": ref, "scope": "+".join(sc),
                            "speedup": round(sum(st[k] for k in sc) / sum(base[k] for k in sc), 3)})
    return out


def varlen_lengths(total: int, n: int = 16, seed: int = 7):
    """n ragged lengths, log-uniform between 1/16 and 1x of total/n*4, summing to total."""
    import numpy as np
    g = np.random.default_rng(seed)
    x = np.exp(g.uniform(np.log(total / n / 4), np.log(total / n * 4), n))
    lens = np.maximum(1, np.floor(x / x.sum() * total)).astype(np.int64)
    lens[-1] += total - lens.sum()
    assert lens.min() >= 1 and lens.sum() == total
    return [int(v) for v in lens]


def varlen_leg(args, layers, hip):
    """Both paths over the same 24 layers' tokens read as packed sequences."""
    import torch
    from gated_deltanet_prefill_chunkwise_amd import ops
    Tn = args.seqlen
    lens = varlen_lengths(B * Tn)
    cu = torch.tensor([0] + list(__import__("itertools").accumulate(lens)), dtype=torch.int32,
                      device="cuda")
    Tm = max(lens)
    inp0 = layers[0][0]
    prob = ops.problem(inp0["q"], inp0["v"], "blockadj", torch.float16, cu, Tm)
    wsb = max(ops.workspace_bytes(prob, True, ops.sparse_params()), ops.workspace_bytes(prob, False))
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    nseq = len(lens)
    sf = torch.empty((nseq, NV, D, D), dtype=torch.float32, device="cuda")
    st = torch.zeros((nseq, ops.STATS_INTS), dtype=torch.int32, device="cuda")
    out = {}
    L = len(layers)
    nev = len(STAGES) + 1
    for mode in ("sparse", "dense"):
        events = [[[hip.event() for _ in range(nev)] for _ in range(L)] for _ in range(args.steps)]
        dbgs = [[ops.debug_struct(events=events[s][l]) for l in range(L)] for s in range(args.steps)]

        def step(dbg_row):
            for l, (inp, o, _, _) in enumerate(layers):
                dbg = dbg_row[l] if dbg_row is not None else None
                if mode == "sparse":
                    ops.prefill_sparse(inp["q"], inp["k"], inp["v"], inp["a"], inp["beta"],
                                       z=inp["z"], keep_budget=0.29, solve="blockadj", o=o,
                                       s_final=sf, stats=st, workspace=ws, cu_seqlens=cu,
                                       max_seqlen=Tm, debug=dbg)
                else:
                    ops.prefill_dense(inp["q"], inp["k"], inp["v"], inp["a"], inp["beta"],
                                      solve="exact", o=o, s_final=sf, workspace=ws,
                                      cu_seqlens=cu, max_seqlen=Tm, debug=dbg)
        for _ in range(args.warmup):
            step(None)
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for s_ in range(args.steps):
            step(dbgs[s_])
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / args.steps
        stage = {name: round(sum(hip.elapsed_ms(events[s_][l][i], events[s_][l][i + 1])
                                 for s_ in range(args.steps) for l in range(L)) / (args.steps * L), 4)
                 for i, name in enumerate(STAGES)}
        out[mode] = {"value_tok_s": round(B * Tn / (ms / 1e3), 1), "ms_per_step": round(ms, 4),
                     "stage_ms_per_launch": stage}
        print(f"[bench] varlen {mode}: {ms:.3f} ms per {args.layers}-layer step "
              f"({nseq} packed sequences); stages (ms/launch) "
              + ", ".join(f"{k} {v:.3f}" for k, v in stage.items()), file=sys.stderr, flush=True)
    out["lengths"] = lens
    return out


def variants_leg(args, layers, ws, C):
    """The sparse 24-layer step under each selector ablation; keep from the
    device statistics."""
    import torch
    from gated_deltanet_prefill_chunkwise_amd import ops, synth
    st = [torch.zeros((B, ops.STATS_INTS), dtype=torch.int32, device="cuda") for _ in layers]
    keys = []
    for l in range(len(layers)):
        g = torch.Generator(device="cuda")
        g.manual_seed(synth.seed_for(7, l))
        keys.append(torch.rand((B, NV // 2, C), generator=g, device="cuda"))
    variants = {"fixed_tiers_3_4_9": dict(fixed_tiers=True), "unit_visibility": dict(unit_visibility=True),
                "random_keys": dict(rank_key=True), "tail8": dict(tail=8), "tail32": dict(tail=32),
                "tail64": dict(tail=64)}
    out = {}
    for name, var in variants.items():
        def step():
            for l, (inp, o, sf, _) in enumerate(layers):
                kw = dict(var)
                if kw.pop("rank_key", False):
                    kw["rank_key"] = keys[l]
                ops.prefill_sparse(inp["q"], inp["k"], inp["v"], inp["a"], inp["beta"], z=inp["z"],
                                   keep_budget=0.29, solve="blockadj", o=o, s_final=sf, stats=st[l],
                                   workspace=ws, **kw)
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(args.steps):
            step()
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / args.steps
        keep = float(torch.stack(st).float()[:, 0, 0].mean()) / (16 * C)
        out[name] = {"ms_per_step": round(ms, 4), "value_tok_s": round(B * args.seqlen / (ms / 1e3), 1),
                     "measured_keep": round(keep, 5)}
        print(f"[bench] sparse {name}: {ms:.3f} ms per {args.layers}-layer step, keep {keep:.4f}",
              file=sys.stderr, flush=True)
    return out


def output_leg(args, layers, ws):
    """Both modes with an fp32 O and with a bf16 O beside the headline's fp16
    O.  fp16 carries an 11-bit significand, so its rounding (at most 2^-11
    of an element) stays well inside the parity bar; a bf16 O (the pages'
    model dtype) rounds to 2^-8 of an element, which alone exceeds the bar
    on the largest outputs; fp32 shows what the wider output stream costs."""
    import torch
    from gated_deltanet_prefill_chunkwise_amd import ops
    res = {}
    for name, dt in (("fp32", torch.float32), ("bf16", torch.bfloat16)):
        outs = [torch.empty(inp["v"].shape, dtype=dt, device="cuda") for (inp, _, _, _) in layers]
        row = {}
        for mode in ("sparse", "dense"):
            def step(_i, mode=mode):
                for l, (inp, _, sf, st) in enumerate(layers):
                    if mode == "sparse":
                        ops.prefill_sparse(inp["q"], inp["k"], inp["v"], inp["a"], inp["beta"],
                                           z=inp["z"], keep_budget=0.29, solve="blockadj",
                                           o=outs[l], s_final=sf, stats=st, workspace=ws)
                    else:
                        ops.prefill_dense(inp["q"], inp["k"], inp["v"], inp["a"], inp["beta"],
                                          solve="exact", o=outs[l], s_final=sf, workspace=ws)
            mean, med = timed_steps(args, step)
            row[mode] = {"ms_per_step": round(mean, 4), "median_ms_per_step": round(med, 4),
                         "value_tok_s": round(B * args.seqlen / (mean / 1e3), 1)}
            print(f"[bench] {mode}, {name} O: {mean:.3f} ms per {args.layers}-layer step",
                  file=sys.stderr, flush=True)
        del outs
        row["sparse_speedup_over_dense"] = round(row["dense"]["ms_per_step"] / row["sparse"]["ms_per_step"], 3)
        res[f"{name}_o"] = row
    return res


def sweep_leg(args, layers, ws):
    """Both modes over the first T tokens of the same 24 layers, T = 4K ...
    64K (the 131072-token point is the headline): Sec. 3.2, Table 1 times
    this sweep (4K, 8K, 16K, 32K, 64K, 128K); 32K is named by the metric."""
    from gated_deltanet_prefill_chunkwise_amd import ops
    out = {}
    for Tn in (4096, 8192, 16384, 32768, 65536):
        if Tn > args.seqlen:
            continue
        row = {}
        for mode in ("sparse", "dense"):
            def step(_i, mode=mode, Tn=Tn):
                for inp, o, sf, st in layers:
                    x = {k: v[:, :Tn] for k, v in inp.items()}
                    if mode == "sparse":
                        ops.prefill_sparse(x["q"], x["k"], x["v"], x["a"], x["beta"], z=x["z"],
                                           keep_budget=0.29, solve="blockadj", o=o[:, :Tn],
                                           s_final=sf, stats=st, workspace=ws)
                    else:
                        ops.prefill_dense(x["q"], x["k"], x["v"], x["a"], x["beta"], solve="exact",
                                          o=o[:, :Tn], s_final=sf, workspace=ws)
            mean, med = timed_steps(args, step)
            row[mode] = {"ms_per_step": round(mean, 4), "median_ms_per_step": round(med, 4),
                         "value_tok_s": round(B * Tn / (mean / 1e3), 1),
                         "per_layer_tok_s": round(B * Tn * len(layers) / (mean / 1e3), 1)}
            if not args.no_graph:
                gmean, gmed = graph_steps(args, step)
                row[mode].update({"graph_ms_per_step": round(gmean, 4),
                                  "graph_median_ms_per_step": round(gmed, 4),
                                  "graph_value_tok_s": round(B * Tn / (gmean / 1e3), 1)})
            if mode == "sparse":
                import torch
                stt = torch.stack([st for (_, _, _, st) in layers]).float().cpu()[:, 0, :]
                C = Tn // 64
                keep = float((stt[:, 0] / (16 * C)).mean())
                sigma = float((stt[:, 8] / (16 * max((C + 1) // 2 - 1, 1))).mean())
                row[mode]["measured_keep"] = round(keep, 5)
                row[mode]["snapshot_fraction"] = round(sigma, 5)
            else:
                sigma, keep = 1.0, 1.0
            per_layer_ms = mean / len(layers)
            alg = path_bytes_per_token(mode, sigma) * B * Tn
            row[mode]["path_roofline_frac"] = round(alg / (per_layer_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4)
            fl = flops_per_token(mode, keep) * B * Tn
            row[mode]["mfma_frac"] = round(fl / (per_layer_ms / 1e3) / 1e12 / MFMA_PEAK_TFLOPS, 4)
        row["sparse_speedup_over_dense"] = round(row["dense"]["ms_per_step"] / row["sparse"]["ms_per_step"], 3)
        gtxt = ""
        if not args.no_graph:
            row["graph_sparse_speedup_over_dense"] = round(
                row["dense"]["graph_ms_per_step"] / row["sparse"]["graph_ms_per_step"], 3)
            gtxt = (f"; graph replay: sparse {row['sparse']['graph_ms_per_step']:.3f} ms, dense "
                    f"{row['dense']['graph_ms_per_step']:.3f} ms ({row['graph_sparse_speedup_over_dense']:.2f}x)")
        out[str(Tn)] = row
        print(f"[bench] T={Tn}: sparse {row['sparse']['ms_per_step']:.3f} ms, dense "
              f"{row['dense']['ms_per_step']:.3f} ms per {len(layers)}-layer step "
              f"({row['sparse_speedup_over_dense']:.2f}x){gtxt}", file=sys.stderr, flush=True)
    return out


def grid_leg(args, dev):
    """Sec. 3.3 (batch 2 / 4 / 8, Fig. 8, Table 2) and Sec. 3.4 (keep budgets,
    Table 3): one layer of 32768 tokens per sequence, bf16, u ~ U(0, ln 16),
    keep 0.15 / 0.29 / 0.5 / 1.0 and the dense exact path at each batch;
    a step is 24 calls (the stack of the pages' timings; one input set is
    reused across the calls and the keep budgets, so that budgets compare on
    identical data)."""
    import torch
    from gated_deltanet_prefill_chunkwise_amd import ops, synth
    Tg, Bmax = 32768, 8
    inp = synth.torch_inputs(synth.seed_for(4, 0) + Bmax, Bmax, Tg, NQ, NV, dtype="bf16",
                             with_z=True, u_max=math.log(16.0), device=dev)
    o = torch.empty((Bmax, Tg, NV, D), dtype=torch.float16, device=dev)
    sf = torch.empty((Bmax, NV, D, D), dtype=torch.float32, device=dev)
    st = torch.zeros((Bmax, ops.STATS_INTS), dtype=torch.int32, device=dev)
    prob = ops.problem(inp["q"], inp["v"], "blockadj", torch.float16)
    ws = torch.empty(max(ops.workspace_bytes(prob, True, ops.sparse_params()),
                         ops.workspace_bytes(prob, False)), dtype=torch.uint8, device=dev)
    out = {}
    for Bg in (2, 4, 8):
        x = {k: v[:Bg] for k, v in inp.items()}
        row = {}
        for keep in (0.15, 0.29, 0.5, 1.0, "dense"):
            def step(_i, keep=keep):
                for _ in range(LAYERS):
                    if keep == "dense":
                        ops.prefill_dense(x["q"], x["k"], x["v"], x["a"], x["beta"], solve="exact",
                                          o=o[:Bg], s_final=sf[:Bg], workspace=ws)
                    else:
                        ops.prefill_sparse(x["q"], x["k"], x["v"], x["a"], x["beta"], z=x["z"],
                                           keep_budget=keep, solve="blockadj", o=o[:Bg],
                                           s_final=sf[:Bg], stats=st[:Bg], workspace=ws)
            mean, med = timed_steps(args, step)
            r = {"ms_per_step": round(mean, 4), "median_ms_per_step": round(med, 4),
                 "value_tok_s": round(Bg * Tg / (mean / 1e3), 1)}
            if keep != "dense":
                r["measured_keep"] = round(float(st[:Bg, 0].float().mean()) / (16 * Tg // 64), 5)
            row[str(keep)] = r
        for keep in (0.15, 0.29, 0.5, 1.0):
            row[str(keep)]["speedup_over_dense"] = round(row["dense"]["ms_per_step"] / row[str(keep)]["ms_per_step"], 3)
        out[f"batch{Bg}"] = row
        print(f"[bench] grid batch {Bg}: " + ", ".join(
            f"{k} {v['ms_per_step']:.2f} ms" for k, v in row.items()), file=sys.stderr, flush=True)
    del inp, o, sf, st, ws
    torch.cuda.empty_cache()
    return out


def decode_bytes_per_launch(Bd: int) -> int:
    """One decode launch: every head's fp32 state read and written once, plus
    the token's bf16 q, k, v, beta, fp32 a and the fp32 output."""
    state = Bd * NV * D * D * 4 * 2
    tok = Bd * (2 * NQ * D * 2 + NV * D * 2 + NV * 4 + NV * 2) + Bd * NV * D * 4
    return state + tok


def decode_leg(args, hip, dev):
    """Single-token decode step through the layer stack: Bd sequences, one
    in-place state per layer; HIP events around every launch."""
    import torch
    from gated_deltanet_prefill_chunkwise_amd import ops, synth
    Bd, L = args.decode_batch, args.layers
    lay = []
    for l in range(L):
        t = synth.torch_inputs(synth.seed_for(5, l), Bd, 1, NQ, NV, dtype="bf16", device=dev)
        t = {k: v[:, 0].contiguous() for k, v in t.items()}
        g = torch.Generator(device=dev)
        g.manual_seed(synth.seed_for(6, l))
        st = torch.randn((Bd, NV, D, D), generator=g, device=dev) * 0.3
        o = torch.empty((Bd, NV, D), dtype=torch.float32, device=dev)
        lay.append((t, st, o))
    stream = torch.cuda.current_stream()

    def step(evs):
        for l, (t, st, o) in enumerate(lay):
            if evs is not None:
                hip.lib.hipEventRecord(ctypes.c_void_p(evs[l]), ctypes.c_void_p(stream.cuda_stream))
            ops.decode_step(t["q"], t["k"], t["v"], t["a"], t["beta"], st, s_out=st, o=o)
        if evs is not None:
            hip.lib.hipEventRecord(ctypes.c_void_p(evs[L]), ctypes.c_void_p(stream.cuda_stream))

    hip.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    evs = [[hip.event() for _ in range(L + 1)] for _ in range(args.steps)]
    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for s in range(args.steps):
        step(evs[s])
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    launch_ms = sum(hip.elapsed_ms(evs[s][l], evs[s][l + 1])
                    for s in range(args.steps) for l in range(L)) / (args.steps * L)
    alg = decode_bytes_per_launch(Bd)
    achieved = alg / (launch_ms / 1e3) / 1e9
    print(f"[bench] decode: {ms:.3f} ms per {L}-layer step at batch {Bd}; "
          f"{launch_ms * 1e3:.1f} us per launch", file=sys.stderr, flush=True)
    return {"value_tok_s": round(Bd / (ms / 1e3), 1), "unit": f"tok/s ({L}-layer stack, batch {Bd})",
            "ms_per_step": round(ms, 4), "batch": Bd, "layers": L, "state_dtype": "fp32",
            "roofline": dict(bound="hbm", kernel="decode", achieved=round(achieved, 1),
                             peak=HBM_PEAK_GBS, unit="GB/s", frac=round(achieved / HBM_PEAK_GBS, 4),
                             traffic=measured_traffic("decode", "decode"),
                             algorithmic_bytes_per_launch=alg,
                             launch_ms=round(launch_ms, 5))}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the GDN-core prefill here runs on a single MI355X "
              "(no sharding, no collectives); --gpus N > 1 is not supported.", file=sys.stderr)
        sys.exit(2)

    import torch
    from gated_deltanet_prefill_chunkwise_amd import ops, synth

    torch.cuda.set_device(0)
    dev = "cuda:0"
    if args.copy_calibration:
        # plain copy kernel of known size: 1 GiB read + 1 GiB written per launch
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read_per_launch": src.numel() * 4,
                          "copy_bytes_written_per_launch": dst.numel() * 4, "launches": 3}))
        return
    hip = Hip()
    L, Tn = args.layers, args.seqlen
    C = -(-Tn // 64)
    layers = []
    for l in range(L):
        inp = synth.torch_inputs(synth.seed_for(3, l), B, Tn, NQ, NV, dtype="bf16", with_z=True,
                                 device=dev)
        o = torch.empty((B, Tn, NV, D), dtype=torch.float16, device=dev)
        sf = torch.empty((B, NV, D, D), dtype=torch.float32, device=dev)
        st = torch.zeros((B, ops.STATS_INTS), dtype=torch.int32, device=dev)
        layers.append((inp, o, sf, st))
    prob = ops.problem(layers[0][0]["q"], layers[0][0]["v"], "blockadj", torch.float16)
    ws_bytes = max(ops.workspace_bytes(prob, True, ops.sparse_params()),
                   ops.workspace_bytes(prob, False))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def run_mode(mode):
        nev = len(STAGES) + 1
        events = [[[hip.event() for _ in range(nev)] for _ in range(L)] for _ in range(args.steps)]
        dbgs = [[ops.debug_struct(events=events[s][l]) for l in range(L)] for s in range(args.steps)]

        def step(dbg_row):
            for l, (inp, o, sf, st) in enumerate(layers):
                dbg = dbg_row[l] if dbg_row is not None else None
                if mode == "sparse":
                    ops.prefill_sparse(inp["q"], inp["k"], inp["v"], inp["a"], inp["beta"],
                                       z=inp["z"], keep_budget=0.29, solve="blockadj", o=o,
                                       s_final=sf, stats=st, workspace=ws, debug=dbg)
                else:
                    ops.prefill_dense(inp["q"], inp["k"], inp["v"], inp["a"], inp["beta"],
                                      solve="exact", o=o, s_final=sf, workspace=ws, debug=dbg)

        for _ in range(args.warmup):
            step(None)
        torch.cuda.synchronize()
        t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        w0 = time.perf_counter()
        t_start.record()
        marks[0].record()
        for s in range(args.steps):
            step(dbgs[s])
            marks[s + 1].record()
        t_end.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - w0
        ms = t_start.elapsed_time(t_end) / args.steps
        import statistics
        med = statistics.median(marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps))
        stage_ms = {}
        for i, name in enumerate(STAGES):
            tot = sum(hip.elapsed_ms(events[s][l][i], events[s][l][i + 1])
                      for s in range(args.steps) for l in range(L))
            stage_ms[name] = tot / (args.steps * L)
        stats = torch.stack([st for (_, _, _, st) in layers]).cpu()
        gmean, gmed = (None, None) if args.no_graph else graph_steps(args, step)
        return dict(ms_per_step=ms, median_ms_per_step=med, wall_s=wall, stage_ms_per_launch=stage_ms,
                    stats=stats, graph_ms_per_step=gmean, graph_median_ms_per_step=gmed)

    res = {}
    for mode in (("sparse", "dense") if args.mode == "both" else (args.mode,)):
        res[mode] = run_mode(mode)
        gtxt = "" if args.no_graph else f" (graph replay {res[mode]['graph_ms_per_step']:.3f} ms)"
        print(f"[bench] {mode}: {res[mode]['ms_per_step']:.3f} ms per {L}-layer step{gtxt}; stages (ms/launch) "
              + ", ".join(f"{k} {v:.3f}" for k, v in res[mode]["stage_ms_per_launch"].items()),
              file=sys.stderr, flush=True)

    head = "sparse" if "sparse" in res else "dense"
    r = res[head]
    value = B * Tn / (r["ms_per_step"] / 1e3)

    # keep fraction and snapshot fraction (sparse) from the device statistics
    keep = sigma = 1.0
    if "sparse" in res:
        stt = res["sparse"]["stats"].float()[:, 0, :]          # [layers, 9]
        keep = float((stt[:, 0] / (16 * C)).mean())
        G = (C + 1) // 2
        sigma = float((stt[:, 8] / (16 * max(G - 1, 1))).mean())

    def roofline(mode):
        st = res[mode]["stage_ms_per_launch"]
        dom = max(st, key=st.get)
        bpt = algorithmic_bytes_per_token(dom, mode, sigma, keep)
        alg = bpt * B * Tn
        achieved = alg / (st[dom] / 1e3) / 1e9
        traffic = measured_traffic(dom, mode)
        return dict(bound="hbm", kernel=dom, achieved=round(achieved, 1), peak=HBM_PEAK_GBS,
                    unit="GB/s", frac=round(achieved / HBM_PEAK_GBS, 4), traffic=traffic,
                    algorithmic_bytes_per_launch=int(alg), launch_ms=round(st[dom], 4))

    def path_roofline(mode, o_bytes=2):
        """The whole layer against HBM: the I/O streams (the 2-byte O this run
        writes) plus the snapshots, over the measured time per layer."""
        per_layer_ms = res[mode]["ms_per_step"] / args.layers
        alg = path_bytes_per_token(mode, sigma if mode == "sparse" else 1.0, o_bytes) * B * Tn
        achieved = alg / (per_layer_ms / 1e3) / 1e9
        return dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4), algorithmic_bytes_per_layer=int(alg),
                    bytes_per_token=round(alg / (B * Tn), 1), o_bytes=o_bytes,
                    ms_per_layer=round(per_layer_ms, 4),
                    roofline_ms_per_layer=round(alg / (HBM_PEAK_GBS * 1e9) * 1e3, 4))

    def mfma_roofline(mode):
        """The whole layer against the dense bf16 matrix-core peak with the
        method's algorithmic flops (keep = measured event fraction)."""
        per_layer_ms = res[mode]["ms_per_step"] / args.layers
        fl = flops_per_token(mode, keep if mode == "sparse" else 1.0) * B * Tn
        achieved = fl / (per_layer_ms / 1e3) / 1e12
        return dict(bound="mfma", achieved=round(achieved, 1), peak=MFMA_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=round(achieved / MFMA_PEAK_TFLOPS, 4), flops_per_layer=int(fl),
                    roofline_ms_per_layer=round(fl / (MFMA_PEAK_TFLOPS * 1e12) * 1e3, 4))

    out = {
        "metric": "GDN-core prefill tokens/s at T=32K/128K, dense vs 29% events; % roofline",
        "value": round(value, 1),
        "unit": "tok/s (24-layer GDN-core stack)" if args.layers == LAYERS else f"tok/s ({args.layers}-layer stack)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{args.layers} independently seeded GDN layers, GDN-core only, "
                               f"{head} path" + (" (SparseGDN, keep budget 0.29, block-adjacent solve)"
                                                 if head == "sparse" else " (exact solve)"),
                   "batch": B, "seq_len": Tn, "n_qk_heads": NQ, "n_v_heads": NV, "d": D,
                   "layers": args.layers, "o_dtype": O_DTYPE, "parallelism": "none (1 GPU)"},
        "roofline": roofline(head),
    }
    for mode, rr in res.items():
        pr, mr = path_roofline(mode), mfma_roofline(mode)
        out[mode] = {"value_tok_s": round(B * Tn / (rr["ms_per_step"] / 1e3), 1),
                     "per_layer_tok_s": round(B * Tn / (rr["ms_per_step"] / 1e3 / args.layers), 1),
                     "ms_per_step": round(rr["ms_per_step"], 4),
                     "median_ms_per_step": round(rr["median_ms_per_step"], 4),
                     "graph_ms_per_step": None if args.no_graph else round(rr["graph_ms_per_step"], 4),
                     "graph_median_ms_per_step": None if args.no_graph else round(rr["graph_median_ms_per_step"], 4),
                     "stage_ms_per_launch": {k: round(v, 4) for k, v in rr["stage_ms_per_launch"].items()},
                     "roofline": roofline(mode), "path_roofline": pr, "mfma_roofline": mr,
                     "binding_roofline": "hbm" if pr["roofline_ms_per_layer"] >= mr["roofline_ms_per_layer"] else "mfma"}
    # group-entry snapshot memory per layer: the workspace holds a slot for
    # every group boundary (fp16, 128 x 128 per head); the compact snapshots
    # the sparse H scan writes use n_snapshots of the pair slots
    G = (C + 1) // 2
    snap_head = 128 * 128 * 2
    for mode in res:
        alloc = B * NV * max(G - 1, 1) * snap_head
        used = alloc if mode == "dense" else int(round(sigma * alloc))
        out[mode]["snapshot_bytes"] = {"allocated": alloc, "used": used}
    if "sparse" in res:
        out["sparse"]["measured_keep"] = round(keep, 5)
        out["sparse"]["snapshot_fraction"] = round(sigma, 5)
    if "sparse" in res and "dense" in res:
        out["sparse_speedup_over_dense"] = round(res["dense"]["ms_per_step"] / res["sparse"]["ms_per_step"], 3)
    if not args.no_sweep and args.mode == "both":
        out["length_sweep"] = sweep_leg(args, layers, ws)
        if "32768" in out["length_sweep"]:
            out["t32k"] = out["length_sweep"]["32768"]
    if not args.no_grid and args.mode == "both":
        out["keep_batch_grid"] = grid_leg(args, dev)
    if not args.no_ablations and "sparse" in res:
        out["pipeline_ablations"] = ablation_leg(args, layers, hip, prob, dev)
    if not args.no_variants and "sparse" in res:
        # the rank-key variant needs one more rank table in the workspace
        key_shape = torch.empty((B, NV // 2, C), device=dev)
        vws = torch.empty(ops.workspace_bytes(prob, True, ops.sparse_params(rank_key=key_shape)),
                          dtype=torch.uint8, device=dev)
        out["selector_variants"] = variants_leg(args, layers, vws, C)
        del vws
    if not args.no_output_types and args.mode == "both":
        out["output_types"] = output_leg(args, layers, ws)
    if not args.no_varlen and args.mode == "both":
        out["varlen"] = varlen_leg(args, layers, hip)
    if args.decode_batch > 0:
        out["decode"] = decode_leg(args, hip, dev)
    out["cpu_baseline"] = None
    if not args.no_cpu_baseline:
        try:
            out["cpu_baseline"] = cpu_baseline(layers, args.cpu_tokens, args.cpu_workers)
        except Exception as e:   # the GPU figures above stand without it
            print(f"[bench] cpu baseline failed: {e!r}", file=sys.stderr, flush=True)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
