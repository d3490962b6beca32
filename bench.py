#!/usr/bin/env python3
"""Throughput of the chunked Gated DeltaNet forward + backward on one MI355X.

One step = gdr_forward (keeping the per-chunk results for the backward) followed by
gdr_backward, i.e. every stage of the operator's training path, on one batch of seeded
synthetic inputs already resident in HBM.  The default workload is the long-context Gated
DeltaNet case: B=1, H=16, T=32768 packed as four sequences (4096, 8192, 12288, 8192 tokens),
d_k = d_v = 128, bf16 inputs, float32 initial memory per sequence.

Prints one JSON line.  `value` is tokens/s = B*T / (time of one step), timed with the
backward's pipelines on (GDR_PIPELINE=1: the reverse scans of the longest sequences, or the
earlier half of a single long one, overlap the chunk gradients of the rest on side streams;
results bitwise the single-stream ones); `ms_per_step_single_stream` is the same step with them
off (--single-stream times the headline that way too).  `roofline` is the dominant kernel
against MI355X's 8 TB/s: its algorithmic bytes (the operator's own tensors it reads or writes,
each once; no per-chunk intermediate) over its average launch time, timed with HIP events
around its launches in every fourth step of a separate single-stream pass (the last included),
where no launch overlaps another; `io_bytes`/`io_frac` beside it count everything the kernel
moves, intermediates included; `measured_copy_GBps` is what a plain 1 GiB device copy reaches
on the same GPU (the practical ceiling beside the published peak) and `frac_of_measured_copy`
the kernel's algorithmic rate against it.  `device` names the GPU as the runtime reports it.
`path_roofline` is the whole step against the bytes the operator must move at minimum.
`sweep` times T = 4k..32k at B*T = 32768 (ratio t(32k)/t(4k) beside the pages' ~1.1x);
`ms_per_step_flushed` times steps separated by a 512 MiB write that evicts the last-level cache.
`cpu_baseline` is the float64 oracle, timed on a bounded sample of the same workload over a
process pool on this host's cores, before the GPU is touched.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload NAME] [--no-sweep] [--single-stream]
"""
from __future__ import annotations

import argparse
import ctypes
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
COPY_CAL_BYTES = 256 << 20   # size of the calibration copy (read + write of this many bytes)
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 matrix cores, published

def kernel_bytes_per_unit(variant: str, kernel: str, D: int = 128, esz: int = 2, has_beta: bool = True,
                          residual: bool = False) -> int:
    """Bytes a kernel must read and write once per (chunk, head) unit: its inputs and outputs,
    each touched once (C = 64 tokens, head size D, I/O element size esz).  The per-chunk
    intermediates the kernels hand to each other (X, U, M, R, memories, float32 partial
    gradients) are inputs and outputs of the kernels that use them.  residual: the forward also
    writes r and the backward reads its gradient dr (with bfloat16 I/O the reverse scan then also
    writes dR without the residual's term, for the separate beta gradient)."""
    C = 64
    TOK, SQR, GRAM, GATE = C * D * esz, D * D * esz, C * C * esz, C * esz
    GLOG, FTOK, FGRAM, FD = C * 4, C * D * 4, C * C * 4, D * 4
    kda, g2, gla = variant == "kda", variant == "gdn2", variant == "gla"
    ALPHA = 0 if variant == "deltanet" else (TOK if (kda or gla) else GATE)
    BETA = GATE if has_beta else 0
    DEC = FD if (kda or gla) else GLOG  # per-chunk decay handed to the scans
    OUT = TOK + GRAM + TOK  # the forward scan also reads q and M and writes o
    XT = 0 if gla else TOK  # the erase-free memory has no X
    table = {
        "fwd_prep": 3 * TOK + BETA + ALPHA + 2 * TOK + GRAM + GLOG + FGRAM,
        "fwd_prep_kda": 3 * TOK + BETA + ALPHA + 4 * TOK + GRAM + FD + 2 * FGRAM,
        "fwd_prep_gdn2": 5 * TOK + BETA + ALPHA + 3 * TOK + 2 * GRAM + GLOG + 3 * FGRAM,
        "fwd_prep_gla": 3 * TOK + BETA + ALPHA + 3 * TOK + GRAM + FD,
        "fwd_scan": (6 * TOK + BETA if g2 else 2 * TOK + XT) + DEC + SQR + TOK + OUT + (GRAM if g2 else 0),
        "bwd_scan": 2 * TOK + XT + TOK + GRAM + DEC + SQR + TOK + ((TOK + BETA) if g2 else 0),
        "bwd_gla_state": 2 * TOK + 2 * SQR + FD + 2 * FTOK + GRAM + FD,
        "bwd_gla_wv": 3 * TOK + 2 * BETA,
        "bwd_gla_gram": 2 * TOK + ALPHA + GRAM + 2 * FTOK + FD + 2 * TOK + ALPHA,
        "bwd_chunk": 4 * TOK + BETA + ALPHA + GRAM + GLOG + 2 * SQR + 2 * TOK + 3 * TOK + BETA + ALPHA + FGRAM,
        "bwd_kda_state": 3 * TOK + 2 * SQR + FD + 3 * FTOK + GRAM + FD,
        "bwd_kda_wy": 3 * TOK + BETA + ALPHA + FTOK + 2 * FGRAM + TOK + BETA + FTOK + GRAM,
        "bwd_kda_gram": 2 * TOK + ALPHA + 2 * GRAM + 3 * FTOK + FD + 2 * TOK + ALPHA,
        "bwd_gdn2_state": 5 * TOK + GLOG + BETA + 2 * SQR + 2 * TOK + 5 * FTOK + 2 * FGRAM + 4 * GLOG,
        "bwd_gdn2_wy": 3 * TOK + GLOG + BETA + 2 * FGRAM + 3 * TOK + GRAM + 3 * FTOK + 2 * TOK + 2 * FGRAM + FTOK
                       + 4 * GLOG,
        "bwd_gdn2_gram": 3 * TOK + BETA + ALPHA + GLOG + 2 * GRAM + 6 * FGRAM + 3 * FTOK + 4 * GLOG
                         + 3 * TOK + BETA + ALPHA,
        "fwd_seg_combine": 0, "bwd_seg_combine": 0,
        # the delta family forms A from K and the log decays; Kimi Delta Attention reads it
        "bwd_res_dbeta": 3 * TOK + BETA + (2 * FGRAM if kda else TOK + GLOG + FGRAM) + BETA,
    }
    if residual:
        table["fwd_scan"] += TOK
        table["bwd_scan"] += TOK + BETA + (TOK if esz == 2 else 0)
        table["bwd_chunk"] += TOK
    if kernel in ("fwd_scan_maps", "bwd_scan_maps"):  # no per-chunk records, twice the value tiles
        base = table[kernel[:8]] - (SQR + TOK + (OUT if kernel.startswith("fwd") else 0))
        return base
    return table[kernel]


def kernel_operator_bytes(variant: str, kernel: str, D: int = 128, esz: int = 2, has_beta: bool = True,
                          residual: bool = False) -> int:
    """Algorithmic bytes of one kernel per head-token: the operator's own tensors (forward q, k,
    v, gates, o; backward q, k, v, dO, gates and every gradient) that the kernel itself reads or
    writes, each counted once.  Per-chunk intermediates (X, U, M, R, stored memories, partial
    gradients) are not counted, so these are the bytes no implementation of the kernel's role
    can avoid.  The chunk-parallel backward of the delta family reads every token tensor the
    backward needs and writes every gradient: the backward's whole 1800 B at d = 128 (bf16)."""
    TOK = D * esz
    BETA = esz if has_beta else 0
    kda, g2 = variant in ("kda", "gla"), variant == "gdn2"
    ALPHA = {"deltanet": 0, "gated": esz, "kda": TOK, "gdn2": esz, "gla": TOK}[variant]
    EW = 2 * TOK if g2 else 0                         # erase [d_k] and write [d_v] gates
    qk = 0 if kda else 2 * TOK                        # per-channel decay: the scans read per-chunk copies
    table = {
        "fwd_prep": 3 * TOK + BETA + ALPHA + EW,
        "fwd_scan": TOK + qk + ((TOK + EW + BETA) if g2 else 0),
        "fwd_scan_maps": (TOK if not kda else 0) + ((TOK + EW + BETA) if g2 else 0),
        "bwd_scan": TOK + qk + ((TOK + BETA) if g2 else 0),
        "bwd_chunk": 4 * TOK + BETA + ALPHA + 3 * TOK + BETA + ALPHA,
        "bwd_kda_state": TOK,
        "bwd_kda_wy": 2 * TOK + BETA + ALPHA + TOK + BETA,
        "bwd_kda_gram": 2 * TOK + ALPHA + 2 * TOK + ALPHA,
        "bwd_gdn2_state": 3 * TOK + EW + BETA,
        "bwd_gdn2_wy": 3 * TOK + EW + BETA + 2 * TOK,
        "bwd_gdn2_gram": 3 * TOK + BETA + ALPHA + 3 * TOK + BETA + ALPHA,
        "bwd_res_dbeta": TOK + BETA + (0 if kda else TOK) + BETA,
        "bwd_gla_state": TOK,
        "bwd_gla_wv": 2 * TOK + 2 * BETA,
        "bwd_gla_gram": 2 * TOK + ALPHA + 2 * TOK + ALPHA,
        "fwd_seg_combine": 0, "bwd_seg_combine": 0,
    }
    table["fwd_prep_kda"] = table["fwd_prep_gdn2"] = table["fwd_prep_gla"] = table["fwd_prep"]
    table["bwd_scan_maps"] = table["bwd_scan"]
    if residual:
        table["fwd_scan"] += TOK
        table["bwd_scan"] += TOK + BETA
        table["bwd_chunk"] += TOK
    return table[kernel]


def kernel_state_bytes(kernel: str, D: int, has_h0: bool) -> int:
    """Per (sequence, head): float32 memories a kernel reads or writes as operator tensors (the
    forward scan reads h0 and writes ht, the reverse scan writes dh0; dht is not given)."""
    sq = D * D * 4
    return {"fwd_scan": (sq if has_h0 else 0) + sq, "bwd_scan": sq}.get(kernel, 0)


def path_bytes_per_head_token(variant: str, D: int = 128, esz: int = 2, has_beta: bool = True,
                              residual: bool = False) -> int:
    """The operator's own minimum per head-token: the forward reads q, k, v and the gates and
    writes o; the backward reads q, k, v, the gates and dO and writes the gradients of q, k,
    v and of every gate (Gated, d = 128, bf16: 2828 bytes).  residual: r written, dr read."""
    tok = D * esz
    beta = esz if has_beta else 0
    gates = beta + {"deltanet": 0, "gated": esz, "kda": tok, "gdn2": esz + 2 * tok, "gla": tok}[variant]
    return (3 * tok + gates + tok) + (4 * tok + gates + 3 * tok + gates) + (2 * tok if residual else 0)


def source_sha() -> str:
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "gated_delta_rule_73_amd", "csrc", "*"))):
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter summaries, if they were taken on
    the current kernel sources; None otherwise."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    d = json.load(open(path))
    if d.get("source_sha") != source_sha():
        return None
    return d.get("bytes_per_launch")


CPU_POOL_MAX = 16  # worker processes at most (the host's share for one GPU)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_item(item):
    """One work item of the CPU baseline: the float64 oracle's forward + backward of one
    (sequence, head) slice, BLAS held to one thread.  Returns (head-tokens, seconds)."""
    from threadpoolctl import threadpool_limits

    from oracle import recurrence as R
    kw, do, variant = item
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        R.forward(**kw, variant=variant)
        if do is not None:
            R.backward(**kw, do=do, variant=variant)
        wall = time.perf_counter() - t0
    return kw["q"].shape[1] * kw["q"].shape[2], wall


def _pool_run(items):
    """Runs the items over a process pool of the host's cores (at most CPU_POOL_MAX); returns
    (wall seconds, workers).  Called before anything touches the GPU (the workers are forked)."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor
    workers = max(1, min(len(os.sched_getaffinity(0)), CPU_POOL_MAX, len(items)))
    t0 = time.perf_counter()
    with ProcessPoolExecutor(workers, mp_context=mp.get_context("fork")) as ex:
        list(ex.map(_oracle_item, items))
    return time.perf_counter() - t0, workers


def cpu_baseline(w, inp, tokens_per_seq: int = 4096):
    """Time the oracle (float64, token by token) on a bounded sample of the workload: the first
    `tokens_per_seq` tokens of every sequence, every head, forward + backward, over a process
    pool.  A task is one sequence and a group of heads (the oracle steps the heads of a task
    together, so groups are as large as the pool allows).  tokens/s counts a token as all H
    heads of it."""
    cu = inp.get("cu_seqlens")
    spans = [(0, int(a), int(b), n) for n, (a, b) in enumerate(zip(cu[:-1], cu[1:]))] if cu is not None \
        else [(b, 0, w.T, b) for b in range(w.B)]
    workers = max(1, min(len(os.sched_getaffinity(0)), CPU_POOL_MAX))
    groups = max(1, min(w.H, workers // len(spans)))
    hb = [(w.H * i // groups, w.H * (i + 1) // groups) for i in range(groups)]
    items = []
    for b, a, e, n in spans:
        e = min(e, a + tokens_per_seq)
        for h0, h1 in hb:
            kw = {x: (None if inp.get(x) is None else inp[x][b:b + 1, h0:h1, a:e])
                  for x in ("q", "k", "v", "beta", "alpha", "erase", "write")}
            kw["h0"] = None if inp.get("h0") is None else inp["h0"][n:n + 1, h0:h1]
            items.append((kw, inp["do"][b:b + 1, h0:h1, a:e] if w.backward else None, w.variant))
    head_tokens = sum(it[0]["q"].shape[1] * it[0]["q"].shape[2] for it in items)
    wall, used = _pool_run(items)
    return {"value": round(head_tokens / w.H / wall, 1), "unit": "tokens/s", "cores": used, "kind": "oracle",
            "cpu_model": cpu_model(), "host_cores_visible": len(os.sched_getaffinity(0)),
            "sample": f"forward{'+backward' if w.backward else ''} of the first {tokens_per_seq} tokens of each of "
                      f"the {len(spans)} sequences, all {w.H} heads ({head_tokens} head-tokens), d={w.dk}, "
                      f"float64 numpy; {len(items)} tasks (a sequence and {w.H // groups} heads each) over "
                      f"{used} processes with one BLAS thread each; {wall:.1f} s wall"}


def _dev(x, dtype: str):
    """A float32 numpy array on the GPU in the I/O dtype (bf16 values are exact: they were
    rounded when drawn)."""
    import numpy as np
    import torch
    if x is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def _dev_inputs(inp, dtype: str) -> dict:
    return {n: _dev(inp.get(n), "f32" if n == "h0" else dtype)
            for n in ("q", "k", "v", "beta", "alpha", "erase", "write", "h0")}


class Runner:
    """Holds the device buffers of one workload and calls the C ABI directly.  residual: the
    forward also writes r = v - v_bar (gdr_forward_residual) and the backward takes a seeded
    standard-normal gradient dr of it (gdr_backward_residual); gate_logits: beta and alpha are
    logits, activated inside the kernels."""

    def __init__(self, w, inp, residual: bool = False, gate_logits: bool = False, qk_norm: bool = False):
        import torch

        from gated_delta_rule_73_amd import binding as bd
        self.bd = bd
        self.lib = bd.load_library()
        self.w = w
        g = _dev_inputs(inp, w.dtype)
        self.g = g
        self.do = _dev(inp["do"], w.dtype)
        self.p, self.keep = bd.make_problem(g["q"], g["v"], variant=w.variant, cu_seqlens=inp.get("cu_seqlens"),
                                            gate_logits=gate_logits, qk_norm=qk_norm)
        N = self.p.n_seqs if self.p.n_seqs > 0 else self.p.B
        dev = g["q"].device
        self.o = torch.empty_like(g["v"])
        self.r = torch.empty_like(g["v"]) if residual else None
        self.dr = None
        if residual:
            import numpy as np
            self.dr = _dev(np.random.default_rng(w.seed + 17).standard_normal(inp["v"].shape), w.dtype)
        self.ht = torch.empty((N, w.H, w.dv, w.dk), dtype=torch.float32, device=dev)
        self.saved = torch.empty(bd.gdr_saved_size(self.p), dtype=torch.uint8, device=dev)
        nws = bd.gdr_workspace_size(self.p, True)
        self.ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
        self.grads = {n: (None if g[x] is None else torch.empty_like(g[x]))
                      for n, x in (("dq", "q"), ("dk", "k"), ("dv", "v"), ("dbeta", "beta"),
                                   ("dalpha", "alpha"), ("derase", "erase"), ("dwrite", "write"))}
        self.grads["dh0"] = torch.empty_like(self.ht)
        self.ins = bd._inputs(*(g[n] for n in ("q", "k", "v", "beta", "alpha", "erase", "write", "h0")))
        self.gr = bd.GdrGrads(**{n: bd._ptr(t) for n, t in self.grads.items()})
        self.stream = torch.cuda.current_stream().cuda_stream

    def fwd(self):
        st = self.lib.gdr_forward_residual(ctypes.byref(self.p), ctypes.byref(self.ins), self.o.data_ptr(),
                                           None if self.r is None else self.r.data_ptr(), self.ht.data_ptr(),
                                           self.saved.data_ptr(), self.ws.data_ptr(), self.ws.numel(),
                                           self.stream)
        self.bd._check(self.lib, st)

    def bwd(self):
        st = self.lib.gdr_backward_residual(ctypes.byref(self.p), ctypes.byref(self.ins), self.do.data_ptr(),
                                            None if self.dr is None else self.dr.data_ptr(), None,
                                            self.saved.data_ptr(), ctypes.byref(self.gr), self.ws.data_ptr(),
                                            self.ws.numel(), self.stream)
        self.bd._check(self.lib, st)

    calls = property(lambda self: (self.fwd, self.bwd))

    def step(self):
        self.fwd()
        self.bwd()


class DecodeRunner:
    """Device buffers of a decoding workload; one step = one gdr_decode call (every sequence's
    new tokens through its memory, updated in place)."""

    def __init__(self, w, inp):
        import torch

        from gated_delta_rule_73_amd import binding as bd
        self.bd = bd
        self.lib = bd.load_library()
        g = _dev_inputs(inp, w.dtype)
        self.p, self.keep = bd.make_problem(g["q"], g["v"], variant=w.variant, cu_seqlens=inp.get("cu_seqlens"))
        self.state = g["h0"]
        self.o = torch.empty_like(g["v"])
        self.g = g
        self.ins = bd._inputs(*(g[n] for n in ("q", "k", "v", "beta", "alpha", "erase", "write")), None)
        self.stream = torch.cuda.current_stream().cuda_stream

    def dec(self):
        st = self.lib.gdr_decode(ctypes.byref(self.p), ctypes.byref(self.ins), self.state.data_ptr(),
                                 self.o.data_ptr(), self.stream)
        self.bd._check(self.lib, st)

    calls = property(lambda self: (self.dec,))

    def step(self):
        self.dec()


def decode_bytes(w, esz: int) -> int:
    """Bytes one decoding step must move: every float32 memory read and written once, plus the
    new tokens' q, k, v, gates and o."""
    N = w.n_states
    state = 2 * N * w.H * w.dv * w.dk * 4
    per_tok = (2 * w.dk + w.dv + w.dv) * esz + (esz if w.has_beta else 0)
    per_tok += {"deltanet": 0, "gated": esz, "kda": w.dk * esz, "gdn2": esz + (w.dk + w.dv) * esz}[w.variant]
    return state + w.B * w.H * w.T * per_tok


def cpu_baseline_decode(w, inp):
    """The oracle's forward over the whole decoding step, split into slices of sequences over
    a process pool (decoding has no backward)."""
    per = max(1, w.B // CPU_POOL_MAX)
    items = []
    for b0 in range(0, w.B, per):
        kw = {n: (None if inp.get(n) is None else inp[n][b0:b0 + per])
              for n in ("q", "k", "v", "beta", "alpha", "erase", "write", "h0")}
        items.append((kw, None, w.variant))
    wall, workers = _pool_run(items)
    tokens = w.B * w.T
    return {"value": round(tokens / wall, 1), "unit": "tokens/s", "cores": workers, "kind": "oracle",
            "cpu_model": cpu_model(), "host_cores_visible": len(os.sched_getaffinity(0)),
            "sample": f"the whole step ({w.B} sequences x {w.H} heads, {w.T} token each), float64 numpy, "
                      f"{len(items)} slices of sequences over {workers} processes; {wall:.2f} s wall"}


def bench_decode(args, w):
    import synth
    print(f"[bench] generating {w.name} inputs", file=sys.stderr, flush=True)
    inp = synth.make_inputs(w)
    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the CPU", file=sys.stderr, flush=True)
        cpu = cpu_baseline_decode(w, inp)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    runner = DecodeRunner(w, inp)
    copy_gbs = measured_copy_gbs()
    print("[bench] timing", file=sys.stderr, flush=True)
    ms, per_kernel = timed(runner, args.steps, args.warmup)
    esz = 2 if w.dtype == "bf16" else 4
    nbytes = decode_bytes(w, esz)
    avg_ms = sum(per_kernel["decode"]) / len(per_kernel["decode"])
    achieved = nbytes / (avg_ms / 1e3) / 1e9
    tokens = w.B * w.T
    out = {
        "metric": "tokens/s recurrent decode step (gdr_decode), H=16 d=128; % of HBM roofline",
        "value": round(tokens / (ms / 1e3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic (seeded; distributions of the workload definition)",
        "config": {"workload": w.name, "variant": w.variant, "B": w.B, "H": w.H, "T": w.T, "d_k": w.dk,
                   "d_v": w.dv, "state": "float32, updated in place"},
        "roofline": {"bound": "hbm", "kernel": "decode", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic("decode", w.name),
                     "avg_launch_ms": round(avg_ms, 4), "launches": len(per_kernel["decode"]),
                     "algorithmic_bytes_per_launch": nbytes,
                     "measured_copy_GBps": round(copy_gbs, 1), "frac_of_measured_copy": round(achieved / copy_gbs, 4)},
        "device": device_info(),
    }
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out))


def make_events(n):
    import torch
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in evs:  # create the underlying hipEvent_t handles
        e.record()
    torch.cuda.synchronize()
    return evs


TRACE_EVERY = 4


def traced_steps(steps: int, trace_every: int = TRACE_EVERY) -> int:
    """How many of `steps` timed steps timed() brackets with events (the last and every
    trace_every-th before it)."""
    return (steps - 1) // trace_every + 1


def timed(runner, steps: int, warmup: int, trace: bool = True, trace_every: int = TRACE_EVERY):
    """Warm up, then time `steps` steps between two events (synchronized on both sides).
    With trace, every kernel launch of every `trace_every`-th timed step (counted back from the
    last, which is always traced) is bracketed by its own event pair.  The event records stall
    the stream briefly (about 0.05 ms per fully traced step at the packed 32k workload, 3%), so
    sampling the steps keeps that out of the throughput while the launch durations, which the
    events bracket exactly, are unaffected."""
    import torch
    for _ in range(warmup):
        runner.step()
    torch.cuda.synchronize()
    per_call = 64  # launches recorded per call at most (the library names 64)
    evs = make_events(2 * per_call * 2 * steps) if trace else []
    handles = (ctypes.c_void_p * max(1, len(evs)))(*[e.cuda_event for e in evs]) if trace else None
    names = []
    start, end = make_events(2)
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        traced = trace and (steps - 1 - i) % trace_every == 0
        for j, call in enumerate(runner.calls):
            if traced:
                off = (2 * i + j) * 2 * per_call
                runner.lib.gdr_trace_launches(ctypes.cast(ctypes.byref(handles, off * ctypes.sizeof(ctypes.c_void_p)),
                                                          ctypes.c_void_p), 2 * per_call)
            call()
            if traced:
                n = min(runner.lib.gdr_traced_launches(), per_call)  # later launches are not recorded
                names.append([(off, k, runner.lib.gdr_traced_launch_name(k).decode()) for k in range(n)])
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    per_kernel = {}
    for call in names:
        for off, k, name in call:
            t = evs[off + 2 * k].elapsed_time(evs[off + 2 * k + 1])
            per_kernel.setdefault(name, []).append(t)
    return ms, per_kernel


FLUSH_BYTES = 512 << 20  # twice MI355X's 256 MiB last-level (Infinity) cache
COPY_BW_BYTES = 1 << 30  # the bandwidth copy: four times the last-level cache


def device_info() -> dict:
    """The GPU the line was measured on, as the runtime reports it."""
    import torch
    pr = torch.cuda.get_device_properties(0)
    return {"name": pr.name, "arch": getattr(pr, "gcnArchName", None), "compute_units": pr.multi_processor_count,
            "memory_GiB": round(pr.total_memory / (1 << 30), 1)}


def measured_copy_gbs(reps: int = 10) -> float:
    """HBM bandwidth a plain device-to-device copy reaches on this GPU (read + write bytes over
    the median time of `reps` copies of 1 GiB), the practical ceiling beside the published peak."""
    import torch
    src = torch.empty(COPY_BW_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    evs = make_events(2 * reps)
    for i in range(reps):
        evs[2 * i].record()
        dst.copy_(src)
        evs[2 * i + 1].record()
    torch.cuda.synchronize()
    ms = sorted(evs[2 * i].elapsed_time(evs[2 * i + 1]) for i in range(reps))[reps // 2]
    del src, dst
    torch.cuda.empty_cache()
    return 2 * COPY_BW_BYTES / (ms / 1e3) / 1e9


def timed_flushed(runner, steps: int) -> float:
    """ms per step with a 512 MiB write between steps (outside the timed spans), so that no
    step finds its inputs in the last-level cache left by the one before."""
    import torch
    buf = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    evs = make_events(2 * steps)
    for i in range(steps):
        buf.fill_(float(i))
        evs[2 * i].record()
        runner.step()
        evs[2 * i + 1].record()
    torch.cuda.synchronize()
    del buf
    return sum(evs[2 * i].elapsed_time(evs[2 * i + 1]) for i in range(steps)) / steps


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gated_varlen_T32768")
    ap.add_argument("--no-sweep", action="store_true", help="skip the T = 4k..32k sweep at B*T = 32768")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--residual", action="store_true", help="the forward also writes the residual r = v - v_bar and the backward takes its gradient")
    ap.add_argument("--gate-logits", action="store_true", help="beta and alpha given as logits")
    ap.add_argument("--qk-norm", action="store_true", help="q and k scaled to unit length inside the library")
    ap.add_argument("--single-stream", action="store_true",
                    help="time the headline with the backward's pipelines off (GDR_PIPELINE=0)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): the operator "
              "has no multi-GPU path here; see the design notes for how it would shard.", file=sys.stderr)
        sys.exit(2)
    import synth
    if args.workload in synth.DECODE_WORKLOADS:
        bench_decode(args, synth.DECODE_WORKLOADS[args.workload])
        return
    w = synth.WORKLOADS.get(args.workload) or synth.EXTRA_WORKLOADS.get(args.workload) \
        or {s.name: s for s in synth.SWEEP}[args.workload]
    print(f"[bench] generating {w.name} inputs", file=sys.stderr, flush=True)
    inp = synth.make_inputs(w, gate_logits=args.gate_logits)
    cpu = None
    if not args.no_cpu_baseline:  # before the GPU is touched: the pool's workers are forked
        print("[bench] timing the oracle on the CPU", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, synth.make_inputs(w) if args.gate_logits else inp)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    runner = Runner(w, inp, residual=args.residual, gate_logits=args.gate_logits, qk_norm=args.qk_norm)
    del inp
    # A plain device copy of known size: its HBM counters calibrate the kernels' counters.
    src = torch.empty(COPY_CAL_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    copy_gbs = measured_copy_gbs()
    # Per-kernel launch durations (and the roofline) come from a traced pass with the backward's
    # pipelines off, where no launch overlaps another; the headline step time from an untraced
    # pass with them on (GDR_PIPELINE=1: side streams overlap the reverse scans with the chunk
    # gradients of finished sequences or parts), unless --single-stream.
    pipe = "0" if args.single_stream else "1"
    print("[bench] timing kernels (single stream, traced)", file=sys.stderr, flush=True)
    os.environ["GDR_PIPELINE"] = "0"
    ms_single, per_kernel = timed(runner, args.steps, args.warmup)
    os.environ["GDR_PIPELINE"] = pipe
    print(f"[bench] timing (GDR_PIPELINE={pipe})", file=sys.stderr, flush=True)
    ms, _ = timed(runner, args.steps, args.warmup, trace=False)
    print("[bench] timing with the last-level cache flushed between steps", file=sys.stderr, flush=True)
    ms_flushed = timed_flushed(runner, max(5, args.steps // 2))
    tokens = w.B * w.T
    value = tokens / (ms / 1e3)
    # dominant kernel: largest total time over the timed steps
    tot = {k: sum(v) for k, v in per_kernel.items()}
    dom = max(tot, key=tot.get)
    launches = len(per_kernel[dom])
    avg_ms = tot[dom] / launches
    head_tokens = tokens * w.H
    cu = w.cu_seqlens or tuple(range(0, w.B * w.T + 1, w.T))
    chunks = sum((b - a + 63) // 64 for a, b in zip(cu[:-1], cu[1:]))
    units = chunks * w.H  # each launch of any kernel covers every (chunk, head) unit once
    esz = 2 if w.dtype == "bf16" else 4
    memories = w.n_states * w.H
    algo = (kernel_operator_bytes(w.variant, dom, w.dk, esz, w.has_beta, args.residual) * head_tokens
            + kernel_state_bytes(dom, w.dk, w.h0_std > 0) * memories)
    io = kernel_bytes_per_unit(w.variant, dom, w.dk, esz, w.has_beta, args.residual) * units
    achieved = algo / (avg_ms / 1e3) / 1e9
    io_gbs = io / (avg_ms / 1e3) / 1e9
    # counters are recorded for the plain workload only (other kernel instances run with these switches)
    traffic = None if (args.residual or args.gate_logits or args.qk_norm) else measured_traffic(dom, w.name)
    path_bytes = path_bytes_per_head_token(w.variant, w.dk, esz, w.has_beta, args.residual) * head_tokens
    path_gbs = path_bytes / (ms / 1e3) / 1e9
    out = {
        "metric": "tokens/s chunked gated-delta-rule fwd+bwd, H=16 d=128, T=4k-32k; % of roofline",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "ms_per_step_flushed": round(ms_flushed, 4),
        "ms_per_step_single_stream": round(ms_single, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic (seeded; distributions of the workload definition)",
        "config": {"workload": w.name, "variant": w.variant, "B": w.B, "H": w.H, "T": w.T, "d_k": w.dk,
                   "d_v": w.dv, "chunk": w.chunk, "cu_seqlens": list(w.cu_seqlens) if w.cu_seqlens else None,
                   "initial_state": w.h0_std > 0, "residual_output": args.residual,
                   "gate_logits": args.gate_logits, "qk_norm": args.qk_norm,
                   "backward_pipelines": not args.single_stream},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "avg_launch_ms": round(avg_ms, 4), "launches": launches,
                     "timed_in": "single-stream traced pass",
                     "algorithmic_bytes_per_launch": algo,
                     "io_bytes": io, "io_achieved": round(io_gbs, 1), "io_frac": round(io_gbs / HBM_PEAK_GBS, 4),
                     "measured_copy_GBps": round(copy_gbs, 1), "frac_of_measured_copy": round(achieved / copy_gbs, 4)},
        "path_roofline": {"bound": "hbm", "algorithmic_bytes_per_step": path_bytes, "achieved": round(path_gbs, 1),
                          "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(path_gbs / HBM_PEAK_GBS, 4)},
        "kernels_ms_per_step": {k: round(v / traced_steps(args.steps), 4) for k, v in tot.items()},
        "device": device_info(),
    }
    del runner
    torch.cuda.empty_cache()
    if not args.no_sweep and not (args.residual or args.gate_logits or args.qk_norm):
        sw = {}
        for sp in synth.SWEEP:
            print(f"[bench] sweep {sp.name}", file=sys.stderr, flush=True)
            r = Runner(sp, synth.make_inputs(sp))
            m, _ = timed(r, max(5, args.steps // 2), 2, trace=False)
            sw[sp.name] = {"ms_per_step": round(m, 4), "tokens_per_s": round(sp.B * sp.T / (m / 1e3), 1)}
            del r
            torch.cuda.empty_cache()
        out["sweep"] = sw
        names = [sp.name for sp in synth.SWEEP]
        out["sweep_ratio_T32k_over_T4k"] = round(sw[names[-1]]["ms_per_step"] / sw[names[0]]["ms_per_step"], 3)
        out["sweep_context"] = "pages: ~1.1x for a whole pure Gated DeltaNet training iteration, 4k -> 32k, hardware unstated"
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out))


if __name__ == "__main__":
    main()
