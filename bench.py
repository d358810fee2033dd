"""Benchmark of the fused SP-region forward + backward on one MI355X.

One step = forward (g* slab sum, bias, dropout, residual, LayerNorm) and
backward (dx, dgamma, dbeta) of the region on one rank's shard.  Default
workload: the 70B-shaped shard of hpc.payai.win lesson 7's worked example
(s = 16384, b = 1, h = 8192, t = 8 -> 2048 local tokens, bf16, p = 0.1).
Inputs are synthetic (seeded) and resident in HBM before timing starts;
several input/output sets rotate so that consecutive steps do not hit the
256 MB Infinity Cache.

Prints ONE JSON line on stdout; diagnostics go to stderr.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--sets R] [--no-extras]
  python bench.py --summarize-rocprof DIR   # rocprofv3 output -> text summary
  python bench.py --traffic FETCH_DIR WRITE_DIR   # --pmc runs -> HBM bytes per launch
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published peak
METRIC = "SP-region fwd+bwd tokens/s and achieved HBM GB/s (% of peak), h=8192 shard"
FWD_KERNEL_SOURCES = ["layernorm_sp_region_amd/csrc/fwd.hip", "layernorm_sp_region_amd/csrc/spr_device.h"]
TRAFFIC_FILE = "profiles/traffic_sp_region_fwd_kernel_shard70b.txt"


def eprint(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# Algorithmic bytes: every input read once, every output written once.
# ---------------------------------------------------------------------------
def fwd_bytes(w, T):
    E, h = w.elem_bytes, w.h
    params = sum([w.has_bias, True, w.has_beta]) * h * E
    stats = T * 4 * (2 if w.norm == "layernorm" else 1)
    return w.t * T * h * E + (T * h * E if w.has_residual else 0) + params + 2 * T * h * E + stats


def bwd_bytes(w, T):
    E, h = w.elem_bytes, w.h
    nstat = 2 if w.norm == "layernorm" else 1
    return 3 * T * h * E + T * 4 * nstat + h * E + h * 4 * nstat


def bwd_dropout_bytes(w, T):
    """The backward through the dropout: bwd_bytes plus dpartial written
    (T*h) and dbias written (h float32)."""
    return bwd_bytes(w, T) + T * w.h * w.elem_bytes + w.h * 4


def code_text(src: str) -> str:
    """C++ source without comments and with whitespace collapsed: what the
    compiler sees (the kernel sources hold no string literals with // or /*)."""
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def kernel_source_hash(read=None):
    """Hash of the forward kernel's code (comments and layout ignored), the
    key under which the committed traffic counters are valid."""
    h = hashlib.sha256()
    for p in FWD_KERNEL_SOURCES:
        if read is None:
            with open(os.path.join(ROOT, p), encoding="utf-8") as f:
                text = f.read()
        else:
            text = read(p)
        h.update(code_text(text).encode())
    return h.hexdigest()[:16]


def read_traffic():
    """HBM bytes per forward launch from the committed counter summary, or None
    when missing or taken on a different kernel source."""
    path = os.path.join(ROOT, TRAFFIC_FILE)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.strip().split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256") != kernel_source_hash():
        return None
    try:
        return int(float(kv["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


# ---------------------------------------------------------------------------
# CPU baseline: the oracle, as it is, on a bounded sample of the workload.
# ---------------------------------------------------------------------------
def plan_timing(W, n=1024, t=8, reps=200):
    """Host-side batch planning (library, then the oracle beside it) on a
    seeded batch of n sequences with the ragged workload's length mix
    (lognormal, mean 4096, CV 0.18): buckets at CV 0.15, the SP gate of each
    bucket and its padded shard layout."""
    import numpy as np
    import layernorm_sp_region_amd as spr
    import oracle.batching as OB
    w = W.BY_NAME["ragged13b"]
    rng = np.random.default_rng(w.input_seed + 7)
    lens = [int(v) for v in np.maximum(1, np.rint(4096 * rng.lognormal(-0.016, 0.1786, n)))]

    def run(bucket, gate, layout):
        order, starts = bucket(lens)
        nsp = 0
        for a, b in zip(starts, starts[1:]):
            bk = [lens[i] for i in order[a:b]]
            if gate(bk, 0.0):
                layout(bk, t)
                nsp += 1
        return len(starts) - 1, nsp

    nb, nsp = run(spr.bucket_by_tokens, spr.sp_gate, spr.shard_layout)
    assert (nb, nsp) == run(OB.bucket_by_tokens, OB.sp_gate, OB.shard_layout)
    t0 = time.perf_counter()
    for _ in range(reps):
        run(spr.bucket_by_tokens, spr.sp_gate, spr.shard_layout)
    lib_us = (time.perf_counter() - t0) / reps * 1e6
    t0 = time.perf_counter()
    for _ in range(max(1, reps // 20)):
        run(OB.bucket_by_tokens, OB.sp_gate, OB.shard_layout)
    oracle_us = (time.perf_counter() - t0) / max(1, reps // 20) * 1e6
    return {"sequences": n, "t": t, "buckets": nb, "sp_buckets": nsp, "us_per_batch": lib_us,
            "oracle_us_per_batch": oracle_us}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, inp, budget_s=12.0, chunk=64):
    import numpy as np
    import oracle.region as ref
    T = inp["T"]
    done, t0 = 0, time.perf_counter()
    start = 0
    while time.perf_counter() - t0 < budget_s:
        rows = np.arange(start, min(T, start + chunk))
        o = ref.region_forward(inp["partials"], t=w.t, rank=0, dtype=w.dtype, norm=w.norm, eps=w.eps,
                               p_drop=w.p_drop, seed=inp["seed"], gamma=inp["gamma"], beta=inp["beta"],
                               bias=inp["bias"], residual=inp["residual"], cu_seqlens=inp["cu_seqlens"], rows=rows)
        ref.region_backward(inp["dy"][rows], o["z"], inp["gamma"], dtype=w.dtype, norm=w.norm, eps=w.eps)
        done += len(rows)
        start = (start + chunk) % T
    el = time.perf_counter() - t0
    return dict(value=done / el, unit="tokens/s", cores=1, kind="oracle", cpu=cpu_model(),
                gbs=done / el * (fwd_bytes(w, T) + bwd_bytes(w, T)) / T / 1e9,
                sample=f"{done} rows of the {T}-row shard, cycled in chunks of {chunk} (forward + backward, "
                       f"{el:.1f} s, single process: numpy element-wise ops on one core)")


def _cpu_worker(args):
    """One process of the token-partitioned oracle baseline: rows [r0, r1) of
    the shard, cycled in chunks, for budget_s seconds.  Returns (rows, s)."""
    name, r0, r1, budget_s, chunk = args
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    import numpy as np
    import oracle.region as ref
    import workloads as W
    w = W.BY_NAME[name]
    inp = W.make_inputs(w)
    done, start, t0 = 0, r0, time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        rows = np.arange(start, min(r1, start + chunk))
        o = ref.region_forward(inp["partials"], t=w.t, rank=0, dtype=w.dtype, norm=w.norm, eps=w.eps,
                               p_drop=w.p_drop, seed=inp["seed"], gamma=inp["gamma"], beta=inp["beta"],
                               bias=inp["bias"], residual=inp["residual"], cu_seqlens=inp["cu_seqlens"], rows=rows)
        ref.region_backward(inp["dy"][rows], o["z"], inp["gamma"], dtype=w.dtype, norm=w.norm, eps=w.eps)
        done += len(rows)
        start = start + chunk if start + chunk < r1 else r0
    return done, time.perf_counter() - t0


def cpu_baseline_parallel(w, T, budget_s=12.0, chunk=64, max_procs=16):
    """The same oracle, token-partitioned over one process per host core (at
    most 16): rows are independent, so process k takes the k-th contiguous
    share of the shard.  Processes are spawned (a fresh interpreter each),
    never forked from this GPU-using process.  Throughput = all rows done /
    the longest process's time.  The parameter-gradient sums are not combined
    across processes (a fixed-order sum of a few [h] vectors)."""
    import multiprocessing as mp
    n = max(1, min(max_procs, len(os.sched_getaffinity(0)), T))
    shares = [(w.name, k * T // n, (k + 1) * T // n, budget_s, chunk) for k in range(n)]
    pool = mp.get_context("spawn").Pool(n)
    try:
        res = pool.map(_cpu_worker, shares)
        pool.close()          # no more work: the workers exit on their own
    finally:
        pool.terminate()      # no-op after close(); ends them on an exception
        pool.join()           # every worker (and the pool's threads) gone before returning
    done = sum(r[0] for r in res)
    el = max(r[1] for r in res)
    return dict(value=done / el, unit="tokens/s", cores=n, kind="oracle", cpu=cpu_model(),
                gbs=done / el * (fwd_bytes(w, T) + bwd_bytes(w, T)) / T / 1e9,
                sample=f"{done} rows of the {T}-row shard over {n} spawned processes, each cycling its own "
                       f"contiguous share in chunks of {chunk} (forward + backward, {el:.1f} s)")


# ---------------------------------------------------------------------------
# The other workloads of the configuration list, each measured like the
# headline one (rotating sets, wall-clock steps, event-stamped kernel times)
# plus a HIP-graph replay of the same steps (the small shards' wall clock is
# bound by the host's per-call work, the replay by the GPU's).
# ---------------------------------------------------------------------------
CONFIGS = [("c1", "tiny"), ("c2", "page_demo"), ("c4", "ragged13b"), ("c5", "long128k")]


def device_inputs(w, dev):
    """Seeded inputs of a shard too large to draw on the host in a short run:
    slabs, residual and dy drawn on the device (workloads.device_normal), the
    [h] parameters from the host generator."""
    import numpy as np
    import workloads as W
    T = w.b * w.s // w.t
    dt = None if w.dtype == "bf16" else __import__("torch").float32
    rng = np.random.default_rng(w.input_seed)
    par = lambda x: W.as_torch(W._to_storage(x, w.dtype), dev)
    return dict(b=w.b, s=w.s, T=T, cu_seqlens=None, seed=w.dropout_seed,
                partials=W.device_normal((w.t, T, w.h), seed=101, device=dev, scale=w.slab_scale, dtype=dt),
                residual=W.device_normal((1, T, w.h), seed=102, device=dev, dtype=dt)[0] if w.has_residual else None,
                dy=W.device_normal((1, T, w.h), seed=103, device=dev, dtype=dt)[0],
                bias=par(0.02 * rng.standard_normal(w.h)) if w.has_bias else None,
                gamma=par(rng.uniform(0.5, 1.5, size=w.h)),
                beta=par(0.1 * rng.standard_normal(w.h)) if w.has_beta else None)


def cpu_full(w, inp, chunk=64, label=None):
    """The oracle over every row of a shard once, one process."""
    import numpy as np
    import oracle.region as ref
    T = inp["T"]
    t0 = time.perf_counter()
    for start in range(0, T, chunk):
        rows = np.arange(start, min(T, start + chunk))
        o = ref.region_forward(inp["partials"], t=w.t, rank=0, dtype=w.dtype, norm=w.norm, eps=w.eps,
                               p_drop=w.p_drop, seed=inp["seed"], gamma=inp["gamma"], beta=inp["beta"],
                               bias=inp["bias"], residual=inp["residual"], cu_seqlens=inp["cu_seqlens"], rows=rows)
        ref.region_backward(inp["dy"][rows], o["z"], inp["gamma"], dtype=w.dtype, norm=w.norm, eps=w.eps)
    el = time.perf_counter() - t0
    return dict(value=T / el, unit="tokens/s", cores=1, kind="oracle", cpu=cpu_model(),
                gbs=(fwd_bytes(w, T) + bwd_bytes(w, T)) / el / 1e9,
                sample=label or f"all {T} rows of the shard once, in chunks of {chunk} ({el:.2f} s, single process)")


def measure_config(w, inp, dev, steps, warmup, nsets):
    """fwd + bwd steps of one workload whose tensors are on the device."""
    import numpy as np
    import torch
    import layernorm_sp_region_amd as spr
    T, h = inp["T"], w.h
    to = lambda a: a if a is None or isinstance(a, torch.Tensor) else W_as_torch(a, dev)
    gamma, beta, bias = to(inp["gamma"]), to(inp["beta"]), to(inp["bias"])
    dt = gamma.dtype
    ln = w.norm == "layernorm"
    cu = torch.tensor(inp["cu_seqlens"], dtype=torch.int32, device=dev) if inp["cu_seqlens"] is not None else None
    base = dict(P=to(inp["partials"]), res=to(inp["residual"]), dy=to(inp["dy"]))
    sets = []
    for i in range(nsets):
        s = {k: (v if i == 0 or v is None else v.clone()) for k, v in base.items()}
        P = spr.empty_partials(w.t, T, h, dt, dev)
        P.copy_(s["P"])
        s["P"] = P
        s["fo"] = spr.FwdOut(torch.empty((T, h), dtype=dt, device=dev), torch.empty((T, h), dtype=dt, device=dev),
                             torch.empty(T, device=dev) if ln else None, torch.empty(T, device=dev), None)
        s["bo"] = spr.BwdOut(torch.empty((T, h), dtype=dt, device=dev), torch.empty(h, device=dev),
                             torch.empty(h, device=dev) if ln else None)
        sets.append(s)
    del base
    ws = torch.empty(max(16, spr.workspace_bytes(T, h)), dtype=torch.uint8, device=dev)

    def step(i, ev=None):
        s = sets[i % nsets]
        if ev is not None:
            spr.time_next_call(ev[0], ev[1])
        fo = spr.fwd(s["P"], gamma, beta, bias=bias, residual=s["res"], b=inp["b"], s=inp["s"], t=w.t, rank=0,
                     eps=w.eps, p_drop=w.p_drop, seed=inp["seed"], norm=w.norm, cu_seqlens=cu, out=s["fo"])
        if ev is not None:
            spr.time_next_call(ev[2], ev[3])
        spr.bwd(s["dy"], fo.z, fo.mean, fo.rstd, gamma, b=inp["b"], s=inp["s"], t=w.t, norm=w.norm,
                workspace=ws, out=s["bo"])

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    wall_us = (time.perf_counter() - t0) / steps * 1e6
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for e in evs:
        for x in e:
            x.record()
    torch.cuda.synchronize()
    for i in range(steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    fwd_us = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]) * 1e3)
    bwd_us = float(np.mean([e[2].elapsed_time(e[3]) for e in evs]) * 1e3)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(nsets):
            step(i)
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(graph):
        for i in range(nsets):
            step(i)
    graph.replay()
    torch.cuda.synchronize()
    reps = max(1, steps // nsets)
    t2 = time.perf_counter()
    for _ in range(reps):
        graph.replay()
    torch.cuda.synchronize()
    graph_us = (time.perf_counter() - t2) / (reps * nsets) * 1e6
    del graph, sets, ws
    fb, bb = fwd_bytes(w, T), bwd_bytes(w, T)
    return {"workload": w.name, "local_tokens": T, "h": h, "dtype": w.dtype, "norm": w.norm, "steps": steps,
            "rotating_sets": nsets, "step_us_wall": wall_us, "step_us_graph_replay": graph_us,
            "fwd_us": fwd_us, "bwd_us": bwd_us,
            "tokens_per_s_wall": T / (wall_us * 1e-6), "tokens_per_s_graph_replay": T / (graph_us * 1e-6),
            "tokens_per_s_kernels": T / ((fwd_us + bwd_us) * 1e-6),
            "fwd_bwd_pct_of_peak": 100 * (fb + bb) / ((fwd_us + bwd_us) * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "fwd_frac": fb / (fwd_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "bwd_gbs": bb / (bwd_us * 1e-6) / 1e9,
            "algorithmic_bytes": {"fwd": fb, "bwd": bb}}


def W_as_torch(a, dev):
    import workloads as W
    return W.as_torch(a, dev)


def run_configs(args, dev):
    import torch
    import workloads as W
    out = {}
    for tag, name in CONFIGS:
        w = W.BY_NAME[name]
        t_gen = time.time()
        big = name == "long128k"
        inp = device_inputs(w, dev) if big else W.make_inputs(w)
        steps = max(10, args.steps // 5) if big else args.steps
        rec = measure_config(w, inp, dev, steps, max(2, args.warmup // 2), 1 if big else args.sets)
        rec["inputs"] = ("seeded on-device draws (workloads.device_normal), [h] parameters from the host generator"
                         if big else "workloads.make_inputs (host, seeded)")
        if not args.no_cpu_baseline:
            if big:
                sub = W.custom(f"{name}_first2048rows", h=w.h, t=w.t, s=w.t * 2048, p_drop=w.p_drop, bias=w.has_bias,
                               residual=w.has_residual, beta=w.has_beta)
                sinp = W.make_inputs(sub)
                rec["cpu_baseline"] = cpu_full(sub, sinp, label=f"a 2048-row sub-shard of the {inp['T']}-row shard "
                                                                 f"(same h, t, p, norm), every row once, single process")
                del sinp
            elif name != "ragged13b":
                rec["cpu_baseline"] = cpu_full(w, inp)
        eprint(f"[bench] {tag} {name}: T={rec['local_tokens']} step {rec['step_us_wall']:.1f} us wall, "
               f"{rec['step_us_graph_replay']:.1f} us graph replay; fwd {rec['fwd_us']:.1f} us "
               f"(frac {rec['fwd_frac']:.3f}), bwd {rec['bwd_us']:.1f} us; {rec['fwd_bwd_pct_of_peak']:.1f}% of peak "
               f"(inputs {time.time() - t_gen:.1f}s)")
        out[tag] = rec
        del inp
        torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------------------
def run(args):
    import numpy as np
    import torch
    import layernorm_sp_region_amd as spr
    import workloads as W

    spr.load_library()
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU (the region has no CPU path)")
    dev = torch.device("cuda:0")
    w = W.BY_NAME[args.workload]
    t_gen = time.time()
    inp = W.make_inputs(w)
    T, h = inp["T"], w.h
    eprint(f"[bench] {w.name}: T={T} h={h} t={w.t} dtype={w.dtype} (inputs {time.time() - t_gen:.1f}s)")
    tt = lambda a: W.as_torch(a, dev)

    gamma, beta, bias = tt(inp["gamma"]), tt(inp["beta"]), tt(inp["bias"])
    dt = gamma.dtype
    sets = []
    base = dict(P=tt(inp["partials"]), res=tt(inp["residual"]), dy=tt(inp["dy"]))
    # Slab layout: the library's recommended stride (the receive-buffer layout
    # a caller controls) unless --slabs contiguous (stride T*h).
    stride = spr.partials_stride(T, h, dt) if args.slabs == "recommended" and T * h > 0 else T * h
    for i in range(args.sets):
        s = {k: (v if i == 0 or v is None else v.clone()) for k, v in base.items()}
        if args.slabs == "recommended":
            P = spr.empty_partials(w.t, T, h, dt, dev)
            P.copy_(s["P"])
            s["P"] = P
        ln = w.norm == "layernorm"
        s["fo"] = spr.FwdOut(torch.empty((T, h), dtype=dt, device=dev), torch.empty((T, h), dtype=dt, device=dev),
                             torch.empty(T, device=dev) if ln else None, torch.empty(T, device=dev), None)
        s["bo"] = spr.BwdOut(torch.empty((T, h), dtype=dt, device=dev), torch.empty(h, device=dev),
                             torch.empty(h, device=dev) if ln else None)
        sets.append(s)
    ws = torch.empty(max(16, spr.workspace_bytes(T, h)), dtype=torch.uint8, device=dev)
    cu = torch.tensor(inp["cu_seqlens"], dtype=torch.int32, device=dev) if inp["cu_seqlens"] is not None else None

    def step(i, ev=None, p_drop=w.p_drop, rotate=True):
        # ev: four events; each region call stamps its first kernel's start and
        # last kernel's end into a pair of them from the dispatch packets.
        s = sets[i % len(sets)] if rotate else sets[0]
        if ev is not None:
            spr.time_next_call(ev[0], ev[1])
        fo = spr.fwd(s["P"], gamma, beta, bias=bias, residual=s["res"], b=inp["b"], s=inp["s"], t=w.t, rank=0,
                     eps=w.eps, p_drop=p_drop, seed=inp["seed"], norm=w.norm, cu_seqlens=cu, out=s["fo"])
        if ev is not None:
            spr.time_next_call(ev[2], ev[3])
        spr.bwd(s["dy"], fo.z, fo.mean, fo.rstd, gamma, b=inp["b"], s=inp["s"], t=w.t, norm=w.norm,
                workspace=ws, out=s["bo"])

    # Copy-kernel ceiling on 1 GiB (also the reference for the traffic counters).
    nb = 1 << 30
    src = torch.empty(nb, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    src.fill_(1)
    for _ in range(2):
        spr.hbm_copy(src, dst)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 5
    e0.record()
    for _ in range(reps):
        spr.hbm_copy(src, dst)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * nb * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    eprint(f"[bench] copy ceiling {copy_gbs:.0f} GB/s ({100 * copy_gbs / HBM_PEAK_GBS:.1f}% of {HBM_PEAK_GBS:.0f})")

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # Timed region: exactly K steps, nothing else on the stream.  (Kernel
    # durations come from the second, otherwise identical, pass below.)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    # Kernel durations: the same K steps, every region call stamping HIP
    # events from its kernels' own dispatch packets (sp_region_time_next_call:
    # no marker packets, which cost the GPU ~3 us each, on the stream the
    # library launches on).  Each event is recorded once first so it exists.
    def timestamped_steps(**kw):
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
        for e in evs:
            for x in e:
                x.record()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for i in range(args.steps):
            step(i, evs[i], **kw)
        torch.cuda.synchronize()
        elapsed_ev = time.perf_counter() - t1
        fwd_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
        bwd_ms = np.array([e[2].elapsed_time(e[3]) for e in evs])
        return fwd_ms, bwd_ms, elapsed_ev

    fwd_ms, bwd_ms, elapsed_ev = timestamped_steps()

    def call_us(call, n):
        """Durations (us) of n region calls, each stamping a pair of HIP events
        from its own kernels' dispatch packets."""
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n)]
        for e in ev:
            for x in e:
                x.record()
        for i in range(n):
            spr.time_next_call(ev[i][0], ev[i][1])
            call(i)
        torch.cuda.synchronize()
        return np.array([a.elapsed_time(b) for a, b in ev]) * 1e3

    # The backward through the dropout and the slab sum (dpartial, dbias), on
    # the same forward outputs.
    ws_d = torch.empty(max(16, spr.dropout_workspace_bytes(T, h)), dtype=torch.uint8, device=dev)
    douts = []
    for s in sets:
        bo = s["bo"]
        douts.append(spr.BwdDropoutOut(bo.dx, torch.empty_like(bo.dx), bo.dgamma, bo.dbeta,
                                       torch.empty(h, device=dev) if w.has_bias else None))

    def bwd_dropout_call(i):
        s, fo = sets[i % len(sets)], sets[i % len(sets)]["fo"]
        spr.bwd_dropout(s["dy"], fo.z, fo.mean, fo.rstd, gamma, b=inp["b"], s=inp["s"], t=w.t, rank=0,
                        p_drop=w.p_drop, seed=inp["seed"], norm=w.norm, cu_seqlens=cu, workspace=ws_d,
                        want_dbias=w.has_bias, out=douts[i % len(sets)])

    bwd_dropout_us = float(np.mean(call_us(bwd_dropout_call, args.steps)))
    del douts, ws_d

    # The same steps with p = 0 (the forward's time prices the hash), and warm
    # steps: one buffer set reused by every step, so whatever the Infinity
    # Cache kept from the previous step is read from there.  Both run whole
    # steps, since a forward's time depends on what the kernel before it left
    # dirty in the caches.
    extras = None
    if not args.no_extras:
        f0, b0, _ = timestamped_steps(p_drop=0.0)
        fw, bw, _ = timestamped_steps(rotate=False)
        # The rotation of steps captured once in a HIP graph and replayed: the
        # same kernels with no per-launch host work.
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(len(sets)):
                step(i)
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(len(sets)):
                step(i)
        graph.replay()
        torch.cuda.synchronize()
        reps = max(1, args.steps // len(sets))
        t2 = time.perf_counter()
        for _ in range(reps):
            graph.replay()
        torch.cuda.synchronize()
        graph_step_us = (time.perf_counter() - t2) / (reps * len(sets)) * 1e6
        del graph
        extras = {"p0_step_us": {"fwd": float(f0.mean() * 1e3), "bwd": float(b0.mean() * 1e3)},
                  "warm_one_set_step_us": {"fwd": float(fw.mean() * 1e3), "bwd": float(bw.mean() * 1e3)},
                  "graph_replay_step_us": graph_step_us}

    fb, bb = fwd_bytes(w, T), bwd_bytes(w, T)
    fwd_s = float(fwd_ms.mean()) * 1e-3
    achieved = fb / fwd_s / 1e9
    step_ms = elapsed / args.steps * 1e3
    eprint(f"[bench] fwd {fwd_ms.mean() * 1e3:.1f} us (p50 {np.median(fwd_ms) * 1e3:.1f}), "
           f"bwd {bwd_ms.mean() * 1e3:.1f} us, step {step_ms * 1e3:.1f} us wall "
           f"({elapsed_ev / args.steps * 1e6:.1f} in the timestamped pass); fwd {achieved:.0f} GB/s, "
           f"fwd+bwd {(fb + bb) / ((fwd_ms.mean() + bwd_ms.mean()) * 1e-3) / 1e9:.0f} GB/s")

    plan = plan_timing(W)
    traffic = read_traffic()
    del sets, ws
    torch.cuda.empty_cache()
    configs = None if args.no_configs else run_configs(args, dev)
    cpu = None if args.no_cpu_baseline else cpu_baseline(w, inp)
    cpu_par = None if args.no_cpu_baseline else cpu_baseline_parallel(w, T)
    kernel_us = (fwd_ms.mean() + bwd_ms.mean()) * 1e3
    rec = {
        "metric": METRIC,
        "value": T * args.steps / elapsed,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1)/sqrt(8) partial slabs, N(0,1) residual and dy, shaped like the pages' workloads)",
        "config": {"workload": w.name, "s": inp["s"], "b": inp["b"], "h": h, "t": w.t, "local_tokens": T,
                   "p_drop": w.p_drop, "norm": w.norm, "rank": 0, "rotating_sets": args.sets,
                   "slabs": args.slabs, "slab_stride": stride},
        "step_us_timestamped_pass": elapsed_ev / args.steps * 1e6,
        "fwd_us": float(fwd_ms.mean() * 1e3),
        "bwd_us": float(bwd_ms.mean() * 1e3),
        "fwd_us_p50_p95": [float(np.median(fwd_ms) * 1e3), float(np.percentile(fwd_ms, 95) * 1e3)],
        "bwd_us_p50_p95": [float(np.median(bwd_ms) * 1e3), float(np.percentile(bwd_ms, 95) * 1e3)],
        "extras": extras,
        "workspace_bytes": {"bwd": spr.workspace_bytes(T, h), "bwd_dropout": spr.dropout_workspace_bytes(T, h)},
        "fwd_bwd_hbm_gbs": (fb + bb) / (kernel_us * 1e-6) / 1e9,
        "fwd_bwd_pct_of_peak": 100 * (fb + bb) / (kernel_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
        "algorithmic_bytes": {"fwd": fb, "bwd": bb, "bwd_dropout": bwd_dropout_bytes(w, T)},
        "bwd_dropout_us": bwd_dropout_us,
        "bwd_dropout_hbm_gbs": bwd_dropout_bytes(w, T) / (bwd_dropout_us * 1e-6) / 1e9,
        "copy_ceiling_gbs": copy_gbs,
        "roofline": {"kernel": "sp_region_fwd_kernel", "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": traffic},
        "cpu_baseline": cpu,
        "cpu_baseline_parallel": cpu_par,
        "host_planning": plan,
        "configs": configs,
    }
    print(json.dumps(rec), flush=True)


# ---------------------------------------------------------------------------
# rocprofv3 output -> short text summary (kernel stats or counters).
# ---------------------------------------------------------------------------
def summarize_rocprof(d):
    out = []
    stats = sorted(glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True))
    for p in stats:
        out.append(f"# kernel stats: {os.path.relpath(p, d)}")
        with open(p) as f:
            rows = list(csv.DictReader(f))
        for r in rows:
            name = r.get("Name", "")[:90]
            out.append(f"{name:90s} calls={r.get('Calls')} avg_ns={float(r.get('AverageNs', 0)):.0f} "
                       f"min_ns={float(r.get('MinNs', 0)):.0f} max_ns={float(r.get('MaxNs', 0)):.0f} "
                       f"pct={float(r.get('Percentage', 0)):.2f}")
    counters = sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True))
    for p in counters:
        out.append(f"# counters: {os.path.relpath(p, d)}")
        agg = {}
        with open(p) as f:
            for r in csv.DictReader(f):
                key = (r.get("Kernel_Name", "")[:90], r.get("Counter_Name"))
                agg.setdefault(key, []).append(float(r.get("Counter_Value", 0)))
        for (k, c), vals in sorted(agg.items()):
            out.append(f"{k:90s} {c}: dispatches={len(vals)} mean_per_dispatch={sum(vals) / len(vals):.1f}")
    print("\n".join(out))


def _counter_means(d):
    """{kernel-name prefix: mean counter value per dispatch} from a --pmc run."""
    out = {}
    for p in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        acc = {}
        with open(p) as f:
            for r in csv.DictReader(f):
                acc.setdefault(r.get("Kernel_Name", ""), []).append(float(r.get("Counter_Value", 0)))
        for k, v in acc.items():
            out[k] = sum(v) / len(v)
    return out


def traffic_summary(fetch_dir, write_dir, copy_bytes=1 << 30):
    """HBM traffic per launch of each region kernel from a FETCH_SIZE run and a
    WRITE_SIZE run (KiB per dispatch), each scaled by what the same counter
    reads for the calibration copy of known size."""
    fe, wr = _counter_means(fetch_dir), _counter_means(write_dir)
    pick = lambda m, key: next(v for k, v in m.items() if key in k)
    f_scale = (copy_bytes / 1024) / pick(fe, "sp_region_copy_kernel")
    w_scale = (copy_bytes / 1024) / pick(wr, "sp_region_copy_kernel")
    lines = [f"# FETCH_SIZE scale {f_scale:.4f}, WRITE_SIZE scale {w_scale:.4f} "
             f"(1 GiB calibration copy: counter KiB vs true KiB)"]
    fwd = None
    # One line per kernel instantiation (the rows kernel with and without the
    # dropout backward are different kernels), in the order of the path.
    order = ("sp_region_fwd_kernel", "sp_region_bwd_rows_kernel", "sp_region_bwd_cols_kernel",
             "sp_region_bwd_direct_kernel")
    names = sorted((k for k in fe if any(o in k for o in order) and k in wr),
                   key=lambda k: (next(i for i, o in enumerate(order) if o in k), k))
    for key in names:
        fb = fe[key] * f_scale * 1024
        wb = wr[key] * w_scale * 1024
        short = key.replace("spr::(anonymous namespace)::", "").replace("void ", "").split("(")[0]
        lines.append(f"{short}: fetch_bytes={fb:.0f} write_bytes={wb:.0f} total_bytes={fb + wb:.0f}")
        if "sp_region_fwd_kernel" in key and fwd is None:
            fwd = fb + wb
    lines.append(f"kernel_source_sha256={kernel_source_hash()}")
    lines.append(f"hbm_bytes_per_launch={fwd:.0f}")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="shard70b")
    ap.add_argument("--sets", type=int, default=4, help="rotating input/output sets (Infinity Cache defeat)")
    ap.add_argument("--slabs", choices=("recommended", "contiguous"), default="recommended",
                    help="partial-slab layout: sp_region_partials_stride, or back to back (stride T*h)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the p = 0 forward and the warm one-set passes (they launch the step's kernels "
                         "again, so a profiler's per-kernel averages would mix them in)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workloads (c1 tiny, c2 page_demo, c4 ragged13b, c5 long128k)")
    ap.add_argument("--summarize-rocprof", metavar="DIR")
    ap.add_argument("--traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    args = ap.parse_args()
    if args.summarize_rocprof:
        summarize_rocprof(args.summarize_rocprof)
        return
    if args.traffic:
        traffic_summary(*args.traffic)
        return
    if args.gpus != 1:
        eprint(f"bench.py measures one GPU's shard; --gpus {args.gpus} is not supported "
               "(the region runs on one MI355X: no collectives or multi-GPU launch are implemented)")
        sys.exit(2)
    run(args)


if __name__ == "__main__":
    main()
