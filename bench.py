"""Benchmark of the HySparse hybrid-block hot path on one MI355X.

Timed step: one HySparse hybrid block on the 80B-MoE-like 32k workload
(B=1, L=32768, 32 query heads, 4 KV heads, head dim 128, bf16; 1 full layer +
11 sparse layers; top-16 of 64-token blocks; window 128; 32 needle keys x4):
  full attention + block scores -> top-k -> 11 x (block-sparse attention,
  window attention + sigmoid gate).
Value: prefill tokens/s of that block (L / step time).  Also reported: the
HySparse2 1M-token decode step (B=4, fp8 MQA cache, top-1024 + recent 128,
11 sparse layers) in microseconds per step, per-kernel times from HIP events
on the launch stream, the roofline of the dominant kernel, and the CPU oracle
timed on a bounded sample of the same workload.

The HySparse2 KV Bridging projection (64k tokens, d_model 4096, fp8 MQA
cache) and the HySparse block-level decode step (B=4, 128k-token bf16 GQA
cache, top-16 blocks, 11 sparse layers with ring window caches) are timed
beside them with their own rooflines.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-decode] [--no-bridge]
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
from hybrid_sparse_attention_flash_amd import ops  # noqa: E402
from hybrid_sparse_attention_flash_amd.block import (HySparse2Block, HySparse2Decode, HySparseBlock,  # noqa: E402
                                                     HySparseTrainer)

METRIC = ("hybrid-block prefill tokens/s at 32k (TFLOP/s, GB/s % peak); decode us/token at 1M")

# HBM traffic of the dominant kernel (the one-pass sparse layer), measured
# with rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE (one counter per pass) over
#   python3 bench.py --no-decode --no-bridge --no-hs-decode --no-bwd --no-cpu --no-peaks --calibrate-copy --steps 2 --warmup 1
# and scaled by the counters' reading for a plain 512 MiB copy in the same run
# (FETCH_SIZE x 2.000, WRITE_SIZE x 1.000; the profiles directory holds the
# summaries).  It is reported only while the kernel sources still hash to the
# value they had when the counters were taken.
TRAFFIC_SOURCES = ("sparse_layer.hip", "block_union.h", "common.h", "kernels.h")
TRAFFIC = {"sources_sha1": "1ad9e7ea641020f1db3c8cd14695a14ce84b82ab", "bytes_per_launch": 1.4688e9}
# The same two passes for the KV Bridging kernel, over
#   python3 bench.py --only-bridge --calibrate-copy --steps 1 --warmup 0
BRIDGE_TRAFFIC_SOURCES = ("bridge.hip", "common.h", "kernels.h")
BRIDGE_TRAFFIC = {"sources_sha1": "6d6eba6b5f5e733c97373c3b33f4b1f406e1e599", "bytes_per_launch": 575.8e6}
# The same two passes for the decode step (every kernel of one hys_decode_step
# call, summed per step), over
#   python3 bench.py --only-decode --no-peaks --calibrate-copy --steps 2 --warmup 1
DECODE_TRAFFIC_SOURCES = ("decode.hip", "decode_split.hip", "decode_split.h", "topk.hip", "common.h", "kernels.h", "abi.hip")
DECODE_TRAFFIC = {"sources_sha1": "66a5c7b9544150ee0b1db9e67897b352217c9420", "bytes_per_step": 1.2456e9}
# The same two passes for the HySparse decode step at 128k (every kernel of one
# hys_hysparse_decode_step call, summed per step), over
#   python3 bench.py --only-hs-decode --calibrate-copy --steps 2 --warmup 1 --no-cpu
HS_DECODE_TRAFFIC_SOURCES = ("hs_decode.hip", "decode.hip", "topk.hip", "common.h", "kernels.h", "abi.hip")
HS_DECODE_TRAFFIC = {"sources_sha1": "1f81ea66ecd6a09580262f823fc28ca4a4e94515", "bytes_per_step": 1.1398e9}
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# algorithmic work
# ---------------------------------------------------------------------------

def full_attention_flops(w):
    L = w.L
    return 4.0 * w.D * w.Hq * L * (L + 1) / 2 * w.B


def sparse_keys_per_query(idx, L, block):
    """Number of visible selected keys per query from the returned block ids."""
    i = torch.arange(L, device=idx.device, dtype=torch.int64).view(1, L, 1)
    c = idx.to(torch.int64)
    valid = c >= 0
    start = c * block
    n = torch.clamp(torch.minimum(i + 1 - start, torch.full_like(start, block)), min=0)
    return (n * valid).sum().item()


# ---------------------------------------------------------------------------
# timing helpers
# ---------------------------------------------------------------------------

class Timer:
    """Accumulates HIP-event intervals per stage on the current stream."""

    def __init__(self):
        self.events = {}

    def span(self, name):
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        self.events.setdefault(name, []).append((s, e))
        return s, e

    def totals_ms(self):
        torch.cuda.synchronize()
        return {k: sum(s.elapsed_time(e) for s, e in v) for k, v in self.events.items()}

    def counts(self):
        return {k: len(v) for k, v in self.events.items()}


def stats_ms(xs):
    xs = sorted(xs)
    n = len(xs)
    med = xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])
    return {"mean_ms": round(sum(xs) / n, 4), "median_ms": round(med, 4), "min_ms": round(xs[0], 4), "n": n}


class CacheFlush:
    """Writes a 512 MiB buffer, more than the L2s and the 256 MB MALL together,
    so the next step starts with its inputs in HBM only (cold-cache timing)."""

    def __init__(self, dev, mib=512):
        self.buf = torch.empty(mib * 2 ** 20 // 4, dtype=torch.float32, device=dev)

    def __call__(self):
        self.buf.fill_(1.0)


def per_step_times(step, steps, flush=None):
    """HIP events around each step on the launch stream; with `flush`, the
    flush runs before each step, outside the timed interval."""
    ev = []
    for _ in range(steps):
        if flush is not None:
            flush()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        step()
        b.record()
        ev.append((a, b))
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def clock_state():
    """The GPU's clock readings as the driver tool reports them (raw text).
    Skipped under rocprofv3: its library attaches every child process to the
    GPU before the tool (a Python script) can start."""
    import subprocess
    if os.environ.get("ROCPROF_OUTPUT_PATH"):
        return None
    for cmd in (["amd-smi", "metric", "--clock"], ["rocm-smi", "--showclocks"]):
        try:
            r = subprocess.run(cmd, capture_output=True, text=True, timeout=20)
        except Exception:
            continue
        if r.returncode == 0 and r.stdout.strip():
            lines = [ln.strip() for ln in r.stdout.splitlines() if ln.strip()]
            keep = [ln for ln in lines if any(t in ln.upper() for t in ("SCLK", "MCLK", "GFX", "MEM", "FCLK", "CLK"))]
            return {"tool": " ".join(cmd), "lines": (keep or lines)[:24]}
    return None


def measured_peaks(dev):
    """Measured denominators beside the datasheet ones: a large bf16 GEMM
    (hipBLASLt through torch) for MFMA, a device copy for HBM."""
    n = 8192
    a = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    b = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b)
    t = per_step_times(lambda: torch.matmul(a, b), 10)
    gemm = 2.0 * n ** 3 / (min(t) * 1e-3) / 1e12
    del a, b
    src = torch.empty(2 ** 30 // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    t = per_step_times(lambda: dst.copy_(src), 10)
    copy = 2.0 * 2 ** 30 / (min(t) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return {"bf16_gemm_tflops": round(gemm, 1), "hbm_copy_GBs": round(copy, 1),
            "how": "best of 10: torch.matmul 8192^3 bf16; 1 GiB device copy (read + write bytes)"}


def run_block(blk, inp, timer=None):
    def rec(name, fn):
        if timer is None:
            fn()
        else:
            s, e = timer.span(name)
            s.record()
            fn()
            e.record()
    q, k, v, kw, vw, gw = inp
    rec("full_attn+scores", lambda: blk.full(q[0], k, v))
    rec("select_topk", blk.select)
    for l in range(blk.n_sparse):
        # one pass per sparse layer: selected blocks of the shared KV, the
        # layer's own window, and the gate
        rec("sparse_layer", lambda: ops.hys_sparse_layer_fwd(q[l + 1], k, v, blk._idx(), kw[l], vw[l], blk.window,
                                                             gw[l], blk.o_layers[l], topk=blk.topk))


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample of the same workload
# ---------------------------------------------------------------------------

class _RowView:
    """Array stand-in that converts only the indexed query rows to float64."""

    def __init__(self, t):
        self.t = t
        self.shape = tuple(t.shape)

    def __getitem__(self, rows):
        return self.t[torch.as_tensor(np.asarray(rows))].to(torch.float64).numpy()


def host_cpu():
    """Cores this process may run on (capped at the 16 a GPU's share of the
    host provides) and the CPU model."""
    try:
        n = len(os.sched_getaffinity(0))
    except Exception:
        n = os.cpu_count() or 1
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except Exception:
        pass
    return min(n, 16), n, model


def cpu_baseline(w, host, nrows, seed=0):
    """The oracle as it stands, on a bounded sample of query rows of the same
    block, spread over the host's cores: the rows are independent, so worker
    threads each evaluate a contiguous share of them (numpy releases the GIL in
    its array loops), with BLAS held to one thread per worker."""
    import concurrent.futures as cf
    import oracle
    cores, allowed, model = host_cpu()
    q, k, v, kw, vw, gw = host
    f = lambda t: t[0].to(torch.float64).numpy()
    kf, vf = f(k), f(v)
    kwf = [f(x) for x in kw]
    vwf = [f(x) for x in vw]
    gwf = [x.numpy().astype(np.float64) for x in gw]
    qv = [_RowView(x[0]) for x in q]
    rows = np.linspace(0, w.L - 1, nrows).round().astype(np.int64)
    shares = [r for r in np.array_split(rows, cores) if len(r)]

    def one(r):
        return oracle.hysparse_block(qv, kf, vf, kwf, vwf, gwf, w.scale, w.block, w.topk, w.window, rows=r)
    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(1)
    except Exception:
        limit = None
    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(len(shares)) as ex:
        list(ex.map(one, shares))
    dt = time.perf_counter() - t0
    if limit is not None:
        limit.restore_original_limits()
    return {"value": nrows / dt, "unit": "tokens/s", "cores": len(shares), "kind": "oracle",
            "cpu_model": model, "host_cores_allowed": allowed,
            "sample": f"{nrows} query rows spread evenly over L={w.L} of the same block "
                      f"(full layer row + block scores + top-{w.topk} + {w.n_sparse} gated sparse layers), "
                      f"{len(shares)} worker threads x 1 BLAS thread, {dt:.1f} s wall"}


# ---------------------------------------------------------------------------

def kernel_sources_sha1(files=TRAFFIC_SOURCES):
    import hashlib
    h = hashlib.sha1()
    for f in files:
        with open(os.path.join(ROOT, "hybrid_sparse_attention_flash_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def calibrate_copy(dev, mib=512, reps=3):
    """A plain device copy of known size, for scaling the HBM byte counters."""
    src = torch.empty(mib * 2 ** 20 // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[bench] calibration copy: {reps} x {mib} MiB read + {mib} MiB written")
    del src, dst


def token_sparse_keys(idx, L, window):
    """Visible keys of the HySparse2 sparse layer, summed over queries: the
    selected tokens j <= i of the query's tile united with [i-window+1, i]."""
    nt, k = idx.shape[1], idx.shape[2]
    sel = torch.where(idx[0] >= 0, idx[0].to(torch.int64), torch.full_like(idx[0], 1 << 40, dtype=torch.int64))
    sel = torch.sort(sel, dim=1).values                                  # [nt, k]
    i = torch.arange(L, device=idx.device, dtype=torch.int64)
    t = i // 64
    rows = sel[t]                                                        # [L, k]
    le_i = torch.searchsorted(rows, i.view(-1, 1), right=True).view(-1)
    lo = torch.clamp(i - window + 1, min=0)
    below_lo = torch.searchsorted(rows, lo.view(-1, 1), right=False).view(-1)
    in_win = le_i - below_lo
    return int((le_i - in_win + torch.clamp(i + 1, max=window)).sum().item())


def bench_prefill2(args, dev, name):
    """HySparse2 block (fp8 MQA KV): full layer + tile-token scores, top-k per
    64-query tile, token-sparse layers with the forced window."""
    w = synth.WORKLOADS[name]
    log(f"[bench] generating {w.name} inputs (L={w.L}, {w.n_sparse + 1} layers)")
    q = [synth.gen_q(w, l).to(dev) for l in range(w.n_sparse + 1)]
    k, ks = synth.gen_kv(w, "k")
    v, vs = synth.gen_kv(w, "v")
    k, v = k.to(dev), v.to(dev)
    wmode = args.window_mode
    sel = "block" if args.selection == "block" else "token"
    blk = HySparse2Block(w.B, w.L, w.Hq, w.Hkv, w.D, w.n_sparse, w.topk, w.window, tile=w.block, device=dev,
                         out_dtype=torch.bfloat16, window_mode=wmode, selection=sel)
    gw = [synth.gen_gate_w(w, l + 1).to(dev) for l in range(w.n_sparse)] if wmode == "gated" else None

    def run(timer=None):
        def rec(nm, fn):
            if timer is None:
                fn()
            else:
                a, b = timer.span(nm)
                a.record(); fn(); b.record()
        rec("full_attn+scores", lambda: blk.full(q[0], k, v, ks, vs))
        rec("select_topk", blk.select)
        for l in range(w.n_sparse):
            rec("sparse_layer", lambda: blk.sparse_layer(l, q[l + 1], k, v, ks, vs, gw[l] if gw else None))
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    timer = Timer()
    g0 = torch.cuda.Event(enable_timing=True)
    g1 = torch.cuda.Event(enable_timing=True)
    g0.record()
    for _ in range(args.steps):
        run(timer)
    g1.record()
    torch.cuda.synchronize()
    step_ms = g0.elapsed_time(g1) / args.steps
    tot = timer.totals_ms()
    per_step = {kk: vv / args.steps for kk, vv in tot.items()}
    launches = {kk: c // args.steps for kk, c in timer.counts().items()}
    fl_full = full_attention_flops(w)
    if wmode == "gated":
        # selected tokens only in the sparse branch, plus the gated window branch's pairs
        win_pairs = sum(min(i + 1, w.window) for i in range(w.L)) * w.B
        fl_layer = 4.0 * w.D * w.Hq * (token_sparse_keys(blk.idx, w.L, 0) + win_pairs)
    else:
        fl_layer = 4.0 * w.D * w.Hq * token_sparse_keys(blk.idx, w.L, w.window)
    stages = {kk: {"ms_per_step": round(per_step[kk], 4), "launches_per_step": launches[kk]} for kk in per_step}
    for kk, fl in (("full_attn+scores", fl_full), ("sparse_layer", w.n_sparse * fl_layer)):
        tf = fl / (per_step[kk] * 1e-3) / 1e12
        stages[kk]["tflops"] = round(tf, 2)
        stages[kk]["frac_mfma_bf16"] = round(tf / PEAK_BF16_TFLOPS, 4)
    dom = max(["full_attn+scores", "sparse_layer"], key=lambda kk: per_step[kk])
    avg = per_step[dom] / launches[dom]
    work = fl_full if dom == "full_attn+scores" else fl_layer
    ach = work / (avg * 1e-3) / 1e12
    roof = {"kernel": "full_attn (causal + tile-token scores)" if dom == "full_attn+scores"
            else ("sparse_layer (selected tokens U forced window, fp8 KV)" if wmode == "forced" else
                  "sparse_layer (selected tokens, then gated window branch: 2 launches, fp8 KV)"), "bound": "mfma",
            "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(ach / PEAK_BF16_TFLOPS, 4), "avg_launch_ms": round(avg, 4),
            "work_per_launch": f"{work:.4g} FLOP (4*D per visible (query, head, key) pair)", "traffic": None}
    log(f"[bench] {w.name}: {step_ms:.3f} ms/step")
    return {"w": w, "step_ms": step_ms, "stages": stages, "roofline": roof, "host": None}


def bench_prefill(args, dev):
    name = args.workload
    if synth.WORKLOADS[name].variant == "hysparse2":
        return bench_prefill2(args, dev, name)
    w = synth.WORKLOADS[name]
    log(f"[bench] generating {w.name} inputs (L={w.L}, {w.n_sparse + 1} layers)")
    t0 = time.time()
    q_h = [synth.gen_q(w, l) for l in range(w.n_sparse + 1)]
    k_h, _ = synth.gen_kv(w, "k")
    v_h, _ = synth.gen_kv(w, "v")
    kw_h = [synth.gen_window_kv(w, l + 1, "kw")[0] for l in range(w.n_sparse)]
    vw_h = [synth.gen_window_kv(w, l + 1, "vw")[0] for l in range(w.n_sparse)]
    gw_h = [synth.gen_gate_w(w, l + 1) for l in range(w.n_sparse)]
    log(f"[bench] inputs generated in {time.time() - t0:.1f} s; uploading")
    inp = ([x.to(dev) for x in q_h], k_h.to(dev), v_h.to(dev), [x.to(dev) for x in kw_h],
           [x.to(dev) for x in vw_h], [x.to(dev) for x in gw_h])
    blk = HySparseBlock(w.B, w.L, w.Hq, w.Hkv, w.D, w.n_sparse, w.topk, w.window, device=dev,
                        out_dtype=torch.bfloat16, selection="kv_group" if args.selection == "kv_group" else "all_heads")
    for i in range(args.warmup):
        run_block(blk, inp)
        torch.cuda.synchronize()
        log(f"[bench] warmup {i + 1}/{args.warmup} done")
    timer = Timer()
    torch.cuda.synchronize()
    g0 = torch.cuda.Event(enable_timing=True)
    g1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    g0.record()
    for i in range(args.steps):
        run_block(blk, inp, timer)
    g1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = g0.elapsed_time(g1) / args.steps
    log(f"[bench] {args.steps} steps: {step_ms:.3f} ms/step (wall {wall * 1000 / args.steps:.3f})")
    # per-step distribution, warm (back to back) and cold (caches flushed before each step)
    warm = per_step_times(lambda: run_block(blk, inp), args.steps)
    flush = CacheFlush(dev)
    cold = per_step_times(lambda: run_block(blk, inp), args.steps, flush)
    del flush
    timing = {"warm": stats_ms(warm), "cold_512MiB_flush": stats_ms(cold)}
    log(f"[bench] per step: warm median {timing['warm']['median_ms']} ms, "
        f"cold median {timing['cold_512MiB_flush']['median_ms']} ms")
    timing["clocks_after_timed_steps"] = clock_state()
    tot = timer.totals_ms()
    per_step = {k: v / args.steps for k, v in tot.items()}
    launches = {k: c // args.steps for k, c in timer.counts().items()}

    # algorithmic work of the step
    fl_full = full_attention_flops(w)
    # visible selected keys per sparse layer over all heads: one set for every
    # head, or one set per KV group serving that group's G heads
    ng = blk.idx.shape[0]
    keys_sel = sum(sparse_keys_per_query(blk.idx[g], w.L, w.block) for g in range(ng)) * (w.Hq // ng)
    fl_sparse = 4.0 * w.D * keys_sel
    win_keys = sum(min(i + 1, w.window) for i in range(w.L)) * w.Hq * w.B
    fl_swa = 4.0 * w.D * win_keys
    fl_layer = fl_sparse + fl_swa
    tflops = {
        "full_attn+scores": fl_full / (per_step["full_attn+scores"] * 1e-3) / 1e12,
        "sparse_layer": w.n_sparse * fl_layer / (per_step["sparse_layer"] * 1e-3) / 1e12,
    }
    # logical gathered K/V bytes of the sparse branch per layer (per KV head reading of each query's keys)
    gather_bytes = keys_sel / w.G * w.D * 2 * 2
    stages = {k: {"ms_per_step": round(per_step[k], 4), "launches_per_step": launches[k]} for k in per_step}
    for k, v in tflops.items():
        stages[k]["tflops"] = round(v, 2)
        stages[k]["frac_mfma_bf16"] = round(v / PEAK_BF16_TFLOPS, 4)
    stages["sparse_layer"]["logical_gather_GBs"] = round(
        w.n_sparse * gather_bytes / (per_step["sparse_layer"] * 1e-3) / 1e9, 1)

    # roofline of the dominant kernel (largest share of the step).  Work is
    # algorithmic: only causal (full layer), or selected-and-causal plus
    # in-window (sparse layer) (query, key) pairs, 4*D FLOP each.  The sparse
    # layer processes each query tile's union of selected blocks on MFMA, so
    # its binding roof is MFMA; its logical gathered bytes (each query reading
    # its own blocks) are reported beside it as context.
    dom = max(["full_attn+scores", "sparse_layer"], key=lambda k: per_step[k])
    avg = per_step[dom] / launches[dom]
    work = fl_full if dom == "full_attn+scores" else fl_layer
    ach = work / (avg * 1e-3) / 1e12
    roof = {"kernel": "full_attn (causal + block scores)" if dom == "full_attn+scores"
            else "sparse_layer (selected 64-key blocks, query-tile union; own 128-key window; gate)",
            "bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(ach / PEAK_BF16_TFLOPS, 4), "avg_launch_ms": round(avg, 4),
            "work_per_launch": f"{work:.4g} FLOP (4*D per visible (query, head, key) pair)", "traffic": None}
    if (dom == "sparse_layer" and args.selection == "default" and TRAFFIC
            and TRAFFIC["sources_sha1"] == kernel_sources_sha1()):
        roof["traffic"] = TRAFFIC["bytes_per_launch"]
    if dom == "sparse_layer":
        roof["logical_gather_GBs"] = round(gather_bytes / (avg * 1e-3) / 1e9, 1)
    res = {"w": w, "step_ms": step_ms, "stages": stages, "roofline": roof, "timing": timing,
           "host": (q_h, k_h, v_h, kw_h, vw_h, gw_h)}
    del inp, blk
    torch.cuda.empty_cache()
    return res


def bench_decode(args, dev):
    w = synth.WORKLOADS["decode_1m"]
    log(f"[bench] generating {w.name} inputs (B={w.B}, N={w.L}, fp8 cache)")
    qf = synth.gen_q(w, 0).to(dev)
    qs = [synth.gen_q(w, l + 1).to(dev) for l in range(w.n_sparse)]
    kc, ks = synth.gen_kv(w, "k")
    kc = kc.to(dev)
    vc, vs = synth.gen_kv(w, "v")
    vc = vc.to(dev)
    dec = HySparse2Decode(w.B, w.L, w.Hq, w.D, w.n_sparse, w.topk, w.window, device=dev)
    lens = w.lens()
    step = lambda: dec.run(qf, kc, vc, lens, qs, ks, vs)
    for _ in range(max(3, args.warmup)):
        step()
    torch.cuda.synchronize()
    steps = max(20, args.steps * 5)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1000 / steps
    warm = per_step_times(step, steps)
    flush = CacheFlush(dev)
    cold = per_step_times(step, steps, flush)
    del flush
    # Algorithmic HBM bytes of the step: the full layer streams each cache's
    # valid fp8 K and V once (2*D bytes per token) and writes one fp32 token
    # score per cached position; the selection reads the scores once; each
    # sparse layer gathers its selected tokens and recent window (2*D bytes
    # each).  Queries and outputs (a few hundred KB) are left out.
    kv_bytes = 2.0 * sum(lens) * w.D
    score_bytes = 2.0 * 4 * w.B * w.L
    gather_bytes = 2.0 * w.D * w.n_sparse * w.B * (w.topk + w.window)
    step_bytes = kv_bytes + score_bytes + gather_bytes
    gbs = step_bytes / (us * 1e-6) / 1e9
    timing = {"warm": stats_ms(warm), "cold_512MiB_flush": stats_ms(cold)}
    log(f"[bench] decode: {us:.1f} us/step ({gbs:.0f} GB/s algorithmic); per step warm median "
        f"{timing['warm']['median_ms'] * 1000:.1f} us, cold median {timing['cold_512MiB_flush']['median_ms'] * 1000:.1f} us")
    return {"workload": w.name, "us_per_step": round(us, 2), "us_per_token": round(us / w.B, 2),
            "batch": w.B, "cache_tokens": w.L, "steps": steps, "timing": timing,
            "roofline": {"kernel": "decode step (split-K full layer with token scores, merge, top-1024, "
                                   f"{w.n_sparse} sparse layers; one ABI call)",
                         "bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4), "avg_step_us": round(us, 2),
                         "work_per_step": f"{step_bytes:.4g} B (fp8 K+V of the valid cache, token scores written "
                                          "and read, gathered tokens of the sparse layers)",
                         "traffic": DECODE_TRAFFIC["bytes_per_step"]
                         if DECODE_TRAFFIC and DECODE_TRAFFIC["sources_sha1"] == kernel_sources_sha1(
                             DECODE_TRAFFIC_SOURCES) else None}}


def bench_hs_decode(args, dev):
    """HySparse (block-level) decode step: full layer + block scores over a
    128k-token bf16 GQA cache per sequence, top-16 blocks, 11 sparse layers
    (block gather, ring window append, gate)."""
    w = synth.HS_DECODE_WORKLOAD
    log(f"[bench] generating {w.name} inputs (B={w.B}, N={w.L}, bf16 cache, {w.n_sparse} sparse layers)")
    x = synth.gen_hs_decode(w)
    q_full, k, v = x["q_full"].to(dev), x["k"].to(dev), x["v"].to(dev)
    qs = [t.to(dev) for t in x["q"]]
    kn, vn = [t.to(dev) for t in x["k_new"]], [t.to(dev) for t in x["v_new"]]
    kr, vr = [t.to(dev) for t in x["k_ring"]], [t.to(dev) for t in x["v_ring"]]
    gw = [t.to(dev) for t in x["gate_w"]]
    nblk = (w.L + 63) // 64
    o_full = torch.empty(w.B, 1, w.Hq, w.D, dtype=torch.bfloat16, device=dev)
    bs = torch.empty(w.B, nblk, dtype=torch.float32, device=dev)
    idx = torch.empty(w.B, w.topk, dtype=torch.int32, device=dev)
    o_sp = [torch.empty_like(o_full) for _ in qs]
    lens = w.lens()
    ws = None

    def step():
        nonlocal ws
        ws = ops.hys_hysparse_decode_step(q_full, k, v, lens, o_full, bs, idx, qs, kn, vn, kr, vr, gw, o_sp,
                                          w.topk, workspace=ws)
    for _ in range(max(3, args.warmup)):
        step()
    torch.cuda.synchronize()
    steps = max(20, args.steps * 5)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1000 / steps
    kv_bytes = 2.0 * sum(lens) * w.Hkv * w.D * 2           # bf16 K + V streamed by the full layer
    gathered = 2.0 * w.n_sparse * w.B * w.Hkv * (w.topk * 64 + w.window) * w.D * 2
    gbs = (kv_bytes + gathered) / (us * 1e-6) / 1e9
    log(f"[bench] HySparse decode: {us:.1f} us/step, {gbs:.0f} GB/s algorithmic")
    return {"workload": w.name, "us_per_step": round(us, 2), "us_per_token": round(us / w.B, 2), "batch": w.B,
            "cache_tokens": w.L, "steps": steps,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "work_per_step": f"{kv_bytes + gathered:.4g} B (full-layer K+V, gathered blocks + windows)",
                         "traffic": HS_DECODE_TRAFFIC["bytes_per_step"]
                         if HS_DECODE_TRAFFIC["sources_sha1"] == kernel_sources_sha1(HS_DECODE_TRAFFIC_SOURCES)
                         else None}}


def bench_bridge(args, dev):
    """HySparse2 KV Bridging: the cross-decoder full layer's K/V projected from
    the self-decoder's hidden states into the fp8 MQA cache, one call per
    step (64k tokens, d_model 4096, one 128-wide KV head)."""
    w = synth.BRIDGE_WORKLOAD
    B, L, dm, Hkv, D = w["B"], w["L"], w["d_model"], w["Hkv"], w["D"]
    n = Hkv * D
    log(f"[bench] generating {w['name']} inputs (L={L}, d_model={dm})")
    h, wk, wv = synth.gen_bridge(0, w["cfg_id"], B, L, dm, n)
    h, wk, wv = h.to(dev), wk.to(dev), wv.to(dev)
    kc = torch.empty((B, L, Hkv, D), dtype=torch.uint8, device=dev)
    vc = torch.empty_like(kc)
    amax = torch.empty(2, dtype=torch.float32, device=dev)
    ks = vs = 8.0 / 448.0
    for _ in range(max(3, args.warmup)):
        ops.hys_kv_bridge_fwd(h, wk, wv, kc, vc, ks, vs, amax)
    torch.cuda.synchronize()
    calls = max(20, args.steps * 5)

    def timed(am):
        # HIP events on the launch stream (the current stream, which ops uses)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(calls):
            ops.hys_kv_bridge_fwd(h, wk, wv, kc, vc, ks, vs, am)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1000 / calls
    us_call = timed(amax)      # the call: amax clear + projection kernel
    us = timed(None)           # the projection kernel alone (no amax, no clear)
    nbytes = B * L * dm * 2 + 2 * n * dm * 2 + 2 * B * L * n      # h, W_k + W_v, fp8 K + V
    flops = 2.0 * B * L * dm * 2 * n
    gbs = nbytes / (us * 1e-6) / 1e9
    tf = flops / (us * 1e-6) / 1e12
    log(f"[bench] kv bridge: {us_call:.1f} us/call, kernel {us:.1f} us, {gbs:.0f} GB/s, {tf:.0f} TFLOP/s")
    traffic = (BRIDGE_TRAFFIC["bytes_per_launch"]
               if BRIDGE_TRAFFIC["sources_sha1"] == kernel_sources_sha1(BRIDGE_TRAFFIC_SOURCES) else None)
    return {"workload": w["name"], "us_per_call": round(us_call, 2),
            "tokens_per_s": round(B * L / (us_call * 1e-6), 1), "calls": calls,
            "roofline": {"kernel": "kv_bridge (bf16 projection, fp8 e4m3 epilogue)", "bound": "hbm",
                         "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4), "avg_launch_us": round(us, 2),
                         "work_per_launch": f"{nbytes:.4g} B (h, both weights, fp8 K and V)",
                         "mfma_tflops": round(tf, 1), "frac_mfma_bf16": round(tf / PEAK_BF16_TFLOPS, 4),
                         "traffic": traffic}}


def bench_bwd(args, dev):
    """Backward pass of the 32k HySparse block (the training step's attention
    gradients): the full layer's causal gradient, then the 11 sparse layers'
    (block-sparse branch, window branch, gate), dK/dV of the shared cache
    accumulated over all 12 layers.  The forward that saves what the backward
    needs runs once before the timed region."""
    w = synth.WORKLOADS["moe80b_32k"]
    log(f"[bench] backward: generating {w.name} inputs")
    q = [synth.gen_q(w, l).to(dev) for l in range(w.n_sparse + 1)]
    k, v = synth.gen_kv(w, "k")[0].to(dev), synth.gen_kv(w, "v")[0].to(dev)
    kw = [synth.gen_window_kv(w, l + 1, "kw")[0].to(dev) for l in range(w.n_sparse)]
    vw = [synth.gen_window_kv(w, l + 1, "vw")[0].to(dev) for l in range(w.n_sparse)]
    gw = [synth.gen_gate_w(w, l + 1).to(dev) for l in range(w.n_sparse)]
    dout = [synth.gen_grad_out(w, l).to(dev) for l in range(w.n_sparse + 1)]
    tr = HySparseTrainer(w.B, w.L, w.Hq, w.Hkv, w.D, w.n_sparse, w.topk, w.window, device=dev)
    inp = (q, k, v, kw, vw, gw)
    f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    f0.record()
    tr.forward(*inp)
    f1.record()
    torch.cuda.synchronize()
    fwd_ms = f0.elapsed_time(f1)

    def step(timer=None):
        def rec(nm, fn):
            if timer is None:
                fn()
            else:
                a, b = timer.span(nm)
                a.record(); fn(); b.record()
        f = tr.fwd
        rec("full_bwd", lambda: ops.hys_full_attn_bwd(q[0], k, v, f.o_full, f.lse, dout[0], tr.dq[0], tr.dk, tr.dv))
        for l in range(w.n_sparse):
            rec("sparse_layer_bwd", lambda: ops.hys_sparse_layer_bwd(
                q[l + 1], k, v, f._idx(), kw[l], vw[l], w.window, gw[l], tr.o_sp[l], tr.lse_sp[l], tr.o_w[l],
                tr.lse_w[l], dout[l + 1], tr.dq[l + 1], tr.dk, tr.dv, tr.dkw[l], tr.dvw[l], tr.dgate_w[l],
                accumulate_kv=True, topk=w.topk))
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    timer = Timer()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record()
    for _ in range(args.steps):
        step(timer)
    g1.record()
    torch.cuda.synchronize()
    step_ms = g0.elapsed_time(g1) / args.steps
    per = {kk: vv / args.steps for kk, vv in timer.totals_ms().items()}
    # algorithmic work: 10*D FLOP per visible (query, head, key) pair (recomputed
    # QK^T, dP = dO V^T, dV = P^T dO, dQ = dS K, dK = dS^T Q)
    pairs_full = w.Hq * w.L * (w.L + 1) / 2 * w.B
    keys_sel = sparse_keys_per_query(tr.fwd.idx[0], w.L, w.block) * w.Hq
    win = sum(min(i + 1, w.window) for i in range(w.L)) * w.Hq * w.B
    fl_full = 10.0 * w.D * pairs_full
    fl_layer = 10.0 * w.D * (keys_sel + win)
    st = {"full_bwd": {"ms_per_step": round(per["full_bwd"], 4),
                       "tflops": round(fl_full / (per["full_bwd"] * 1e-3) / 1e12, 2)},
          "sparse_layer_bwd": {"ms_per_step": round(per["sparse_layer_bwd"], 4), "launches_per_step": w.n_sparse,
                               "tflops": round(w.n_sparse * fl_layer / (per["sparse_layer_bwd"] * 1e-3) / 1e12, 2)}}
    for kk in st:
        st[kk]["frac_mfma_bf16"] = round(st[kk]["tflops"] / PEAK_BF16_TFLOPS, 4)
    tot = fl_full + w.n_sparse * fl_layer
    log(f"[bench] backward {w.name}: {step_ms:.3f} ms/step (forward with saved branches {fwd_ms:.3f} ms)")
    return {"workload": w.name, "ms_per_step": round(step_ms, 4), "tokens_per_s": round(w.L * w.B / (step_ms * 1e-3), 1),
            "tflops": round(tot / (step_ms * 1e-3) / 1e12, 2), "forward_saving_ms": round(fwd_ms, 4),
            "work": "10*D FLOP per visible (query, head, key) pair", "stages": st}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-bridge", action="store_true")
    ap.add_argument("--no-hs-decode", action="store_true")
    ap.add_argument("--only-hs-decode", action="store_true", help="time only the HySparse decode step")
    ap.add_argument("--only-bridge", action="store_true", help="time only the KV Bridging projection")
    ap.add_argument("--only-decode", action="store_true", help="time only the HySparse2 1M decode step")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured-peak microbenchmarks")
    ap.add_argument("--no-bwd", action="store_true")
    ap.add_argument("--only-bwd", action="store_true", help="time only the backward pass of the 32k HySparse block")
    ap.add_argument("--cpu-rows", type=int, default=192)
    ap.add_argument("--workload", default="moe80b_32k",
                    choices=["moe80b_32k", "dense7b_16k", "hysparse2_64k", "tiny_fp32"],
                    help="prefill block to time (default: the 32k HySparse block the metric is quoted on)")
    ap.add_argument("--selection", default="default", choices=["default", "kv_group", "block"],
                    help="ablation: per-KV-group block selection (HySparse) or block-level selection at the "
                         "token budget (HySparse2)")
    ap.add_argument("--window-mode", default="forced", choices=["forced", "gated"],
                    help="HySparse2 ablation: gated window branch instead of the forced recent window")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run a plain copy of known size (for scaling HBM byte counters)")
    args = ap.parse_args()
    v2 = synth.WORKLOADS[args.workload].variant == "hysparse2"
    if (args.selection == "kv_group" and v2) or ((args.selection == "block" or args.window_mode == "gated")
                                                 and not v2):
        print("--selection kv_group applies to the HySparse workloads; --selection block and --window-mode gated "
              "to the HySparse2 workload", file=sys.stderr)
        sys.exit(2)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the hot path is built for a single MI355X and has no "
              "multi-GPU mode; run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = "cuda:0"
    ops.abi_version()      # fail loudly if libhys.so is missing
    if args.calibrate_copy:
        calibrate_copy(dev)
    if args.only_bridge:
        print(json.dumps({"kv_bridge": bench_bridge(args, dev)}), flush=True)
        return
    if args.only_hs_decode:
        print(json.dumps({"hs_decode": bench_hs_decode(args, dev)}), flush=True)
        return
    if args.only_bwd:
        print(json.dumps({"backward": bench_bwd(args, dev)}), flush=True)
        return
    if args.only_decode:
        print(json.dumps({"decode": bench_decode(args, dev)}), flush=True)
        return
    clocks = clock_state()      # before any timed work (idle clocks)
    pre = bench_prefill(args, dev)
    w = pre["w"]
    dec = None if args.no_decode else bench_decode(args, dev)
    bridge = None if args.no_bridge else bench_bridge(args, dev)
    hs_dec = None if args.no_hs_decode else bench_hs_decode(args, dev)
    bwd = None if args.no_bwd else bench_bwd(args, dev)
    cpu = None
    ablation = args.selection != "default" or args.window_mode != "forced"
    if not args.no_cpu and not ablation and pre["host"] is not None:
        log(f"[bench] timing the CPU oracle on {args.cpu_rows} sampled rows")
        cpu = cpu_baseline(w, pre["host"], args.cpu_rows)
        log(f"[bench] oracle: {cpu['value']:.2f} tokens/s on {cpu['cores']} threads")
    peaks = None if args.no_peaks else measured_peaks(dev)
    if peaks:
        log(f"[bench] measured peaks: bf16 GEMM {peaks['bf16_gemm_tflops']} TFLOP/s, copy {peaks['hbm_copy_GBs']} GB/s")
        roof = pre["roofline"]
        mp = peaks["bf16_gemm_tflops"] if roof["unit"] == "TFLOP/s" else peaks["hbm_copy_GBs"]
        roof["measured_peak"] = mp
        roof["frac_of_measured_peak"] = round(roof["achieved"] / mp, 4)
        if dec:
            dec["roofline"]["measured_peak"] = peaks["hbm_copy_GBs"]
            dec["roofline"]["frac_of_measured_peak"] = round(dec["roofline"]["achieved"] / peaks["hbm_copy_GBs"], 4)
    tok_s = w.L * w.B / (pre["step_ms"] * 1e-3)
    out = {
        "metric": METRIC, "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(pre["step_ms"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.q_dtype,
        "data": f"synthetic (seeded N(0,1); {w.q_dtype} Q, {w.kv_dtype} K/V"
                + (f"; {w.needles} needle keys x{w.needle_scale:g})" if w.needles else ")"),
        "config": {"workload": w.name, "batch": w.B, "seq_len": w.L, "q_heads": w.Hq, "kv_heads": w.Hkv,
                   "head_dim": w.D, "layers": f"1 full + {w.n_sparse} sparse",
                   "selection": (f"top-{w.topk} of {w.block}-token blocks per query" if w.variant == "hysparse"
                                 else f"top-{w.topk} tokens per {w.block}-query tile"),
                   "window": w.window,
                   **({"ablation": {"selection": args.selection, "window_mode": args.window_mode}}
                      if args.selection != "default" or args.window_mode != "forced" else {})},
        "roofline": pre["roofline"],
        "cpu_baseline": cpu,
        "stages": pre["stages"],
        "timing": pre.get("timing"),
        "measured_peaks": peaks,
        "clocks_at_start": clocks,
        "decode": dec,
        "kv_bridge": bridge,
        "hs_decode": hs_dec,
        "backward": bwd,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
