#!/usr/bin/env python3
"""Benchmark of the ragged pack -> attend -> unpack path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step = one whole pass of the path (pack: keep mask -> cu_seqlens, gather
index, packed rows; ragged attention; unpack) over one batch of synthetic DeiT-S
tokens (N = 197, H = 6, head dim 64, bf16), enqueued by one host call (three
kernel launches from C++; --graph times the captured HIP graph instead).
The headline workload is 80 % token pruning (40 kept tokens per image, CLS
included) at batch 256, the top of the 1-256 batch range the metric covers.

Printed: one JSON line with packed tokens/s over the timed steps, the attention
kernel latency, per-kernel HIP-event durations and their HBM roofline
fractions, the padded comparator, the prune-rate sweep at B in {1, 2, 4, 256},
the host dispatch floor (measured in C++), and the CPU oracle's throughput on the
host cores.

Other modes (used under rocprofv3, see profiles/):
    --kernels-only   run only the timed pipeline steps, then as many fused passes
                     (no sweep, no oracle)
    --pmc-calib      run a plain device copy of a known size (counter scale)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
METRIC = "rag_attn latency us + packed tokens/s, DeiT-S 80% prune BS=1-256; HBM/MFMA %"
PROFILES = os.path.join(ROOT, "profiles")


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--batch", type=int, default=256)
    ap.add_argument("--prune", type=int, default=800, help="prune rate in thousandths")
    ap.add_argument("--workload", default="deits", choices=("deits", "deitb_ragged", "deitb384"),
                    help="deits: DeiT-S at --batch/--prune (the headline); deitb_ragged: DeiT-B "
                         "B=64 N=197 with lengths uniform in [20, 197]; deitb384: DeiT-B at 384x384 "
                         "(N=577) B=32, keep 0.5 +- 0.1 (--kernels-only profiling of those shapes)")
    ap.add_argument("--graph", action="store_true", help="time steps as hipGraphLaunch")
    ap.add_argument("--kernels-only", action="store_true")
    ap.add_argument("--pmc-calib", action="store_true")
    ap.add_argument("--block-only", action="store_true",
                    help="only the encoder-block timings (DeiT-S B=256 80%% prune, DeiT-B 384x384), "
                         "for profiling the block's kernels")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="bound on the oracle's CPU time for cpu_baseline")
    return ap.parse_args()


# ----------------------------------------------------------------- buffers
class Bufs:
    """Device buffers of one workload, sized to the B*N capacity."""

    def __init__(self, w, out_dtype=None):
        import torch
        from ragged_attention_token_amd import binding

        self.w = w
        B, N, C = w.B, w.N, w.C
        rows = np.ascontiguousarray(w.qkv.reshape(B * N, 3 * C))
        if w.dtype == "f32":
            self.src = torch.from_numpy(rows).cuda()
        else:
            self.src = torch.from_numpy(rows.view(np.int16)).view(torch.bfloat16).cuda()
        out_dtype = out_dtype or self.src.dtype
        self.keep = torch.from_numpy(w.keep).cuda()
        self.packed = torch.empty(B * N, 3 * C, dtype=self.src.dtype, device="cuda")
        self.cu = torch.zeros(B + 1, dtype=torch.int32, device="cuda")
        self.gather = torch.zeros(B * N, dtype=torch.int32, device="cuda")
        self.mx = torch.zeros(1, dtype=torch.int32, device="cuda")
        self.o_packed = torch.empty(B * N, C, dtype=out_dtype, device="cuda")
        self.dst = torch.zeros(B * N, C, dtype=out_dtype, device="cuda")
        self.o_pad = torch.empty(B * N, C, dtype=out_dtype, device="cuda")
        # host bound of the kept count per image: a top-k pruning rate fixes it
        # (every image keeps the same number of tokens), so no device value is
        # read back to size the attention launches
        self.max_seqlen = int(w.lengths.max())
        self.pipe = binding.Pipeline(self.keep, self.src, self.packed, self.cu, self.gather,
                                     self.o_packed, self.dst, H=w.H, scale=w.scale,
                                     max_seqlen=self.max_seqlen, max_seqlen_dev=self.mx)
        self.binding = binding

    # the three stages and the comparator, each one launch on the current stream
    def pack(self):
        self.binding.rag_pack(self.keep, self.src, self.packed, self.cu, self.gather, self.mx)

    def attn(self):
        C = self.w.C
        p = self.packed
        self.binding.rag_attn(p[:, :C], p[:, C:2 * C], p[:, 2 * C:], self.cu, self.max_seqlen,
                              self.o_packed, H=self.w.H, scale=self.w.scale)

    def unpack(self):
        self.binding.rag_unpack(self.o_packed, self.cu, self.gather, self.dst, N=self.w.N)

    def padded(self):
        C = self.w.C
        s = self.src
        self.binding.rag_attn_padded(s[:, :C], s[:, C:2 * C], s[:, 2 * C:], self.keep, self.o_pad,
                                     H=self.w.H, scale=self.w.scale)


# ------------------------------------------------------------ algorithmic work
def algorithmic(w, out_bytes):
    """Algorithmic bytes per launch of each kernel and attention flops."""
    T, B, N, C, H, d = w.T, w.B, w.N, w.C, w.H, w.d
    s_in = w.elem_bytes
    L = w.lengths.astype(np.int64)
    attn_flops = int(4 * (L * L).sum() * d * H)
    return {
        # keep mask + (read + write) of each kept fused row + gather index + offsets
        "pack": B * N + T * (2 * 3 * C * s_in + 4) + 4 * (B + 1),
        # q, k, v rows read once, o rows written once
        "attn": T * (3 * C * s_in + C * out_bytes),
        # read + write of each kept output row + gather index + offsets
        "unpack": T * (2 * C * out_bytes + 4) + 4 * (B + 1),
        # padded: every position read and written, whatever the prune rate
        "padded": B * N * (3 * C * s_in + C * out_bytes) + B * N,
        # the whole pass as one gathered launch: keep mask, kept q/k/v rows in, o rows out
        "fused": B * N + T * (3 * C * s_in + C * out_bytes),
        "attn_flops": attn_flops,
        "padded_flops": int(4 * B * N * N * d * H),
    }


def source_sha(path):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def read_traffic(kernel, workload):
    """HBM bytes per launch from a committed rocprofv3 PMC summary, or None when
    none exists or the kernel source changed since the counters were taken."""
    path = os.path.join(PROFILES, "pmc_%s_%s.txt" % (kernel, workload))
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    try:
        src = os.path.join(ROOT, "ragged_attention_token_amd", "csrc", kv["source_file"])
        if source_sha(src) != kv["source_sha256"]:
            return None
        calib_bytes = float(kv["calib_bytes"])
        fetch = float(kv["fetch_kib_per_dispatch"]) * calib_bytes / float(kv["calib_fetch_kib"])
        write = float(kv["write_kib_per_dispatch"]) * calib_bytes / float(kv["calib_write_kib"])
        return int(round(fetch + write))
    except (KeyError, ValueError, OSError):
        return None


# ------------------------------------------------------------------- modes
def pmc_calib():
    """A plain device-to-device copy of 1 GiB, five times: the known-size
    reference that scales the FETCH_SIZE / WRITE_SIZE counters."""
    import torch

    nbytes = 1 << 30
    a = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calib_copy_bytes_read": nbytes, "calib_copy_bytes_written": nbytes,
                      "launches": 5}))


def cpu_baseline(w, seconds):
    """The oracle (plain C, fp64, one thread) on the same workload: pack,
    attention, unpack, repeated until `seconds` of CPU time (at least once)."""
    import oracle
    from ragged_attention_token_amd import workloads as wl

    rows = wl.rows(w)
    dst0 = np.zeros((w.B * w.N, w.C), dtype=np.float64)
    reps, t_total = 0, 0.0
    while reps == 0 or (t_total < seconds and reps < 50):
        t0 = time.perf_counter()
        packed, cu, gather = oracle.pack(w.keep, rows)
        q, k, v = wl.split_qkv(packed, w.C)
        o = oracle.attn(q, k, v, cu, w.H, w.d, w.scale)
        oracle.unpack(o, cu, gather, dst0)
        t_total += time.perf_counter() - t0
        reps += 1
    return {"value": w.T * reps / t_total, "unit": "packed tokens/s", "cores": 1, "kind": "oracle",
            "sample": "whole workload (%s, T=%d), %d pass(es) of fp64 pack+attention+unpack in "
                      "%.1f s on one host thread" % (w.name, w.T, reps, t_total),
            "seconds_per_pass": t_total / reps,
            "host_cpu": _cpu_model(), "host_threads_available": len(os.sched_getaffinity(0))}


def cpu_baseline_threads(w, seconds, threads):
    """The same oracle passes on `threads` host threads at once: the batch is
    split into contiguous image ranges and each thread runs the oracle's pack,
    attention and unpack on its range (the oracle's C routines release the
    interpreter lock, so the ranges run in parallel).  Images are independent
    in every stage, so this is the whole workload's work, split by image."""
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    from ragged_attention_token_amd import workloads as wl

    rows = wl.rows(w)
    bounds = np.linspace(0, w.B, threads + 1).astype(int)
    chunks = [(int(a), int(b)) for a, b in zip(bounds[:-1], bounds[1:]) if b > a]
    dst0 = np.zeros((w.B * w.N, w.C), dtype=np.float64)

    def one(ch):
        b0, b1 = ch
        packed, cu, gather = oracle.pack(w.keep[b0:b1], rows[b0 * w.N:b1 * w.N])
        q, k, v = wl.split_qkv(packed, w.C)
        o = oracle.attn(q, k, v, cu, w.H, w.d, w.scale)
        oracle.unpack(o, cu, gather, dst0[b0 * w.N:b1 * w.N])
        return int(cu[-1])

    reps, t_total = 0, 0.0
    with ThreadPoolExecutor(max_workers=len(chunks)) as ex:
        while reps == 0 or (t_total < seconds and reps < 200):
            t0 = time.perf_counter()
            assert sum(ex.map(one, chunks)) == w.T
            t_total += time.perf_counter() - t0
            reps += 1
    return {"value": w.T * reps / t_total, "unit": "packed tokens/s", "cores": len(chunks),
            "kind": "oracle",
            "sample": "whole workload (%s, T=%d), %d pass(es) of fp64 pack+attention+unpack in "
                      "%.1f s, the images split over %d host threads" % (w.name, w.T, reps, t_total,
                                                                        len(chunks)),
            "seconds_per_pass": t_total / reps}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def measure_repack(steps):
    """A second pruning stage on a packed batch (progressive pruning): DeiT-S at B = 256 packed at 50% prune (99 kept per image), then
    re-packed to 40 per image (the headline's kept count) with rag_repack.
    Device time per launch from a captured run of back-to-back launches (no host
    work between them), and the launch's algorithmic bytes."""
    import torch
    from ragged_attention_token_amd import binding
    from ragged_attention_token_amd import workloads as wl

    w = wl.deits(256, 500)
    bf = Bufs(w)
    bf.pack()
    rows = w.B * w.N
    k2 = torch.zeros(rows, dtype=torch.uint8, device="cuda")
    k2_np = wl.second_stage_keep(w, 40, seed=1)
    k2[:w.T] = torch.from_numpy(k2_np).cuda()
    T2 = int(np.count_nonzero(k2_np))
    dst = torch.empty_like(bf.packed)
    cu2 = torch.zeros(w.B + 1, dtype=torch.int32, device="cuda")
    g2 = torch.zeros(rows, dtype=torch.int32, device="cuda")

    def call():
        binding.rag_repack(k2, bf.cu, bf.gather, bf.max_seqlen, bf.packed, dst, cu2, g2)

    call()
    torch.cuda.synchronize()
    eager = dst[:T2].clone()
    per_graph = 50
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(per_graph):
            call()
    graph.replay()
    torch.cuda.synchronize()
    assert torch.equal(dst[:T2].view(torch.uint8), eager.view(torch.uint8)), "replay differs"
    reps = max(4, min(40, steps // per_graph))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (reps * per_graph)
    row_bytes = 3 * w.C * w.elem_bytes
    alg = w.T + 4 * (w.B + 1) + T2 * (2 * row_bytes + 4 + 4) + 4 * (w.B + 1)
    return {"workload": "deits_b256_n197_h6: packed at 50%% prune (T=%d), re-packed to 40 per "
                        "image (T'=%d)" % (w.T, T2),
            "us": us, "alg_bytes": alg, "achieved_GBs": alg / us * 1e-3,
            "hbm_frac": alg / us * 1e-3 / HBM_PEAK_GBS,
            "timing": "%d launches captured in one graph, %d replays, HIP events" % (per_graph, reps)}


def measure_block(steps, w=None, label=None):
    """One encoder block (random weights, bf16) on a pruned batch: on the packed
    rows (ragged attention) against the same block on all B * N rows (padded
    attention with masked keys).  The analogue of the pages' end-to-end
    comparison for one post-pruning block.  Device time per forward from
    back-to-back calls between HIP events (host enqueue is faster than the GPU
    work here).  Default: DeiT-S at B = 256, 80% prune."""
    import torch
    from ragged_attention_token_amd import binding
    from ragged_attention_token_amd import workloads as wl

    w = w or wl.deits(256, 800)
    C, H = w.C, w.H
    P = wl.vit_block_params(C, 4, 1)
    # matrices drawn [in, out], uploaded in the [out, in] layout the block takes
    prm = {k: (torch.from_numpy(np.ascontiguousarray(v.T).view(np.int16)).view(torch.bfloat16).cuda()
               if k.startswith("w_") else torch.from_numpy(v).cuda()) for k, v in P.items()}
    blk = binding.Block(prm, H=H, scale=w.scale)
    xb = wl.hidden_rows(w.B, w.N, C, 2)
    x_all = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).cuda()
    keep = torch.from_numpy(w.keep).cuda()
    rows = w.B * w.N
    xp = torch.empty_like(x_all)
    cu = torch.zeros(w.B + 1, dtype=torch.int32, device="cuda")
    gather = torch.zeros(rows, dtype=torch.int32, device="cuda")
    binding.rag_pack(keep, x_all, xp, cu, gather)
    T, L = w.T, int(w.lengths.max())
    y_p, y_pad = torch.empty_like(x_all), torch.empty_like(x_all)

    def timed(fn):
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
        k = max(20, min(200, steps // 10))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(k):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / k

    packed_us = timed(lambda: blk.forward(xp, y_p, T, cu, L))
    padded_us = timed(lambda: blk.forward_padded(x_all, y_pad, keep))
    blk.close()
    label = label or ("DeiT-S block (C=384, H=6, MLP 4x, random bf16 weights), B=256: "
                      "%d packed rows (80%% prune) vs %d padded rows" % (T, rows))
    return {"workload": label, "packed_block_us": packed_us, "padded_block_us": padded_us,
            "speedup": padded_us / packed_us, "packed_tokens_per_s": T / packed_us * 1e6}


def sweep(steps):
    """Prune-rate sweep on the DeiT-S shape: per-launch device time of each kernel
    and of a whole pass (three launches, and one graph launch), and the host
    round trip (launch + synchronize) of each at that point."""
    import torch
    from ragged_attention_token_amd import binding
    from ragged_attention_token_amd import workloads as wl

    out = {}
    for B in wl.SWEEP_BATCHES:
        for p in wl.SWEEP_PRUNE_PERMILLE:
            w = wl.deits(B, p)
            bf = Bufs(w)
            bf.pipe.launch()
            torch.cuda.synchronize()
            it = max(50, min(steps, 400))
            m = bf.pipe.measure_stages(it)
            rec = {"T": w.T, "pack_us": m["pack"], "attn_us": m["attn"], "unpack_us": m["unpack"],
                   "padded_attn_us": m["padded"], "pipeline_us": m["eager_pass"],
                   "graph_pipeline_us": m["graph_pass"], "fused_pass_us": m["fused_pass"]}
            rec["ragged_pipeline_vs_padded_attn"] = rec["padded_attn_us"] / rec["pipeline_us"]
            # the point's dispatch-inclusive latency: host launch call(s) + stream
            # synchronize, p50 over 200 round trips from C++
            fl = bf.pipe.measure_dispatch(warmup=20, iters=200)
            rec["roundtrip_us"] = {k: fl[k + "_roundtrip"]["p50"]
                                   for k in ("attn", "eager3", "graph", "padded", "fused")}
            if B <= 4:
                # the serving configuration of the pipeline object itself: created
                # with the direct and fused flags, rag_pipeline_launch is one launch
                dp = binding.Pipeline(bf.keep, bf.src, bf.packed, bf.cu, bf.gather, bf.o_packed,
                                      bf.dst, H=w.H, scale=w.scale, max_seqlen=bf.max_seqlen,
                                      fused_graph=True, direct=True)
                rec["roundtrip_us"]["pipeline_direct_fused"] = \
                    dp.measure_dispatch(warmup=20, iters=200)["graph_roundtrip"]["p50"]
                dp.close()
            out["B%d_p%03d" % (B, p)] = rec
            print("sweep B=%d p=%03d: attn %.2f us, pipeline %.2f us" %
                  (B, p, rec["attn_us"], rec["pipeline_us"]), file=sys.stderr, flush=True)
            del bf
    return out


def graph_us(call, steps, per_graph=50):
    """Device microseconds per call: `per_graph` back-to-back calls captured in
    one graph, replayed, timed with events on the capturing stream."""
    import torch

    call()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(per_graph):
            call()
    graph.replay()
    torch.cuda.synchronize()
    reps = max(4, min(40, steps // per_graph))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (reps * per_graph)


def _pct(xs):
    xs = np.sort(np.asarray(xs, dtype=np.float64))
    return {"p10": float(np.percentile(xs, 10)), "p50": float(np.percentile(xs, 50)),
            "p90": float(np.percentile(xs, 90)), "n": int(xs.size)}


def stage_samples(bf, hot_samples=100, cold_samples=30, per_graph=20):
    """Per-launch device time of pack, attention and unpack as distributions.

    hot: `hot_samples` samples, each one replay of a graph of `per_graph`
    back-to-back launches between two events (the same graph replayed just
    before, untimed, keeps the GPU busy while the host enqueues, so no host gap
    is timed); per-launch time = elapsed / per_graph.
    cold: `cold_samples` samples of ONE direct launch between two events, each
    after 512 MiB of scratch traffic outside the timed region (about 100 us of
    GPU work, during which the host enqueues the events and the launch, so no
    host gap is timed either), which evicts the L2s and the 256 MB MALL so that
    the stage reads its inputs from HBM:
      cold_write_us: the scratch is written (what a preceding layer leaves: the
        caches full of dirty lines, written back as the stage evicts them);
      cold_read_us: the scratch is read (clean lines: HBM reads only)."""
    import torch

    stages = {"pack": bf.pack, "attn": bf.attn, "unpack": bf.unpack}
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    sink = torch.empty(1, dtype=torch.int64, device="cuda")
    out = {}
    for name, fn in stages.items():
        fn()
        torch.cuda.synchronize()
        g_many = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_many):
            for _ in range(per_graph):
                fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(max(hot_samples, cold_samples))]
        for i in range(hot_samples):
            g_many.replay()
            ev[i][0].record()
            g_many.replay()
            ev[i][1].record()
        torch.cuda.synchronize()
        rec = {"hot_us": _pct([a.elapsed_time(b) * 1e3 / per_graph for a, b in ev[:hot_samples]])}
        # one launch at a time, caches hot: the graph replay before it keeps the
        # GPU busy while the events and the launch are enqueued
        xs = []
        for i in range(hot_samples):
            g_many.replay()
            ev[i][0].record()
            fn()
            ev[i][1].record()
            torch.cuda.synchronize()
            xs.append(ev[i][0].elapsed_time(ev[i][1]) * 1e3)
        rec["hot_single_us"] = _pct(xs)
        for kind in ("write", "read"):
            xs = []
            for i in range(cold_samples):
                if kind == "write":
                    scratch.fill_(i & 0xFF)
                else:
                    torch.sum(scratch.view(torch.int64), dim=0, keepdim=True, out=sink)
                ev[i][0].record()
                fn()
                ev[i][1].record()
                torch.cuda.synchronize()
                xs.append(ev[i][0].elapsed_time(ev[i][1]) * 1e3)
            rec["cold_%s_us" % kind] = _pct(xs)
        out[name] = rec
        del g_many
    del scratch
    return out


def timing_distributions(w_main, main_samples):
    """stage_samples on the headline workload (already taken) and on the DeiT-B
    and B = 256, p = 0 shapes."""
    from ragged_attention_token_amd import workloads as wl

    out = {w_main.name: main_samples}
    for w in (wl.deitb_ragged(64), wl.deitb384(32), wl.deits(256, 0)):
        bf = Bufs(w)
        out[w.name] = stage_samples(bf)
        del bf
    return out


def python_binding_floor(iters=1000):
    """rag_attn at minimal work (B = 1, L = 1) called from Python, then a
    synchronize: wall-clock p10/p50/p90, to set against the C++ round trip of
    the same call (launch + hipStreamSynchronize).  Three forms:
      call_device_sync: the binding's rag_attn (arguments checked and converted
        on every call) + torch.cuda.synchronize();
      plan_stream_sync: a prepared binding.AttnPlan + a synchronize of torch's
        current stream (the C++ figure's form);
      plan_device_sync: the prepared plan + torch.cuda.synchronize()."""
    import torch
    from ragged_attention_token_amd import binding
    from ragged_attention_token_amd import workloads as wl

    bf = Bufs(wl.custom(B=1, N=197, H=6, lengths=[1], seed=0, name="floor_l1"))
    bf.pack()
    torch.cuda.synchronize()
    C, p = bf.w.C, bf.packed
    plan = binding.AttnPlan(p[:, :C], p[:, C:2 * C], p[:, 2 * C:], bf.cu, bf.max_seqlen, bf.o_packed,
                            H=bf.w.H, scale=bf.w.scale)
    stream = torch.cuda.current_stream()
    out = {}
    for name, call, sync in (("call_device_sync", bf.attn, torch.cuda.synchronize),
                             ("plan_stream_sync", plan, stream.synchronize),
                             ("plan_device_sync", plan, torch.cuda.synchronize)):
        for _ in range(100):
            call()
            sync()
        xs = []
        for _ in range(iters):
            t0 = time.perf_counter()
            call()
            sync()
            xs.append((time.perf_counter() - t0) * 1e6)
        out[name] = _pct(xs)
    return out


def serving_summary(sweep_res):
    """The BS = 1-4 half of the metric: per sweep point with B <= 4, the round
    trip (host launch call(s) + synchronize, p50 from C++) of every way to run
    the pass, and the fastest of them."""
    names = {"eager3": "pack+attn+unpack, three launches from one host call",
             "graph": "the same pass as one hipGraphLaunch",
             "fused": "the pass as one gathered launch",
             "pipeline_direct_fused": "rag_pipeline_launch of a pipeline created with "
                                      "RAG_PIPELINE_DIRECT | RAG_PIPELINE_FUSED (one launch)",
             "padded": "padded attention alone (comparator)"}
    out = {"paths": names}
    for key, rec in sweep_res.items():
        B = int(key.split("_")[0][1:])
        if B > 4:
            continue
        rt = {k: rec["roundtrip_us"][k] for k in names}
        ragged = {k: v for k, v in rt.items() if k != "padded"}
        best = min(ragged, key=ragged.get)
        out[key] = {"roundtrip_us": rt, "fastest_ragged_path": best,
                    "fastest_ragged_vs_padded": rt["padded"] / ragged[best]}
    return out


def copy_reference(w, steps):
    """A plain device-to-device copy of the bytes pack moves (its kept rows read
    and written once, T x 3C elements), timed like the kernels: the practical
    floor of a copy of that size on this GPU, for reading pack's roofline
    fraction.  Captured as 50 back-to-back copies in one graph."""
    import torch

    n = w.T * 3 * w.C * w.elem_bytes // 2
    a = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    b = torch.empty_like(a)
    a.view(torch.int16).random_()
    us = graph_us(lambda: b.copy_(a), steps)
    nbytes = 2 * n * 2
    # one copy at a time between events, caches hot, as the kernels'
    # single_launch_us: a graph of copies replayed just before keeps the GPU
    # busy while the events and the copy are enqueued
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(20):
            b.copy_(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    xs = []
    for _ in range(100):
        g.replay()
        e0.record()
        b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        xs.append(e0.elapsed_time(e1) * 1e3)
    us1 = _pct(xs)["p50"]
    return {"bytes_read_plus_written": nbytes, "us": us, "achieved_GBs": nbytes / us * 1e-3,
            "hbm_frac": nbytes / us * 1e-3 / HBM_PEAK_GBS,
            "single_launch_us": us1, "single_launch_GBs": nbytes / us1 * 1e-3,
            "single_launch_hbm_frac": nbytes / us1 * 1e-3 / HBM_PEAK_GBS}


def tile_list_comparison(steps):
    """rag_attn (grid with one slot per (head, image[, query split])) against
    rag_attn_tiled (the device-built tile list) on the ragged and long-sequence
    shapes and on uniform lengths; the outputs are checked equal bit for bit."""
    import torch
    from ragged_attention_token_amd import binding
    from ragged_attention_token_amd import workloads as wl

    out = {}
    for w in (wl.deitb_ragged(64), wl.deitb384(32), wl.deits(256, 0), wl.deits(256, 800),
              wl.deits(4, 0), wl.deits(1, 500)):
        bf = Bufs(w)
        bf.pack()
        C, p = w.C, bf.packed
        o_t = torch.empty_like(bf.o_packed)

        def attn(o, tiled):
            binding.rag_attn(p[:, :C], p[:, C:2 * C], p[:, 2 * C:], bf.cu, bf.max_seqlen, o, H=w.H,
                             scale=w.scale, tiled=tiled)

        attn(bf.o_packed, False)
        attn(o_t, True)
        torch.cuda.synchronize()
        assert torch.equal(bf.o_packed[:w.T].view(torch.uint8), o_t[:w.T].view(torch.uint8))
        grid = graph_us(lambda: attn(bf.o_packed, False), steps)
        tiled = graph_us(lambda: attn(o_t, True), steps)
        out[w.name] = {"B": w.B, "N": w.N, "H": w.H, "T": w.T, "max_seqlen": bf.max_seqlen,
                       "rag_attn_us": grid, "rag_attn_tiled_us": tiled, "tiled_vs_grid": grid / tiled}
        print("%s: rag_attn %.2f us, rag_attn_tiled %.2f us" % (w.name, grid, tiled), file=sys.stderr,
              flush=True)
        del bf
    return out


def other_shapes(steps):
    """The DeiT-B shapes: highly ragged lengths at N = 197 (B = 64) and the 384x384
    input (N = 577, B = 32, about half the tokens kept): per-launch device time of
    each kernel, the passes, and the padded comparator."""
    import torch
    from ragged_attention_token_amd import workloads as wl

    out = {}
    for w in (wl.deitb_ragged(64), wl.deitb384(32)):
        bf = Bufs(w)
        bf.pipe.launch()
        torch.cuda.synchronize()
        m = bf.pipe.measure_stages(max(50, min(steps, 400)))
        alg = algorithmic(w, 2)
        rec = {"B": w.B, "N": w.N, "H": w.H, "T": w.T, "max_seqlen": bf.max_seqlen,
               "pack_us": m["pack"], "attn_us": m["attn"], "unpack_us": m["unpack"],
               "padded_attn_us": m["padded"], "pipeline_us": m["eager_pass"],
               "fused_pass_us": m["fused_pass"],
               "attn_hbm_frac": alg["attn"] / m["attn"] * 1e-3 / HBM_PEAK_GBS,
               "attn_mfma_frac": alg["attn_flops"] / m["attn"] * 1e-6 / BF16_PEAK_TFLOPS,
               "padded_mfma_frac": alg["padded_flops"] / m["padded"] * 1e-6 / BF16_PEAK_TFLOPS}
        rec["ragged_pipeline_vs_padded_attn"] = m["padded"] / m["eager_pass"]
        out[w.name] = rec
        print("%s: attn %.2f us, pipeline %.2f us, padded %.2f us" %
              (w.name, m["attn"], m["eager_pass"], m["padded"]), file=sys.stderr, flush=True)
        del bf
    return out


def main():
    args = parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this path has no multi-GPU step (images shard "
              "across GPUs with no exchange); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.pmc_calib:
        pmc_calib()
        return
    if args.block_only:
        from ragged_attention_token_amd import workloads as wl
        w384 = wl.deitb384(32)
        print(json.dumps({"vit_block": measure_block(args.steps),
                          "vit_block_384": measure_block(args.steps, w384, "DeiT-B block at 384x384")}))
        return
    from ragged_attention_token_amd import workloads as wl

    if args.workload == "deitb_ragged":
        w = wl.deitb_ragged(64)
    elif args.workload == "deitb384":
        w = wl.deitb384(32)
    else:
        w = wl.deits(args.batch, args.prune)
    if args.workload != "deits" and not args.kernels_only:
        print("--workload %s is a profiling mode: use it with --kernels-only" % args.workload,
              file=sys.stderr)
        sys.exit(2)
    bf = Bufs(w)
    print("workload %s B=%d N=%d H=%d T=%d" % (w.name, w.B, w.N, w.H, w.T), file=sys.stderr,
          flush=True)

    # ---- timed region: K whole passes ------------------------------------------
    # One host call per pass: the three launches from C++ (on ROCm 7.2 this beats
    # one hipGraphLaunch of the captured pass, which is reported beside it).
    step = bf.pipe.launch if args.graph else bf.pipe.launch_eager
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    tokens_per_s = w.T * args.steps / wall
    print("timed %d steps: %.3f ms/step" % (args.steps, ms_per_step), file=sys.stderr, flush=True)
    if args.kernels_only:
        # the same passes as one gathered launch each, so that a profiler run of
        # this mode also sees the fused kernel
        for _ in range(args.steps):
            bf.pipe.launch_fused()
        torch.cuda.synchronize()
        print(json.dumps({"metric": METRIC, "value": tokens_per_s, "unit": "packed tokens/s",
                          "ms_per_step": ms_per_step, "steps": args.steps}))
        return

    # ---- per-kernel durations: HIP events on the launch stream around
    # back-to-back launches issued from C++ (no Python between launches) --------
    it = max(200, min(args.steps, 2000))
    st = bf.pipe.measure_stages(it)
    out_bytes = 2
    alg = algorithmic(w, out_bytes)
    per_kernel = {}
    st["fused"] = st["fused_pass"]
    for name in ("pack", "attn", "unpack", "padded", "fused"):
        us = st[name]
        per_kernel[name] = {"us": us, "alg_bytes": alg[name], "achieved_GBs": alg[name] / us * 1e-3,
                            "hbm_frac": alg[name] / us * 1e-3 / HBM_PEAK_GBS}
    per_kernel["attn"]["alg_flops"] = alg["attn_flops"]
    per_kernel["attn"]["mfma_frac"] = alg["attn_flops"] / st["attn"] * 1e-6 / BF16_PEAK_TFLOPS
    per_kernel["padded"]["alg_flops"] = alg["padded_flops"]
    per_kernel["padded"]["mfma_frac"] = alg["padded_flops"] / st["padded"] * 1e-6 / BF16_PEAK_TFLOPS
    # Per-launch durations as the step sees them: one launch at a time between
    # HIP events with hot caches (p50 of 100).  The kernel trace of the step
    # agrees with these; the back-to-back figures above run lower because
    # consecutive launches of one kernel overlap drain and ramp-up.
    main_samples = stage_samples(bf)
    for name in ("pack", "attn", "unpack"):
        us1 = main_samples[name]["hot_single_us"]["p50"]
        per_kernel[name]["single_launch_us"] = us1
        per_kernel[name]["single_launch_GBs"] = alg[name] / us1 * 1e-3
    dominant = max(("pack", "attn", "unpack"), key=lambda n: per_kernel[n]["single_launch_us"])
    dk = per_kernel[dominant]
    roofline = {"bound": "hbm", "kernel": dominant, "achieved": dk["single_launch_GBs"],
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": dk["single_launch_GBs"] / HBM_PEAK_GBS,
                "traffic": read_traffic(dominant, w.name),
                "alg_bytes_per_launch": alg[dominant], "launch_us": dk["single_launch_us"],
                "launch_timing": "p50 of HIP events around single launches (hot caches) on the "
                                 "launch stream; back_to_back_us is the mean over back-to-back "
                                 "launches of the kernel",
                "back_to_back_us": dk["us"]}

    # ---- host dispatch floor, measured in C++ (minimal work: one image) -------
    floor = {}
    for lab, wf in (("B1_L1", wl.custom(B=1, N=197, H=6, lengths=[1], seed=0, name="floor_l1")),
                    ("B1_p800", wl.deits(1, 800))):
        fb = Bufs(wf)
        floor[lab] = fb.pipe.measure_dispatch(warmup=100, iters=1000)
        del fb

    res = {
        "metric": METRIC, "value": tokens_per_s, "unit": "packed tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "%s: DeiT-S layer (N=197, H=6, d=64), 80%% prune (40 kept incl. "
                               "CLS), B=%d, bf16 in/out, pack+attn+unpack" %
                               (w.name, w.B),
                   "B": w.B, "N": w.N, "H": w.H, "head_dim": w.d, "kept_per_image": int(w.lengths[0]),
                   "T": w.T, "seed": w.seed, "generator": "numpy PCG64; " + w.recipe},
        "rag_attn_latency_us": st["attn"],
        "roofline": roofline,
        "kernels": per_kernel,
        "pipeline_us": {"eager_3_launches": st["eager_pass"], "graph": st["graph_pass"],
                        "fused_1_launch": st["fused_pass"], "padded_attn_only": st["padded"],
                        "ragged_pass_vs_padded_attn": st["padded"] / st["eager_pass"],
                        "fused_pass_vs_padded_attn": st["padded"] / st["fused_pass"]},
        "fused_tokens_per_s": w.T / st["fused_pass"] * 1e6,
        "dispatch_floor_us": floor,
    }
    res["copy_reference"] = copy_reference(w, args.steps)
    res["dispatch_floor_us"]["B1_L1"]["attn_roundtrip_python"] = python_binding_floor()
    res["timing_distributions"] = timing_distributions(w, main_samples)
    res["repack"] = measure_repack(args.steps)
    res["vit_block"] = measure_block(args.steps)
    w384 = wl.deitb384(32)
    res["vit_block_384"] = measure_block(
        args.steps, w384, "DeiT-B block at 384x384 (N=577, C=768, H=12, MLP 4x, random bf16 "
        "weights), B=32, keep 0.5 +- 0.1: %d packed rows vs %d padded rows" % (w384.T, w384.B * w384.N))
    res["deitb_shapes"] = other_shapes(args.steps)
    res["tile_list"] = tile_list_comparison(args.steps)
    if not args.no_sweep:
        res["sweep"] = sweep(args.steps)
        res["serving_bs1_4"] = serving_summary(res["sweep"])
    if not args.no_cpu:
        print("timing the CPU oracle (<= %.0f s)" % args.cpu_seconds, file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
        # the machine's CPU share for one GPU is 16 threads
        nthr = max(1, min(16, len(os.sched_getaffinity(0))))
        res["cpu_baseline_threads"] = cpu_baseline_threads(w, args.cpu_seconds / 2, nthr)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
