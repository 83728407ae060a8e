"""Throughput of the tensor-parallel MLP shard forward on one MI355X.

One step is one pass of the whole per-layer path at the decode shape of a
70B-class MLP (d_model 8192, ffn 28672, SwiGLU, bf16 weights N(0, 0.02), tokens
N(0, 1)): the eight rank shards of tensor-parallel degree 8 (per-rank hidden width
3584, M = 32 tokens) are computed one after another on the GPU, each a
``tp_mlp_shard_fwd`` call (gate/up projection with the fused SiLU-gate epilogue,
then the down projection into an fp32 partial), and ``tp_partials_reduce`` sums the
eight partials.  The eight shards hold 1.41 GB of distinct weights, more than the
256 MB last-level cache, so every step streams its weights from HBM.

The step is captured once in a HIP graph and the timed region replays it back to
back (launch-bound decode steps are run from graphs in practice; the eager step
time is reported next to it).  ``value`` is decode weight bandwidth: bf16 weight
bytes per step / time per step.
The JSON line also carries

* ``roofline``: the dominant kernel (the gate/up projection, 2/3 of the weight
  bytes) timed by HIP events attached to each of its launches (the library's
  timing hook) over the same steps launched eagerly, against the 8 TB/s HBM peak;
* ``prefill``: one rank shard at the prefill shape (M = 8192), TFLOP/s against the
  2.5 PFLOP/s dense bf16 matrix-core peak, with its own per-kernel event timing;
* ``vendor_gemm``: the same two products on torch.matmul (hipBLASLt, plain bf16
  output, no epilogue) on the same GPU, at both shapes, for reference;
* ``tp_sweep``: single-rank shards at tensor-parallel degree 1, 2, 4, 8 (per-rank
  hidden width 28672 / k) and M in {1, 8, 32, 64, 4096}, each against its roofline;
* ``all_shards_m2048``: the eight TP=8 shards and their partials sum at M = 2048;
* ``attention_projections``: the attention block's column-parallel QKV and
  row-parallel output projections of the same model (decode and prefill shapes);
* ``grouped_experts``: the 16 experts of one GPU as one grouped SwiGLU MLP;
* ``reduce_add_rmsnorm``: the partials sum fused with the residual add and RMSNorm
  that follow it, against the same work in two launches;
* ``fp8_partials``: the decode partials quantized to FP8 with per-row scales and
  summed in fp32, against the fp32 sum (time, wire bytes, transport error);
* ``attn_partials_merge``: the decode-context-parallel merge of 8 ranks' attention
  partials (32 tokens x 64 heads, head width 128) on one GPU;
* ``cpu_baseline``: the fp64 oracle on the host cores over a bounded sample of the
  same decode workload, and on a seeded subset of the prefill shard's token rows,
  scaled by M / rows and labelled extrapolated.

Inputs are seeded synthetic tensors (torch CPU generator), copied to the GPU
before the timed region.  Usage: ``python bench.py [--steps K] [--warmup W]``.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 matrix cores, published
D_MODEL, FFN, TP, M_DECODE, M_PREFILL = 8192, 28672, 8, 32, 8192
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


_COMMENT = re.compile(r"//[^\n]*|/\*.*?\*/", re.S)


def kernel_source_hash() -> str:
    """Hash of the kernel sources (comments and layout left out: they change no
    kernel) and build flags, to tell whether stored counter readings still describe
    the kernels that are built."""
    from tensor_mlp_shard_amd import build as b
    h = hashlib.sha256()
    for src in sorted(b.SOURCES) + ["device_common.h", "tpm_internal.h"]:
        with open(os.path.join(b.CSRC, src), encoding="utf-8") as f:
            code = " ".join(_COMMENT.sub(" ", f.read()).split())
        h.update(src.encode() + b"\0" + code.encode())
    h.update(" ".join(b.HIP_FLAGS[:-1]).encode())
    return h.hexdigest()[:16]


def stored_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary, or None if
    there is none or the kernels changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != kernel_source_hash():
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


def _median(v):
    v = sorted(v)
    n = len(v)
    return v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])


def device_peaks(props):
    """The published peaks the fractions use, and the dense bf16 peak that the device's
    own CU count and maximum engine clock give (4096 bf16 flops per clock per CU)."""
    clock_ghz = None
    try:
        # hipDeviceGetAttribute(hipDeviceAttributeClockRate = 5, in kHz) from the HIP runtime
        hip = ctypes.CDLL("libamdhip64.so")
        v = ctypes.c_int(0)
        if hip.hipDeviceGetAttribute(ctypes.byref(v), 5, 0) == 0 and v.value > 0:
            clock_ghz = v.value / 1e6
    except OSError:
        pass
    cus = props.multi_processor_count
    out = {"cus": cus, "hbm_peak_GBs_published": HBM_PEAK_GBS,
           "bf16_peak_TFLOPs_published": BF16_PEAK_TFLOPS}
    if clock_ghz:
        out["max_engine_clock_GHz"] = round(clock_ghz, 3)
        out["bf16_peak_TFLOPs_from_clock"] = round(cus * 4096 * clock_ghz * 1e9 / 1e12, 1)
    return out


class Rank:
    """One rank's shard handle plus the raw C arguments of its fwd call."""

    def __init__(self, tpm, lib, a, b, x, max_tokens):
        import torch
        self.shard = tpm.Shard(a, b, "silu_gate", max_tokens=max_tokens)
        self.out = torch.empty((x.shape[0], D_MODEL), dtype=torch.float32, device=x.device)
        self.args = (ctypes.c_void_p(self.shard.handle), ctypes.c_void_p(x.data_ptr()),
                     ctypes.c_int64(x.shape[0]), ctypes.c_void_p(self.out.data_ptr()))
        self.lib = lib

    def fwd(self, stream_ptr):
        rc = self.lib.tp_mlp_shard_fwd(*self.args, stream_ptr)
        if rc:
            raise RuntimeError("tp_mlp_shard_fwd failed: %d" % rc)


class EventPool:
    """Pre-created timing events, handed to the library's timing hook one call at a
    time; durations are read after the timed region."""

    def __init__(self, n):
        import torch
        self.ev = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for e in self.ev:
            e.record()
        torch.cuda.synchronize()
        self.raw = [ctypes.c_void_p(int(e.cuda_event)) for e in self.ev]
        self.next = 0

    def take4(self):
        i = self.next
        self.next += 4
        return (ctypes.c_void_p * 4)(*self.raw[i:i + 4]), self.ev[i:i + 4]


def decode_workload(tpm, lib, synth, dev):
    import torch
    spec = synth.ModelSpec()
    log("drawing the 70B-class model shards (TP=8) ...")
    a_sh, b_sh = spec.shards(TP)
    x_cpu = synth.tokens(M_DECODE)
    x = x_cpu.to(dev)
    ranks = []
    for a, b in zip(a_sh, b_sh):
        ranks.append(Rank(tpm, lib, a.to(dev), b.to(dev), x, M_DECODE))
    torch.cuda.synchronize()
    z = torch.empty((M_DECODE, D_MODEL), dtype=torch.float32, device=dev)
    parts = (ctypes.c_void_p * TP)(*[r.out.data_ptr() for r in ranks])
    red_args = (parts, ctypes.c_int32(TP), ctypes.c_int64(M_DECODE * D_MODEL), ctypes.c_int32(0),
                ctypes.c_void_p(z.data_ptr()), ctypes.c_int32(0))
    return ranks, red_args, z, (x_cpu, a_sh, b_sh)


def _stream_ptr(stream=None):
    import torch
    st = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(int(st.cuda_stream))


def decode_step(lib, ranks, red_args, stream_ptr, hooks=None):
    """One decode step: the 8 rank shards in turn, then the partials sum."""
    for i, r in enumerate(ranks):
        if hooks is not None:
            lib.tp_mlp_shard_set_timing_events(r.args[0], hooks[i][0], 4)
        r.fwd(stream_ptr)
    rc = lib.tp_partials_reduce(*red_args, stream_ptr)
    if rc:
        raise RuntimeError("tp_partials_reduce failed: %d" % rc)


def run_decode_graph(lib, ranks, red_args, steps, warmup):
    """Capture one decode step in a HIP graph and time `steps` replays of it."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        decode_step(lib, ranks, red_args, _stream_ptr(side))
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        decode_step(lib, ranks, red_args, _stream_ptr())
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return t1 - t0, g


def run_fwd_graph(lib, ranks, reps):
    """Time per tp_mlp_shard_fwd call as the stream sees it (both launches and the gap
    between them): one pass over the ranks captured in a HIP graph, replayed `reps`
    times; replay time / number of ranks."""
    g = _graph_of(lambda sp: [r.fwd(sp) for r in ranks])
    t = _time_graph(g, reps) / len(ranks)
    del g
    return t


def _sleep_cycles_per_ms():
    """Rate of torch's bounded spin kernel (cycles per ms), measured on the device."""
    import torch
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(1000)
    start.record()
    torch.cuda._sleep(2_000_000)
    stop.record()
    torch.cuda.synchronize()
    return 2_000_000 / max(start.elapsed_time(stop), 1e-3)


EAGER_CHUNK = 16         # timed decode steps queued behind one spin kernel
EAGER_HOST_MS = 0.6      # host time to enqueue one event-timed step (generous)


def run_decode_eager(lib, ranks, red_args, steps, warmup):
    """`steps` eager decode steps, every kernel timed by events attached to its launch.

    Returns the wall time of `steps` plain eager steps, and the per-launch durations of
    the gate/up and down kernels.  Enqueuing a step from Python takes longer than the
    GPU needs to run it, so launches issued one by one would each start on an idle
    GPU, unlike the back-to-back kernels of the graph replays in the timed region.
    The timed steps therefore go in chunks queued behind a bounded spin kernel
    (long enough for the host to enqueue the whole chunk), each chunk led by one
    untimed step, so that every timed launch runs right after the previous kernel."""
    import torch
    sp = _stream_ptr()
    for _ in range(warmup):
        decode_step(lib, ranks, red_args, sp)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        decode_step(lib, ranks, red_args, sp)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    pool = EventPool(4 * len(ranks) * steps)
    hooks = [[pool.take4() for _ in ranks] for _ in range(steps)]
    rate = _sleep_cycles_per_ms()
    torch.cuda.synchronize()
    for c0 in range(0, steps, EAGER_CHUNK):
        n = min(EAGER_CHUNK, steps - c0)
        torch.cuda._sleep(int(rate * EAGER_HOST_MS * (n + 1)))
        decode_step(lib, ranks, red_args, sp)
        for st in range(c0, c0 + n):
            decode_step(lib, ranks, red_args, sp, hooks[st])
        for r in ranks:
            lib.tp_mlp_shard_set_timing_events(r.args[0], None, 0)
        torch.cuda.synchronize()
    k1 = [evs[0].elapsed_time(evs[1]) for per_step in hooks for _, evs in per_step]
    k2 = [evs[2].elapsed_time(evs[3]) for per_step in hooks for _, evs in per_step]
    return (t1 - t0), k1, k2


def run_prefill(tpm, lib, synth, dev, iters, warmup):
    import torch
    a, b = synth.ModelSpec().shard(0, TP)
    x = synth.tokens(M_PREFILL).to(dev)
    r = Rank(tpm, lib, a.to(dev), b.to(dev), x, M_PREFILL)
    del a, b
    sp = _stream_ptr()
    for _ in range(warmup):
        r.fwd(sp)
    pool = EventPool(4 * iters)
    hooks = [pool.take4() for _ in range(iters)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for arr, _ in hooks:
        lib.tp_mlp_shard_set_timing_events(r.args[0], arr, 4)
        r.fwd(sp)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    lib.tp_mlp_shard_set_timing_events(r.args[0], None, 0)
    k1 = [e[0].elapsed_time(e[1]) for _, e in hooks]
    k2 = [e[2].elapsed_time(e[3]) for _, e in hooks]
    plan = {k: r.shard.plan[k] for k in ("packed_weight_bytes", "workspace_bytes")}
    r.shard.close()
    return (t1 - t0) / iters, k1, k2, plan


def run_vendor_gemm(synth, dev, host_inputs, reps_decode, reps_prefill):
    """The shard's two products on the vendor GEMM (torch.matmul, which calls hipBLASLt),
    plain bf16 output and no epilogue, on the same GPU, for reference: at the decode
    shape (M = 32) over the 8 ranks' weights in turn, as the decode step streams them,
    and at the prefill shape (M = 8192) on rank 0's weights.  Each product is timed as
    a run of back-to-back calls between two events (time per call); not part of the
    library."""
    import torch
    x_cpu, a_sh, b_sh = host_inputs
    F = FFN // TP
    A = [a.to(dev) for a in a_sh]
    B = [b.to(dev) for b in b_sh]
    g = torch.Generator(device="cpu").manual_seed(4242)

    def per_call(fn, calls, warm):
        for i in range(warm):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(calls):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / calls

    res = {"library": "torch.matmul -> hipBLASLt, bf16 in and out, fp32 accumulation, no epilogue"}
    x = x_cpu.to(dev)
    h = (torch.randn(M_DECODE, F, generator=g) * 0.5).to(torch.bfloat16).to(dev)
    t1 = per_call(lambda i: x @ A[i % TP], reps_decode, 2 * TP)
    t2 = per_call(lambda i: h @ B[i % TP], reps_decode, 2 * TP)
    w1, w2 = D_MODEL * 2 * F * 2, F * D_MODEL * 2
    res["decode_m32"] = {"gate_up_us": round(t1 * 1e6, 2), "down_us": round(t2 * 1e6, 2),
                         "gate_up_GBs_weights": round(w1 / t1 / 1e9, 1),
                         "down_GBs_weights": round(w2 / t2 / 1e9, 1)}
    del x, h
    xp = synth.tokens(M_PREFILL).to(dev)
    hp = (torch.randn(M_PREFILL, F, generator=g) * 0.5).to(torch.bfloat16).to(dev)
    t1 = per_call(lambda i: xp @ A[0], reps_prefill, reps_prefill)
    t2 = per_call(lambda i: hp @ B[0], reps_prefill, reps_prefill)
    f1, f2 = 2 * M_PREFILL * D_MODEL * 2 * F, 2 * M_PREFILL * F * D_MODEL
    res["prefill_m8192"] = {"gate_up_us": round(t1 * 1e6, 1), "down_us": round(t2 * 1e6, 1),
                            "gate_up_TFLOPs": round(f1 / t1 / 1e12, 1),
                            "down_TFLOPs": round(f2 / t2 / 1e12, 1)}
    del xp, hp, A, B
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


SWEEP_TP = (1, 2, 4, 8)
SWEEP_M = (1, 8, 32, 64, 4096)
M_ALL_SHARDS = 2048


def _graph_of(fn):
    """Capture fn(stream_ptr) in a HIP graph (after one eager run on a side stream)."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn(_stream_ptr(side))
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn(_stream_ptr())
    return g


def _repeat(fn, n):
    """fn(stream) n times in a row: small kernels are captured many to a graph, so a
    replay's own launch cost does not hide their duration."""
    def run(sp):
        for _ in range(n):
            fn(sp)
    return run


def _time_graph(g, reps, warmup=3):
    import torch
    for _ in range(warmup):
        g.replay()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(reps):
        g.replay()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) * 1e-3 / reps


def _fractions(flops, nbytes, t):
    t_roof = max(flops / (BF16_PEAK_TFLOPS * 1e12), nbytes / (HBM_PEAK_GBS * 1e9))
    bound = "mfma" if flops / (BF16_PEAK_TFLOPS * 1e12) >= nbytes / (HBM_PEAK_GBS * 1e9) else "hbm"
    return {"bound": bound, "roofline_us": round(t_roof * 1e6, 2),
            "frac": round(t_roof / t, 4)}


def run_sweep(tpm, lib, dev, host_shards8, log_fn=log):
    """Tensor-parallel degree sweep on single-rank shards of the same model, plus the
    eight TP=8 shards and their partials sum at M = 2048.

    For each degree k the k rank shards (together the whole model, 1.41 GB) are
    created, and for each token count M one pass over them (one tp_mlp_shard_fwd per
    rank, ranks in turn so each call streams weights the previous call did not
    touch) is captured in a HIP graph and replayed; the time per call is the pass
    time / k, stream-side (HIP events around the replays), both kernels and the gap
    between them included."""
    import torch
    from tensor_mlp_shard_amd import synth
    a8, b8 = host_shards8
    F8 = FFN // TP
    points, all_shards = [], None
    xs = {M: synth.tokens(M).to(dev) for M in SWEEP_M + (M_ALL_SHARDS,)}
    for k in SWEEP_TP:
        per = TP // k
        F = FFN // k
        shards = []
        for r in range(k):
            ps = range(r * per, (r + 1) * per)
            gate = torch.cat([a8[p][:, :F8] for p in ps], dim=1)
            up = torch.cat([a8[p][:, F8:] for p in ps], dim=1)
            a = torch.cat([gate, up], dim=1).contiguous().to(dev)
            b = torch.cat([b8[p] for p in ps], dim=0).contiguous().to(dev)
            shards.append(tpm.Shard(a, b, "silu_gate", max_tokens=max(SWEEP_M)))
            del a, b, gate, up
        torch.cuda.synchronize()
        w_bytes = D_MODEL * 2 * F * 2 + F * D_MODEL * 2
        for M in SWEEP_M:
            x = xs[M]
            outs = [torch.empty((M, D_MODEL), dtype=torch.float32, device=dev) for _ in range(k)]
            args = [(ctypes.c_void_p(sh.handle), ctypes.c_void_p(x.data_ptr()), ctypes.c_int64(M),
                     ctypes.c_void_p(o.data_ptr())) for sh, o in zip(shards, outs)]

            def one_pass(sp, args=args):
                for a_ in args:
                    rc = lib.tp_mlp_shard_fwd(*a_, sp)
                    if rc:
                        raise RuntimeError("tp_mlp_shard_fwd failed: %d" % rc)
            g = _graph_of(one_pass)
            reps = 4 if M > 64 else max(8, 64 // k)
            t = _time_graph(g, reps) / k
            del g
            flops = 6 * M * D_MODEL * F
            nbytes = w_bytes + M * D_MODEL * 2 + M * D_MODEL * 4
            pt = {"tp": k, "ffn_shard": F, "M": M, "us_per_call": round(t * 1e6, 2),
                  "GBs": round(nbytes / t / 1e9, 1), "TFLOPs": round(flops / t / 1e12, 1)}
            pt.update(_fractions(flops, nbytes, t))
            points.append(pt)
            log_fn("sweep: tp %d M %5d  %9.2f us/call  %7.1f GB/s  %7.1f TFLOP/s  frac %.3f (%s)"
                   % (k, M, pt["us_per_call"], pt["GBs"], pt["TFLOPs"], pt["frac"], pt["bound"]))
            del outs
        if k == TP:
            M = M_ALL_SHARDS
            x = xs[M]
            outs = [torch.empty((M, D_MODEL), dtype=torch.float32, device=dev) for _ in range(k)]
            z = torch.empty((M, D_MODEL), dtype=torch.float32, device=dev)
            args = [(ctypes.c_void_p(sh.handle), ctypes.c_void_p(x.data_ptr()), ctypes.c_int64(M),
                     ctypes.c_void_p(o.data_ptr())) for sh, o in zip(shards, outs)]
            parts = (ctypes.c_void_p * k)(*[o.data_ptr() for o in outs])
            red = (parts, ctypes.c_int32(k), ctypes.c_int64(M * D_MODEL), ctypes.c_int32(0),
                   ctypes.c_void_p(z.data_ptr()), ctypes.c_int32(0))

            def step(sp, args=args, red=red):
                for a_ in args:
                    rc = lib.tp_mlp_shard_fwd(*a_, sp)
                    if rc:
                        raise RuntimeError("tp_mlp_shard_fwd failed: %d" % rc)
                rc = lib.tp_partials_reduce(*red, sp)
                if rc:
                    raise RuntimeError("tp_partials_reduce failed: %d" % rc)
            g = _graph_of(step)
            t = _time_graph(g, 5)
            del g
            flops = 6 * M * D_MODEL * FFN
            red_bytes = (k + 1) * M * D_MODEL * 4
            nbytes = TP * (D_MODEL * 2 * F * 2 + F * D_MODEL * 2) + k * (M * D_MODEL * 6) + red_bytes
            all_shards = {"workload": "8 TP=8 rank shards at M=2048 in turn + tp_partials_reduce "
                                      "of the 8 fp32 partials (HIP-graph replay)",
                          "ms_per_step": round(t * 1e3, 4),
                          "TFLOPs": round(flops / t / 1e12, 1)}
            all_shards.update(_fractions(flops, nbytes, t))
            log_fn("all 8 shards + reduce at M=%d: %.3f ms/step, %.1f TFLOP/s"
                   % (M, t * 1e3, all_shards["TFLOPs"]))
            del outs, z
        for sh in shards:
            sh.close()
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return {"points": points,
            "note": "per call: one rank shard (gate/up + SiLU-gate + down into the fp32 partial) "
                    "at per-rank ffn 28672/tp; frac = roofline time / measured time, roofline "
                    "time = max(flops / 2.5 PFLOP/s, (weights + X + partial bytes) / 8 TB/s); "
                    "calls replayed from a HIP graph over all tp ranks in turn"}, all_shards


def run_attention_projections(tpm, lib, synth, dev):
    """The attention block's projections of all 8 TP=8 ranks of the 70B-class model
    (64 query heads and 8 KV heads of width 128): per rank the column-parallel QKV
    shard [8192 x 1280] (bf16 out) and the row-parallel output shard [1024 x 8192]
    (fp32 partial), one after another, at the decode shape (M = 32: weight GB/s; the
    16 shards hold 302 MB, more than the last-level cache) and at the prefill shape
    (M = 8192, rank 0: TFLOP/s).  Calls captured in HIP graphs."""
    import torch
    spec = synth.AttentionSpec()
    res = {}
    for M in (M_DECODE, M_PREFILL):
        ranks = range(TP) if M == M_DECODE else range(1)
        projs, calls, wbytes, flops = [], [], 0, 0
        x = synth.tokens(M).to(dev)
        for r in ranks:
            wqkv, wo = spec.shard(r, TP)
            pq = tpm.Projection(wqkv.to(dev), max_tokens=M, out_dtype=torch.bfloat16)
            po = tpm.Projection(wo.to(dev), max_tokens=M, out_dtype=torch.float32)
            y = torch.empty(M, wqkv.shape[1], dtype=torch.bfloat16, device=dev)
            a = torch.empty(M, wo.shape[0], dtype=torch.bfloat16, device=dev).normal_()
            p = torch.empty(M, D_MODEL, dtype=torch.float32, device=dev)
            projs += [pq, po]
            calls.append((pq.handle, x, y))
            calls.append((po.handle, a, p))
            wbytes += (wqkv.numel() + wo.numel()) * 2
            flops += 2 * M * (wqkv.numel() + wo.numel())
        vp = ctypes.c_void_p
        args = [(vp(h), vp(xx.data_ptr()), ctypes.c_int64(M), vp(yy.data_ptr()))
                for h, xx, yy in calls]

        def step(sp, args=args):
            for a_ in args:
                rc = lib.tp_proj_fwd(*a_, sp)
                if rc:
                    raise RuntimeError("tp_proj_fwd failed: %d" % rc)
        g = _graph_of(step)
        t = _time_graph(g, 50 if M == M_DECODE else 10)
        del g
        if M == M_DECODE:
            res["decode"] = {"M": M, "ranks": TP, "us_per_step": round(t * 1e6, 2),
                             "weight_bytes": wbytes, "GBs": round(wbytes / t / 1e9, 1),
                             "frac_of_hbm_peak": round(wbytes / t / 1e9 / HBM_PEAK_GBS, 4)}
            log("attention projections, decode (8 ranks QKV + O, M=32): %.2f us, %.1f GB/s"
                % (t * 1e6, wbytes / t / 1e9))
        else:
            res["prefill"] = {"M": M, "ranks": 1, "us_per_step": round(t * 1e6, 2),
                              "flops": flops, "TFLOPs": round(flops / t / 1e12, 1),
                              "frac_of_bf16_peak": round(flops / t / 1e12 / BF16_PEAK_TFLOPS, 4)}
            log("attention projections, prefill (rank 0 QKV + O, M=8192): %.2f us, %.1f TFLOP/s"
                % (t * 1e6, flops / t / 1e12))
        for pr in projs:
            pr.close()
        del x
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    res["note"] = ("Llama-3-70B-style heads: per rank 8 query heads + 1 K + 1 V head of width "
                   "128 (QKV shard [8192 x 1280]) and Wo rows [1024 x 8192]; the attention "
                   "itself is not part of this library")
    return res


def run_grouped_experts(tpm, lib, synth, dev):
    """The 16 experts of one GPU (64 experts, top-2, EP = 4) as one grouped SwiGLU MLP
    (tp_moe_fwd: two launches for all experts) at d_model 8192, expert width 2048,
    with seeded token counts around the page's 64-128 per expert; against one
    tp_mlp_shard_fwd per expert (32 launches).  HIP-graph replays."""
    import torch
    spec = synth.ExpertSpec()
    counts = synth.expert_counts(spec.n_experts)
    T = sum(counts)
    w1, w2 = spec.weights()
    w1d, w2d = w1.to(dev), w2.to(dev)
    del w1, w2
    x = synth.tokens(T).to(dev)
    y = torch.empty(T, D_MODEL, device=dev)
    c = torch.tensor(counts, dtype=torch.int32, device=dev)
    ge = tpm.GroupedExperts(w1d, w2d, "silu_gate", max_tokens=T)
    vp = ctypes.c_void_p

    def grouped(sp):
        rc = lib.tp_moe_fwd(vp(ge.handle), vp(x.data_ptr()), vp(c.data_ptr()), T,
                            vp(y.data_ptr()), sp)
        if rc:
            raise RuntimeError("tp_moe_fwd failed: %d" % rc)
    shards, args, off = [], [], 0
    for e, n in enumerate(counts):
        sh = tpm.Shard(w1d[e], w2d[e], "silu_gate", max_tokens=n)
        shards.append(sh)
        args.append((vp(sh.handle), vp(x[off].data_ptr()), ctypes.c_int64(n),
                     vp(y[off].data_ptr())))
        off += n

    def per_expert(sp):
        for a_ in args:
            rc = lib.tp_mlp_shard_fwd(*a_, sp)
            if rc:
                raise RuntimeError("tp_mlp_shard_fwd failed: %d" % rc)
    gg, gp = _graph_of(grouped), _graph_of(per_expert)
    t_g, t_p = _time_graph(gg, 10), _time_graph(gp, 10)
    del gg, gp
    for sh in shards:
        sh.close()
    ge.close()
    F = spec.ffn_expert
    wbytes = spec.n_experts * (D_MODEL * 2 * F + F * D_MODEL) * 2
    flops = 6 * T * D_MODEL * F
    nbytes = wbytes + T * D_MODEL * 2 + T * D_MODEL * 4
    out = {"experts": spec.n_experts, "d_model": D_MODEL, "ffn_expert": F, "tokens": T,
           "counts": counts, "grouped_us": round(t_g * 1e6, 2),
           "per_expert_launches_us": round(t_p * 1e6, 2),
           "TFLOPs": round(flops / t_g / 1e12, 1), "weight_GBs": round(wbytes / t_g / 1e9, 1)}
    out.update(_fractions(flops, nbytes, t_g))
    log("grouped experts (16 x d 8192 x F 2048, %d tokens): grouped %.1f us, per-expert "
        "launches %.1f us, %.1f TFLOP/s, %.1f GB/s weights, frac %.3f (%s)"
        % (T, t_g * 1e6, t_p * 1e6, flops / t_g / 1e12, wbytes / t_g / 1e9, out["frac"],
           out["bound"]))
    del w1d, w2d, x, y
    torch.cuda.empty_cache()
    return out


def run_reduce_norm(lib, dev, reps=200):
    """The step after the all-reduce: the 8 fp32 rank partials summed, the residual
    added and RMSNorm applied, in one kernel (tp_partials_reduce_add_rmsnorm), against
    the same work as two launches (tp_partials_reduce, then the fused call with k = 1
    on the sum).  Residual, gamma and y in bf16, eps 1e-5; many calls per HIP graph."""
    import torch
    out = []
    for rows in (M_DECODE, 2048):
        g = torch.Generator().manual_seed(rows)
        parts = [torch.randn(rows, D_MODEL, generator=g).to(dev) for _ in range(TP)]
        res = torch.randn(rows, D_MODEL, generator=g).to(torch.bfloat16).to(dev)
        res_out = torch.empty_like(res)
        gamma = torch.rand(D_MODEL, generator=g).add(0.5).to(torch.bfloat16).to(dev)
        y = torch.empty_like(res)
        z = torch.empty(rows, D_MODEL, dtype=torch.float32, device=dev)
        arr = (ctypes.c_void_p * TP)(*[p.data_ptr() for p in parts])
        one = (ctypes.c_void_p * 1)(z.data_ptr())
        vp = ctypes.c_void_p

        def fused(sp):
            rc = lib.tp_partials_reduce_add_rmsnorm(arr, TP, rows, D_MODEL, 0, vp(res.data_ptr()),
                                                    vp(res_out.data_ptr()), 1,
                                                    vp(gamma.data_ptr()), ctypes.c_float(1e-5),
                                                    vp(y.data_ptr()), 1, sp)
            if rc:
                raise RuntimeError("tp_partials_reduce_add_rmsnorm failed: %d" % rc)

        def unfused(sp):
            rc = lib.tp_partials_reduce(arr, TP, rows * D_MODEL, 0, vp(z.data_ptr()), 0, sp)
            rc = rc or lib.tp_partials_reduce_add_rmsnorm(one, 1, rows, D_MODEL, 0,
                                                          vp(res.data_ptr()),
                                                          vp(res_out.data_ptr()), 1,
                                                          vp(gamma.data_ptr()),
                                                          ctypes.c_float(1e-5), vp(y.data_ptr()),
                                                          1, sp)
            if rc:
                raise RuntimeError("reduce / norm failed: %d" % rc)
        inner = 50 if rows <= 64 else 5
        n = max(4, reps // inner)
        gf, gu = _graph_of(_repeat(fused, inner)), _graph_of(_repeat(unfused, inner))
        t_f, t_u = _time_graph(gf, n) / inner, _time_graph(gu, n) / inner
        del gf, gu
        nbytes = TP * rows * D_MODEL * 4 + 3 * rows * D_MODEL * 2 + D_MODEL * 2
        out.append({"rows": rows, "k": TP, "cols": D_MODEL, "fused_us": round(t_f * 1e6, 2),
                    "two_launch_us": round(t_u * 1e6, 2),
                    "fused_GBs": round(nbytes / t_f / 1e9, 1),
                    "frac_of_hbm_peak": round(nbytes / t_f / 1e9 / HBM_PEAK_GBS, 4),
                    "algorithmic_bytes": nbytes})
        log("reduce+residual+RMSNorm rows %d: fused %.2f us, two launches %.2f us, %.1f GB/s"
            % (rows, t_f * 1e6, t_u * 1e6, nbytes / t_f / 1e9))
        del parts, res, res_out, gamma, y, z
    return {"points": out,
            "note": "8 fp32 partials + bf16 residual -> bf16 residual_out and bf16 y "
                    "(RMSNorm, eps 1e-5); two_launch = tp_partials_reduce to fp32, then the "
                    "same fused call with k = 1; many calls per HIP graph, time per call"}


def run_fp8_partials(lib, dev, reps=200):
    """Low-precision partials: each of the 8 fp32 rank partials of a decode step
    ([32 x 8192]) quantized to FP8 with per-row scales (tp_partials_quantize_fp8),
    then the 8 summed in fp32 (tp_partials_reduce_fp8), against the fp32 partials
    summed directly (tp_partials_reduce), many calls per HIP graph; the transport error is
    the FP8 sum against the fp32 sum, max-abs over RMS."""
    import torch
    rows, cols = M_DECODE, D_MODEL
    g = torch.Generator().manual_seed(17)
    parts = [torch.randn(rows, cols, generator=g).to(dev) for _ in range(TP)]
    qs = [torch.empty(rows, cols, dtype=torch.uint8, device=dev) for _ in range(TP)]
    ss = [torch.empty(rows, dtype=torch.float32, device=dev) for _ in range(TP)]
    z8 = torch.empty(rows, cols, device=dev)
    z32 = torch.empty(rows, cols, device=dev)
    vp = ctypes.c_void_p
    parr = (vp * TP)(*[p.data_ptr() for p in parts])
    qarr = (vp * TP)(*[q.data_ptr() for q in qs])
    sarr = (vp * TP)(*[s.data_ptr() for s in ss])

    def quant(sp):
        for p, q, s in zip(parts, qs, ss):
            rc = lib.tp_partials_quantize_fp8(vp(p.data_ptr()), rows, cols, 0, vp(q.data_ptr()),
                                              vp(s.data_ptr()), sp)
            if rc:
                raise RuntimeError("tp_partials_quantize_fp8 failed: %d" % rc)

    def red8(sp):
        rc = lib.tp_partials_reduce_fp8(qarr, sarr, TP, rows, cols, vp(z8.data_ptr()), 0, sp)
        if rc:
            raise RuntimeError("tp_partials_reduce_fp8 failed: %d" % rc)

    def red32(sp):
        rc = lib.tp_partials_reduce(parr, TP, rows * cols, 0, vp(z32.data_ptr()), 0, sp)
        if rc:
            raise RuntimeError("tp_partials_reduce failed: %d" % rc)
    inner = 25
    gq, g8, g32 = (_graph_of(_repeat(f, inner)) for f in (quant, red8, red32))
    n = max(4, reps // inner)
    t_q = _time_graph(gq, n) / inner / TP
    t_8, t_32 = _time_graph(g8, n) / inner, _time_graph(g32, n) / inner
    del gq, g8, g32
    torch.cuda.synchronize()
    err = float((z8 - z32).abs().max() / z32.pow(2).mean().sqrt())
    out = {"rows": rows, "cols": cols, "k": TP,
           "quantize_us_per_partial": round(t_q * 1e6, 2), "reduce_fp8_us": round(t_8 * 1e6, 2),
           "reduce_fp32_us": round(t_32 * 1e6, 2),
           "wire_bytes_per_partial": {"fp32": rows * cols * 4, "bf16": rows * cols * 2,
                                      "fp8_e4m3_plus_row_scales": rows * cols + rows * 4},
           "transport_err_max_abs_over_rms": round(err, 5),
           "note": "partials N(0,1) fp32; quantize = one partial; reduce_fp8 dequantizes the 8 "
                   "FP8 partials with their row scales and sums in fp32; many calls per HIP "
                   "graph, time per call"}
    log("fp8 partials: quantize %.2f us/partial, reduce fp8 %.2f us, reduce fp32 %.2f us, "
        "err %.4f" % (t_q * 1e6, t_8 * 1e6, t_32 * 1e6, err))
    return out


ATTN_HEADS, HEAD_DIM = 64, 128


def run_attn_merge(tpm, synth, dev, reps=200):
    """Merge of the attention partials of 8 decode-context-parallel ranks for one
    decode step (32 tokens x 64 query heads = 2048 rows, head width 128, fp32 values
    and statistics, fp32 output plus merged statistics), many calls per HIP graph."""
    import torch
    rows, dim, k = M_DECODE * ATTN_HEADS, HEAD_DIM, TP
    vals, maxs, sums = synth.attn_partials(rows, dim, k)
    vals = [v.to(dev) for v in vals]
    maxs = [m.to(dev) for m in maxs]
    sums = [e.to(dev) for e in sums]
    out = torch.empty(rows, dim, device=dev)
    mo = torch.empty(rows, device=dev)
    eo = torch.empty(rows, device=dev)

    def merge(sp):  # the binding launches on torch's current stream (the capture stream)
        tpm.tp_attn_partials_merge(vals, maxs, sums, out, mo, eo)
    inner = 50
    g = _graph_of(_repeat(merge, inner))
    t = _time_graph(g, max(4, reps // inner)) / inner
    del g
    torch.cuda.synchronize()
    nbytes = k * rows * dim * 4 + 2 * k * rows * 4 + rows * dim * 4 + 2 * rows * 4
    gbs = nbytes / t / 1e9
    log("attention partials merge: %.2f us, %.1f GB/s" % (t * 1e6, gbs))
    return {"rows": rows, "dim": dim, "k": k, "us_per_call": round(t * 1e6, 2),
            "algorithmic_bytes": nbytes, "GBs": round(gbs, 1),
            "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "note": "8 ranks' partials (weighted value sums [2048 x 128] fp32, per-row maxima "
                    "and sums of exponentials) merged to the attention output and merged "
                    "statistics; many calls per HIP graph, time per call"}


def cpu_model() -> str:
    """The host CPU's model name from /proc/cpuinfo (empty if unavailable)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


def cpu_baseline(host_inputs, budget_s=12.0, prefill_rows=256):
    """The fp64 oracle on the host over whole decode steps (8 shards at M = 32 plus
    the partials sum) until about `budget_s` seconds of oracle compute have run; then
    the prefill shard (M = 8192) on a seeded sample of `prefill_rows` token rows,
    scaled by M / rows (token rows are independent, so the cost is linear in M) and
    labelled as extrapolated."""
    import numpy as np
    import oracle
    from tensor_mlp_shard_amd import synth
    x, a_sh, b_sh = host_inputs
    X = oracle._f64(x)
    widened = [(oracle._f64(a), oracle._f64(b)) for a, b in zip(a_sh, b_sh)]
    t_total, shards_done, steps_done = 0.0, 0, 0
    while True:
        parts = []
        for A, B in widened:
            P, dt = oracle.timed_shard_forward(X, A, B, "silu_gate")
            parts.append(P)
            t_total += dt
            shards_done += 1
        t0 = time.perf_counter()
        oracle.partials_sum(parts)
        t_total += time.perf_counter() - t0
        steps_done += 1
        if t_total >= budget_s or steps_done >= 40:
            break
    weight_bytes = sum(a.shape[0] * a.shape[1] * 2 + b.shape[0] * b.shape[1] * 2
                       for a, b in zip(a_sh, b_sh))
    per_step = t_total / steps_done
    # prefill: rank 0's shard, the same seeded rows the prefill parity test samples
    rows = synth.sample_rows(M_PREFILL, prefill_rows)
    xp = synth.tokens(M_PREFILL)[rows]
    _, t_rows = oracle.timed_shard_forward(oracle._f64(xp), widened[0][0], widened[0][1],
                                           "silu_gate")
    F = FFN // TP
    flops_call = 2 * M_PREFILL * D_MODEL * 2 * F + 2 * M_PREFILL * F * D_MODEL
    t_call = t_rows * M_PREFILL / len(rows)
    return {"value": round(weight_bytes / per_step / 1e9, 4), "unit": "GB/s",
            "cores": oracle.num_threads(), "cpu_model": cpu_model(), "kind": "oracle",
            "sample": "%d whole decode step(s): 8 TP=8 rank shards at M=32 + partials sum, "
                      "fp64, %.1f s of oracle compute" % (steps_done, t_total),
            "s_per_step": round(per_step, 4),
            "prefill": {"value": round(flops_call / t_call / 1e12, 6), "unit": "TFLOP/s",
                        "kind": "oracle", "extrapolated": True,
                        "rows_timed": len(rows), "seconds_timed": round(t_rows, 3),
                        "s_per_call_extrapolated": round(t_call, 2),
                        "sample": "prefill shard (rank 0 of TP=8, M=8192): %d seeded token rows "
                                  "timed, scaled by M/rows (rows are independent, cost linear "
                                  "in M)" % len(rows)}}


def calib_copy(dev, nbytes=1 << 30, reps=3):
    """A plain device-to-device copy of known size, for scaling HBM counters."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    log("calibration copy: %d bytes read, %d bytes written, %d times" % (nbytes, nbytes, reps))


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--prefill-iters", type=int, default=20)
    ap.add_argument("--prefill-warmup", type=int, default=20,
                    help="untimed prefill calls first (the clock settles over ~10 ms of load)")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the tensor-parallel degree sweep and the M=2048 eight-shard step")
    ap.add_argument("--no-vendor", action="store_true",
                    help="skip the same products on the vendor GEMM (torch.matmul)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a 1 GiB device copy (for HBM counter scaling)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library has no cross-GPU path (no collectives); "
              "run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import tensor_mlp_shard_amd as tpm
    from tensor_mlp_shard_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    lib = tpm.capi()  # raises if libtpmlp.so is not built: there is no fallback
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)
    log("device:", props.name, "CUs:", props.multi_processor_count)

    ranks, red_args, _, host_inputs = decode_workload(tpm, lib, synth, dev)
    handle_mem = {"decode_rank_shard": {k: ranks[0].shard.plan[k]
                                        for k in ("packed_weight_bytes", "workspace_bytes")}}
    w_bytes_rank = D_MODEL * 2 * (FFN // TP) * 2 + (FFN // TP) * D_MODEL * 2
    w_bytes_step = TP * w_bytes_rank
    log("decode: %d steps (warmup %d), HIP-graph replay ..." % (args.steps, args.warmup))
    elapsed, graph = run_decode_graph(lib, ranks, red_args, args.steps, args.warmup)
    ms_step = elapsed / args.steps * 1e3
    value = w_bytes_step / (elapsed / args.steps) / 1e9
    del graph
    log("decode: the same %d steps launched eagerly, each kernel timed by its own events ..."
        % args.steps)
    elapsed_eager, k1, k2 = run_decode_eager(lib, ranks, red_args, args.steps, args.warmup)
    fwd_s = run_fwd_graph(lib, ranks, args.steps)
    ms_step_eager = elapsed_eager / args.steps * 1e3

    F = FFN // TP
    # algorithmic bytes: the weights and X read once; the H round trip is not credited
    k1_bytes = D_MODEL * 2 * F * 2 + M_DECODE * D_MODEL * 2
    k2_bytes = F * D_MODEL * 2 + M_DECODE * D_MODEL * 4
    k1_ms = sum(k1) / len(k1)
    k2_ms = sum(k2) / len(k2)
    achieved = k1_bytes / (k1_ms * 1e-3) / 1e9
    traffic = stored_traffic("gate_up_decode")
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic,
                "kernel": "k_stream<SILU_GATE> (gate/up projection, decode shard M=32)",
                "algorithmic_bytes_per_launch": k1_bytes, "avg_launch_us": round(k1_ms * 1e3, 2),
                "median_launch_us": round(_median(k1) * 1e3, 2),
                "min_launch_us": round(min(k1) * 1e3, 2), "launches": len(k1),
                "timing": "HIP events attached to each launch (start/end of execution), "
                          "eager pass of the same steps right after the timed replays, queued %d at a time behind a bounded spin kernel so the timed launches run back to back as in the replays" % EAGER_CHUNK}
    down = {"kernel": "k_stream<OUT_F32> (down projection, decode shard M=32)",
            "algorithmic_bytes_per_launch": k2_bytes, "avg_launch_us": round(k2_ms * 1e3, 2),
            "median_launch_us": round(_median(k2) * 1e3, 2),
            "min_launch_us": round(min(k2) * 1e3, 2),
            "achieved_GBs": round(k2_bytes / (k2_ms * 1e-3) / 1e9, 1)}
    shard_us = (k1_ms + k2_ms) * 1e3
    fwd_us = fwd_s * 1e6
    shard_bytes = w_bytes_rank + M_DECODE * D_MODEL * 2 + M_DECODE * D_MODEL * 4
    log("decode: %.3f ms/step (graph), %.3f ms/step (eager), %.1f GB/s weights; "
        "gate/up %.2f us, down %.2f us" % (ms_step, ms_step_eager, value, k1_ms * 1e3, k2_ms * 1e3))

    prefill = None
    if not args.no_prefill:
        for r in ranks:
            r.shard.close()
        ranks = None
        torch.cuda.empty_cache()
        log("prefill: %d iterations ..." % args.prefill_iters)
        t_call, p1, p2, pplan = run_prefill(tpm, lib, synth, dev, args.prefill_iters,
                                                 args.prefill_warmup)
        handle_mem["prefill_rank_shard"] = pplan
        flops1 = 2 * M_PREFILL * D_MODEL * 2 * F
        flops2 = 2 * M_PREFILL * F * D_MODEL
        p1_ms, p2_ms = sum(p1) / len(p1), sum(p2) / len(p2)
        tf = (flops1 + flops2) / t_call / 1e12
        prefill = {"metric": "prefill shard TFLOP/s", "value": round(tf, 1), "unit": "TFLOP/s",
                   "ms_per_call": round(t_call * 1e3, 4),
                   "frac_of_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4),
                   "config": {"workload": "prefill shard: one TP=8 rank, d_model 8192, F 3584, "
                                          "SwiGLU, X [8192 x 8192] bf16"},
                   "roofline": {"bound": "mfma", "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                "kernel": "k_gemm<SILU_GATE> (gate/up projection)",
                                "achieved": round(flops1 / (p1_ms * 1e-3) / 1e12, 1),
                                "frac": round(flops1 / (p1_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                                "avg_launch_us": round(p1_ms * 1e3, 1),
                                "median_launch_us": round(_median(p1) * 1e3, 1),
                                "min_launch_us": round(min(p1) * 1e3, 1),
                                "launches": len(p1), "warmup_calls": args.prefill_warmup,
                                "traffic": stored_traffic("gate_up_prefill")},
                   "down": {"kernel": "k_gemm<OUT_F32> (down projection)",
                            "achieved_TFLOPs": round(flops2 / (p2_ms * 1e-3) / 1e12, 1),
                            "avg_launch_us": round(p2_ms * 1e3, 1)}}
        log("prefill: %.3f ms/call, %.1f TFLOP/s" % (t_call * 1e3, tf))

    vendor = None
    if not args.no_vendor:
        if ranks is not None:
            for r in ranks:
                r.shard.close()
            ranks = None
            torch.cuda.empty_cache()
        log("vendor GEMM on the same products ...")
        vendor = run_vendor_gemm(synth, dev, host_inputs, args.steps, args.prefill_iters)
        log("vendor GEMM: decode gate/up %.2f us, down %.2f us; prefill gate/up %.1f us, down %.1f us"
            % (vendor["decode_m32"]["gate_up_us"], vendor["decode_m32"]["down_us"],
               vendor["prefill_m8192"]["gate_up_us"], vendor["prefill_m8192"]["down_us"]))

    sweep = all_shards = None
    if not args.no_sweep:
        if ranks is not None:
            for r in ranks:
                r.shard.close()
            ranks = None
            torch.cuda.empty_cache()
        log("tensor-parallel degree sweep ...")
        sweep, all_shards = run_sweep(tpm, lib, dev, host_inputs[1:])

    reduce_norm = fp8 = attn = moe = attn_merge = None
    if not args.no_sweep:
        log("attention projections ...")
        attn = run_attention_projections(tpm, lib, synth, dev)
        log("grouped experts ...")
        moe = run_grouped_experts(tpm, lib, synth, dev)
        log("partials sum + residual + RMSNorm ...")
        reduce_norm = run_reduce_norm(lib, dev)
        log("fp8 partials ...")
        fp8 = run_fp8_partials(lib, dev)
        log("attention partials merge ...")
        attn_merge = run_attn_merge(tpm, synth, dev)

    if args.calib_copy:
        calib_copy(dev)

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (fp64 oracle) ...")
        cpu = cpu_baseline(host_inputs)

    line = {
        "metric": "TP-shard MLP fwd decode weight GB/s (%HBM peak)",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "decode: 8 TP=8 rank shards of a 70B-class MLP (d_model 8192, "
                               "ffn 28672, per-rank F 3584, SwiGLU, bf16) at M=32 tokens, "
                               "computed in turn + tp_partials_reduce of the 8 fp32 partials",
                   "global_batch": M_DECODE, "seq_len": 1, "parallelism": "tp8 shards on 1 GPU",
                   "weight_bytes_per_step": w_bytes_step,
                   "launch": "each step's 17 kernels captured once in a HIP graph, timed region "
                             "= back-to-back graph replays"},
        "ms_per_step_eager": round(ms_step_eager, 4),
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "roofline": roofline,
        "down_projection": down,
        "decode_shard": {"avg_us": round(shard_us, 2),
                         "GBs": round(shard_bytes / (shard_us * 1e-6) / 1e9, 1),
                         "algorithmic_bytes": shard_bytes,
                         "fwd_us": round(fwd_us, 2),
                         "fwd_frac_of_hbm_peak": round(shard_bytes / (fwd_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                         "note": "avg_us: the two kernels' own durations (launch-attached "
                                 "events); fwd_us: the whole tp_mlp_shard_fwd as the stream "
                                 "sees it, gap between the launches included: one pass over "
                                 "the 8 ranks captured in a HIP graph, replay time / 8"},
        "prefill": prefill,
        "vendor_gemm": vendor,
        "tp_sweep": sweep,
        "all_shards_m2048": all_shards,
        "attention_projections": attn,
        "grouped_experts": moe,
        "reduce_add_rmsnorm": reduce_norm,
        "fp8_partials": fp8,
        "attn_partials_merge": attn_merge,
        "cpu_baseline": cpu,
        "device": props.name,
        "device_peaks": device_peaks(props),
        "handle_device_bytes": handle_mem,
        "source_hash": kernel_source_hash(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
