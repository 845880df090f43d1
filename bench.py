#!/usr/bin/env python3
"""Benchmark of the KDA hot path on one MI355X.

One step = one kda_chunk_fwd over the 8192-token, 96-head, d = 128 prefill (bf16 q, k, v;
fp32 g, beta and state; entering state h0 ~ N(0, 0.02^2); bf16 output plus fp32 final
state), inputs resident in HBM before the timed region: that is the line's ``value``. The
call takes the path the library recommends for the shape (two launches here, with a
workspace allocated before the timed region); the one-launch path is timed beside it. Six
more legs ride on the same line: ``decode`` (kda_decode_replay on the 256-request, 96-head
speculative verify: window of 7 drafts plus the bonus token, HBM GB/s and latency),
``verify_tiny`` (the same call for 1 request x 12 heads x 4 new tokens, replayed from a HIP
graph), ``decode_sweep`` (the 256 x 96 verify's latency for 1, 2, 4 and 8 new tokens),
``segment_cp`` (kda_segment_cp_fwd on the 262144-token, 12-head ultra-long prefill),
``varlen`` (kda_chunk_fwd on the 64-sequence packed batch with per-sequence h0) and
``raw_prefill`` (kda_chunk_fwd_raw: the prefill shape from raw projections).
Prints ONE JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--legs ...]

The line carries the roofline of the prefill kernel (algorithmic bytes per launch over the
average launch time measured with HIP events on the launch stream), the MFMA rate, the fp64
CPU oracle timed on the host cores, and, when they were taken on the current kernel source,
the HBM bytes read and written per launch from rocprofv3 counters (profiles/).
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
CHUNK = 64
CSRC = os.path.join(ROOT, "linear_attention_recurrence_chunk_amd", "csrc")
KERNEL_SRC = (os.path.join(CSRC, "kda_chunk.hip"), os.path.join(CSRC, "kda_walk.hip"),
              os.path.join(CSRC, "kda_chunk_io.h"))
COUNTERS = os.path.join(ROOT, "profiles", "chunk_two_pass_prefill_8k_counters.txt")
DECODE_SRC = os.path.join(CSRC, "kda_decode.hip")
DECODE_COUNTERS = os.path.join(ROOT, "profiles", "decode_replay_verify_counters.txt")
DECODE_TRACE = os.path.join(ROOT, "profiles", "decode_replay_verify_trace.txt")
# the other legs' counter summaries and the sources that shape their traffic
RAW_COUNTERS = os.path.join(ROOT, "profiles", "raw_prefill_8k_counters.txt")
SEGMENT_SRC = KERNEL_SRC + (os.path.join(CSRC, "kda_segment.hip"),)
SEGMENT_COUNTERS = os.path.join(ROOT, "profiles", "segment_cp_ultralong_256k_counters.txt")
VARLEN_SRC = KERNEL_SRC + (os.path.join(CSRC, "kda_api.hip"),)
VARLEN_COUNTERS = os.path.join(ROOT, "profiles", "varlen_64_counters.txt")
BACKWARD_SRC = (os.path.join(CSRC, "kda_bwd_chunk.hip"),)
BACKWARD_COUNTERS = os.path.join(ROOT, "profiles", "chunk_bwd_8k_counters.txt")


def algorithmic_bytes(T, H, dk, dv, io_bytes, out_bytes, n_seqs=1):
    """Bytes the method must move: q, k, v in, g (fp32) and beta (fp32) in, o out, the fp32
    entering state in and final state out."""
    per_tok_head = io_bytes * (2 * dk + dv) + 4 * dk + 4 + out_bytes * dv
    return T * H * per_tok_head + 2 * n_seqs * H * dk * dv * 4


def algorithmic_flops(T, H, dk, dv):
    """Per token and head: 6 dk dv for the inter-chunk products (W S / K_Gamma S, Q_Gamma S,
    K^T U) plus C (3 dk + 2 dv) for the causal intra-chunk products (A, M, W, U, M U),
    counted triangular-aware."""
    return T * H * (6 * dk * dv + CHUNK * (3 * dk + 2 * dv))


def hbm_roofline(nbytes, ms, traffic=None):
    """The roofline object of a leg bound by HBM: algorithmic bytes over the measured time."""
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": gbs / HBM_PEAK_GBS, "traffic": traffic}


def source_digest(paths=KERNEL_SRC):
    """sha256 of the kernel source file, or of the concatenated files of a tuple."""
    h = hashlib.sha256()
    for path in ((paths,) if isinstance(paths, str) else paths):
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def trace_avg_ms(summary, source):
    """A kernel's average duration (ms) from a committed rocprofv3 trace summary (its
    ``avg_ns:`` line), or None when the kernel source changed since the trace was taken."""
    if not os.path.exists(summary):
        return None
    vals = {}
    with open(summary) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                vals[key.strip()] = val.strip()
    if vals.get("kernel_source_sha256") != source_digest(source):
        return None
    try:
        return float(vals["avg_ns"]) * 1e-6
    except (KeyError, ValueError):
        return None


def counter_traffic(counters=COUNTERS, source=KERNEL_SRC):
    """HBM bytes per step (every launch of one call) from a committed rocprofv3 counter
    summary, or None when the kernel source changed since the counters were taken."""
    if not os.path.exists(counters):
        return None
    vals = {}
    with open(counters) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                vals[key.strip()] = val.strip()
    if vals.get("kernel_source_sha256") != source_digest(source):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(inp, scale):
    """The fp64 C oracle, untuned, on the host cores over the same workload."""
    import numpy as np
    from oracle import c_recurrence_fwd, max_threads
    f32 = lambda t: None if t is None else t.detach().float().cpu().numpy()
    host = {k: f32(inp[k]) for k in ("q", "k", "v", "g", "beta", "h0")}
    threads = max_threads()
    t0 = time.perf_counter()
    c_recurrence_fwd(host["q"], host["k"], host["v"], host["g"], host["beta"], h0=host["h0"],
                     scale=scale, col_block=16)
    dt = time.perf_counter() - t0
    T, H = host["q"].shape[0], host["q"].shape[1]
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    del np
    return {"value": T / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"the whole workload ({T} tokens x {H} heads, fp64 per-token recurrence, "
                      f"{dt:.2f} s on {threads} threads, {cpu_model})"}


FLUSH_BYTES = 512 << 20   # written between timed launches: more than the 256 MB MALL


def make_flush(torch, dev):
    """A 512 MiB device buffer and a function that reads all of it (a sum on the current
    stream), so that no timed launch finds its inputs left in L2 or the MALL by the previous
    work. A read, not a write: the caches are left holding clean lines, so the timed launch
    does not pay for writing back the flush's own data (or the state restore's, which the
    read evicts first)."""
    buf = torch.zeros(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)

    def flush():
        buf.sum()
    return flush


def timed_launches(fn, stream, steps, warmup, before=None, flush=None):
    """Per-launch durations (ms) from HIP events recorded on the launch stream; ``before``
    runs untimed ahead of every launch (e.g. restoring state updated in place), then
    ``flush`` (a cache-flushing write), both outside the events."""
    import torch
    for _ in range(warmup):
        if before:
            before()
        fn()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for i in range(steps):
        if before:
            before()
        if flush:
            flush()
        starts[i].record(stream)
        fn()
        ends[i].record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in zip(starts, ends)]


def decode_bytes(R, H, D, W, n_new, n_acc_total, out_bytes):
    """Bytes the fused verify must move: the fp32 state read once and written twice (accepted
    and bonus states), the convolution tail read and written, the bf16 projected inputs of the
    tokens it replays (q, k, v, g, beta of n_acc accepted drafts per request) and of the new
    window (q, k, v, g, z, beta), the outputs, the taps and the norm weight."""
    state = 3 * R * H * D * D * 4
    tail = 2 * R * H * 3 * D * (W - 1) * 4
    inputs = n_acc_total * H * (4 * D + 1) * 2 + R * n_new * H * (5 * D + 1) * 2
    return state + tail + inputs + R * n_new * H * D * out_bytes + H * 3 * D * W * 4 + D * 4


def bench_decode(kda, wl, torch, dev, stream, steps, warmup, cpu_baseline):
    cfg = wl.CONFIGS["decode_verify"]
    R, H, D, W, n_new = cfg["R"], cfg["H"], cfg["dk"], cfg["conv_width"], cfg["n_new"]
    w = wl.decode_inputs(R=R, H=H, dk=D, dv=D, conv_width=W, n_new=n_new, window=cfg["window"],
                         seed=cfg["seed"], device=dev)
    state = w.state.clone()
    tail = w.conv_tail.clone()
    acc = torch.empty_like(state)
    o = torch.empty(R, n_new, H, D, dtype=torch.bfloat16, device=dev)

    def restore():
        state.copy_(w.state)
        tail.copy_(w.conv_tail)

    def launch():
        kda.decode_replay(state, tail, w.n_acc, w.prev, w.new, w.conv_w, w.norm_w,
                          state_acc=acc, o=o, stream=stream)

    # the state restore writes 1.6 GB just before each launch: a 512 MiB flush after it
    ms = timed_launches(launch, stream, steps, warmup, before=restore, flush=make_flush(torch, dev))
    avg = sum(ms) / len(ms)
    n_acc_total = int(w.n_acc.sum().item())
    nbytes = decode_bytes(R, H, D, W, n_new, n_acc_total, 2)
    gbs = nbytes / (avg * 1e-3) / 1e9
    traced = trace_avg_ms(DECODE_TRACE, DECODE_SRC)
    out = {"workload": f"decode_verify: {R} requests x {H} heads, d_k=d_v={D}, fp32 state, "
                       f"window of {cfg['window'] - 1} drafts + 1 bonus, accepted drafts "
                       f"uniform in 0..{cfg['window'] - 1} (mean {n_acc_total / R:.2f}), "
                       f"conv width {W}, bf16 inputs and output",
           "latency_ms": avg, "min_latency_ms": min(ms),
           "verified_tokens_per_s": R * n_new / (avg * 1e-3),
           "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": gbs / HBM_PEAK_GBS,
                        "traffic": counter_traffic(DECODE_COUNTERS, DECODE_SRC)},
           "algorithmic_bytes_per_launch": nbytes, "kernel": "decode_replay_kernel",
           "cache_flush_bytes": FLUSH_BYTES,
           "rocprof_avg_ms": traced,
           "rocprof_frac": None if traced is None else nbytes / (traced * 1e-3) / 1e9 / HBM_PEAK_GBS,
           "note": "latency_ms: HIP events around each launch, after the state restore and a "
                   "512 MiB cache-flushing read; rocprof_avg_ms: the kernel's average duration "
                   "in the committed rocprofv3 trace of the same bench command (null once the "
                   "kernel source changed since)"}
    if cpu_baseline:
        import numpy as np
        from oracle import kda_oracle as ko
        rs = list(range(4))
        host = lambda x: None if x is None else x[rs].double().cpu().numpy()
        t0 = time.perf_counter()
        ko.decode_replay(host(w.state), host(w.conv_tail), w.n_acc[rs].cpu().numpy(),
                         {k: host(v) for k, v in w.prev.items()},
                         {k: host(v) for k, v in w.new.items()},
                         w.conv_w.double().cpu().numpy(), w.norm_w.double().cpu().numpy())
        dt = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": len(rs) * n_new / dt, "unit": "verified tokens/s",
                               "cores": 1, "kind": "oracle",
                               "sample": f"{len(rs)} requests x {H} heads of the same workload "
                                         f"(fp64 NumPy oracle, {dt:.2f} s)"}
        del np
    return out


def bench_verify_tiny(kda, wl, torch, dev, stream, steps, warmup, per_graph=50):
    """The fused verify at one tensor-parallel rank's share of a single request: 1 request,
    12 heads, d = 128, 4 new tokens (3 drafts + 1 bonus), launched back to back from a
    captured HIP graph so that host launch cost is off the critical path; also the eager
    per-launch duration."""
    R, H, D, W, n_new = 1, 12, 128, 4, 4
    w = wl.decode_inputs(R=R, H=H, dk=D, dv=D, conv_width=W, n_new=n_new, window=n_new, seed=5,
                         device=dev)
    state, tail = w.state.clone(), w.conv_tail.clone()
    acc = torch.empty_like(state)
    o = torch.empty(R, n_new, H, D, dtype=torch.bfloat16, device=dev)

    def launch(s):
        kda.decode_replay(state, tail, w.n_acc, w.prev, w.new, w.conv_w, w.norm_w,
                          state_acc=acc, o=o, stream=s)

    eager = timed_launches(lambda: launch(stream), stream, steps, warmup)
    # the state is updated in place, so back-to-back launches do the same work on evolving
    # values (the delta rule keeps them bounded)
    launch(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    with torch.cuda.graph(graph, stream=cap):
        for _ in range(per_graph):
            launch(torch.cuda.current_stream())
    replay = timed_launches(graph.replay, stream, steps, warmup)
    per_call_us = [1e3 * x / per_graph for x in replay]
    n_acc_total = int(w.n_acc.sum().item())
    nbytes = decode_bytes(R, H, D, W, n_new, n_acc_total, 2)
    avg_us = sum(per_call_us) / len(per_call_us)
    return {"workload": f"verify_tiny: {R} request x {H} heads, d_k=d_v={D}, {n_new} new tokens, "
                        f"{n_acc_total} accepted drafts replayed, conv width {W}",
            "graph_latency_us": avg_us, "graph_min_latency_us": min(per_call_us),
            "launches_per_graph": per_graph,
            "eager_latency_us": 1e3 * sum(eager) / len(eager),
            "achieved_gbs": nbytes / (avg_us * 1e-6) / 1e9,
            "algorithmic_bytes_per_launch": nbytes}


def bench_decode_sweep(kda, wl, torch, dev, stream, steps, warmup, n_news=(1, 2, 4, 8)):
    """Verify latency of the 256-request, 96-head workload as the new-token window grows."""
    cfg = wl.CONFIGS["decode_verify"]
    R, H, D, W = cfg["R"], cfg["H"], cfg["dk"], cfg["conv_width"]
    out = {}
    flush = make_flush(torch, dev)
    for n_new in n_news:
        w = wl.decode_inputs(R=R, H=H, dk=D, dv=D, conv_width=W, n_new=n_new, window=cfg["window"],
                             seed=cfg["seed"], device=dev)
        state, tail = w.state.clone(), w.conv_tail.clone()
        acc = torch.empty_like(state)
        o = torch.empty(R, n_new, H, D, dtype=torch.bfloat16, device=dev)

        def restore():
            state.copy_(w.state)
            tail.copy_(w.conv_tail)

        def launch():
            kda.decode_replay(state, tail, w.n_acc, w.prev, w.new, w.conv_w, w.norm_w,
                              state_acc=acc, o=o, stream=stream)

        ms = timed_launches(launch, stream, steps, warmup, before=restore, flush=flush)
        out[str(n_new)] = sum(ms) / len(ms)
        del w, state, tail, acc, o
    return {"workload": f"decode_verify with n_new in {list(n_news)} (window 8, accepted drafts "
                        "uniform in 0..7)", "latency_ms_by_n_new": out}


def bench_varlen(kda, wl, torch, dev, stream, steps, warmup):
    """kda_chunk_fwd on the 64-sequence packed batch (lengths uniform in [512, 16384], per
    sequence h0, final states written), on the library's automatic path."""
    cfg = wl.CONFIGS["varlen_64"]
    H, dk, dv = cfg["H"], cfg["dk"], cfg["dv"]
    lengths = wl.varlen_lengths(cfg["n_seqs"], cfg["len_lo"], cfg["len_hi"], cfg["seed"])
    inp = wl.prefill_inputs(H=H, dk=dk, dv=dv, dtype=cfg["dtype"], seed=cfg["seed"],
                            h0_std=cfg["h0_std"], lengths=lengths, device=dev)
    q, k, v, g, beta, h0 = (inp[n] for n in ("q", "k", "v", "g", "beta", "h0"))
    cu = inp["cu_seqlens"].to(dev)
    T, N = sum(lengths), len(lengths)
    o = torch.empty(T, H, dv, dtype=torch.bfloat16, device=dev)
    ht = torch.empty(N, H, dk, dv, dtype=torch.float32, device=dev)
    ws_bytes = kda.chunk_fwd_workspace_size(1, T, N, H, dk, dv,
                                            cu_seqlens_host=inp["cu_seqlens"])
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None

    def launch():
        kda.chunk_fwd(q, k, v, g, beta, h0=h0, cu_seqlens=cu, o=o, ht=ht, workspace=ws,
                      stream=stream)

    ms = timed_launches(launch, stream, steps, warmup, flush=make_flush(torch, dev))
    avg = sum(ms) / len(ms)
    nbytes = algorithmic_bytes(T, H, dk, dv, 2, 2, n_seqs=N)
    del inp, q, k, v, g, beta, h0, o, ht, ws
    torch.cuda.empty_cache()
    return {"workload": f"varlen_64: {N} packed sequences, {T} tokens (lengths uniform in "
                        f"[512, 16384]), H={H}, d_k=d_v={dk}, bf16 q/k/v and output, fp32 "
                        "g/beta/state, h0 per sequence, final states written",
            "tokens_per_s": T / (avg * 1e-3), "ms_per_call": avg,
            "achieved_gbs": nbytes / (avg * 1e-3) / 1e9, "peak_gbs": HBM_PEAK_GBS,
            "roofline": hbm_roofline(nbytes, avg, counter_traffic(VARLEN_COUNTERS, VARLEN_SRC)),
            "algorithmic_bytes_per_call": nbytes, "workspace_bytes": ws_bytes,
            "kernels": ("prep pass (chunk kernel) + walk per group of sequences" if ws_bytes
                        else "chunk kernel (one launch)")}


def bench_prefill_f32(kda, wl, torch, dev, stream, steps, warmup):
    """kda_chunk_fwd on the prefill shape (8192 tokens x 96 heads, d = 128) with fp32 inputs
    and output: the 16-token chunk form on fp32 matrix cores (operand pass + walk)."""
    cfg = wl.CONFIGS["prefill_8k"]
    T, H, dk, dv = cfg["T"], cfg["H"], cfg["dk"], cfg["dv"]
    inp = wl.prefill_inputs(T=T, H=H, dk=dk, dv=dv, dtype="f32", seed=cfg["seed"],
                            h0_std=cfg["h0_std"], device=dev)
    q, k, v, g, beta, h0 = (inp[n] for n in ("q", "k", "v", "g", "beta", "h0"))
    o = torch.empty_like(v)
    ht = torch.empty_like(h0)
    ws_bytes = kda.chunk_fwd_workspace_size(1, T, 1, H, dk, dv, io_dtype=kda.KDA_F32)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

    def launch():
        kda.chunk_fwd(q, k, v, g, beta, h0=h0, o=o, ht=ht, workspace=ws, stream=stream)

    ms = timed_launches(launch, stream, steps, warmup, flush=make_flush(torch, dev))
    avg = sum(ms) / len(ms)
    nbytes = algorithmic_bytes(T, H, dk, dv, 4, 4)
    del inp, q, k, v, g, beta, h0, o, ht, ws
    torch.cuda.empty_cache()
    return {"workload": f"prefill_8k in fp32: T={T}, H={H}, d_k=d_v={dk}, fp32 q/k/v, output, "
                        "g/beta/state, with h0 and final state",
            "tokens_per_s": T / (avg * 1e-3), "ms_per_call": avg,
            "roofline": hbm_roofline(nbytes, avg), "algorithmic_bytes_per_call": nbytes,
            "workspace_bytes": ws_bytes,
            "kernels": "cbwd_prep_kernel (per-chunk operand blocks) + c16_prefill_kernel (walk)"}


def bench_raw(kda, wl, torch, dev, stream, steps, warmup):
    """kda_chunk_fwd_raw on the prefill shape (8192 tokens x 96 heads, d = 128) from raw bf16
    projections: short convolution (width 4), SiLU, L2 input norms and gates fused into the
    prep pass, entering conv tails and h0 given."""
    cfg = wl.CONFIGS["prefill_8k"]
    T, H, dk, dv = cfg["T"], cfg["H"], cfg["dk"], cfg["dv"]
    inp = wl.raw_prefill_inputs(T=T, H=H, dk=dk, dv=dv, conv_width=4, seed=cfg["seed"],
                                h0_std=cfg["h0_std"], device=dev)
    o = torch.empty(T, H, dv, dtype=torch.bfloat16, device=dev)
    ht = torch.empty(1, H, dk, dv, dtype=torch.float32, device=dev)
    tail_out = torch.empty_like(inp["conv_tail"])
    need = ctypes_size(kda, T, H, dk, dv)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)

    def launch():
        kda.chunk_fwd_raw(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["conv_w"],
                          conv_tail=inp["conv_tail"], h0=inp["h0"], o=o, ht=ht, workspace=ws,
                          conv_tail_out=tail_out, stream=stream)

    ms = timed_launches(launch, stream, steps, warmup)
    avg = sum(ms) / len(ms)
    # raw bf16 q, k, v, g (4 d) and beta in, o out, conv taps and tails, h0 and final state
    nbytes = (T * H * (2 * 4 * dk + 2 + 2 * dv) + 2 * H * dk * dv * 4
              + 2 * H * (2 * dk + dv) * 3 * 4 + H * (2 * dk + dv) * 4 * 4)
    del inp, o, ht, ws, tail_out
    torch.cuda.empty_cache()
    return {"workload": f"prefill_8k from raw projections: T={T}, H={H}, d_k=d_v={dk}, bf16 raw "
                        "q/k/v/g/beta, conv width 4 with entering tails, SiLU, h0, bf16 output",
            "tokens_per_s": T / (avg * 1e-3), "ms_per_call": avg,
            "achieved_gbs": nbytes / (avg * 1e-3) / 1e9, "peak_gbs": HBM_PEAK_GBS,
            "roofline": hbm_roofline(nbytes, avg, counter_traffic(RAW_COUNTERS)),
            "algorithmic_bytes_per_call": nbytes, "workspace_bytes": need,
            "kernels": "prep pass with the fused token stage (chunk kernel) + walk"}


def ctypes_size(kda, T, H, dk, dv):
    """Workspace bytes of kda_chunk_fwd_raw for one sequence."""
    import ctypes
    out = ctypes.c_size_t(0)
    st = kda.library().kda_chunk_fwd_raw_workspace_size(1, T, 1, H, dk, dv, ctypes.byref(out))
    if st != 0:
        raise RuntimeError(f"kda_chunk_fwd_raw_workspace_size: status {st}")
    return int(out.value)


def backward_bytes(T, H, dk, dv, io_bytes, n_seqs=1):
    """Bytes the backward must move: q, k, v, do (io dtype), g and beta read; dq, dk, dg, dv
    and dbeta written in fp32; h0 and dht read and dh0 written per sequence and head."""
    per_tok = (2 * dk + 2 * dv) * io_bytes + 4 * dk + 4 + 4 * (3 * dk + dv) + 4
    return T * H * per_tok + 3 * n_seqs * H * dk * dv * 4


def bench_backward(kda, wl, torch, dev, stream, steps, warmup):
    """kda_chunk_bwd on the prefill shape (8192 tokens x 96 heads, d = 128, bf16 inputs, h0,
    random do and dht)."""
    cfg = wl.CONFIGS["prefill_8k"]
    T, H, dk, dv = cfg["T"], cfg["H"], cfg["dk"], cfg["dv"]
    inp = wl.prefill_inputs(T=T, H=H, dk=dk, dv=dv, dtype=cfg["dtype"], seed=cfg["seed"],
                            h0_std=cfg["h0_std"], device=dev)
    gen = torch.Generator(device=dev).manual_seed(7)
    do = torch.randn(T, H, dv, device=dev, generator=gen).to(torch.bfloat16)
    dht = torch.randn(1, H, dk, dv, device=dev, generator=gen)
    ws = torch.empty(kda.chunk_bwd_workspace_size(1, T, 1, H, dk, dv), dtype=torch.uint8,
                     device=dev)

    def launch():
        kda.chunk_bwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], do, dht=dht,
                      h0=inp["h0"], workspace=ws, stream=stream)

    ms = timed_launches(launch, stream, steps, warmup, flush=make_flush(torch, dev))
    avg = sum(ms) / len(ms)
    nbytes = backward_bytes(T, H, dk, dv, 2)
    del inp, do, dht, ws
    torch.cuda.empty_cache()
    return {"workload": f"backward of prefill_8k: T={T}, H={H}, d_k=d_v={dk}, bf16 q/k/v/do, "
                        "fp32 g/beta/h0/dht, fp32 gradients",
            "tokens_per_s": T / (avg * 1e-3), "ms_per_call": avg,
            "roofline": hbm_roofline(nbytes, avg,
                                     counter_traffic(BACKWARD_COUNTERS, BACKWARD_SRC)),
            "algorithmic_bytes_per_call": nbytes,
            "kernels": "cbwd_fwd_kernel (forward walk: chunk-entering states) + cbwd_rev_kernel "
                       "(reverse walk: leaving-state gradients, dv, dh0) + cbwd_grad_kernel "
                       "(dq, dk, dbeta, dg per 16-token chunk)"}


def bench_segment(kda, wl, torch, dev, stream, steps, warmup, counts=(0, 64, 256)):
    """kda_segment_cp_fwd on the ultralong workload: the library's automatic segment count
    (the leg's figure) and the two ends of the workload's 64..256 range."""
    cfg = wl.CONFIGS["ultralong_256k"]
    T, H, dk, dv = cfg["T"], cfg["H"], cfg["dk"], cfg["dv"]
    inp = wl.prefill_inputs(T=T, H=H, dk=dk, dv=dv, dtype=cfg["dtype"], seed=cfg["seed"],
                            h0_std=cfg["h0_std"], device=dev)
    q, k, v, g, beta = (inp[n] for n in ("q", "k", "v", "g", "beta"))
    o = torch.empty(T, H, dv, dtype=torch.bfloat16, device=dev)
    ht = torch.empty(1, H, dk, dv, dtype=torch.float32, device=dev)
    flush = make_flush(torch, dev)
    by_count = {}
    for n_seg in counts:
        ws = torch.empty(kda.segment_cp_workspace_size(1, T, 1, H, dk, dv, kda.KDA_BF16, n_seg),
                         dtype=torch.uint8, device=dev)

        def launch():
            kda.segment_cp_fwd(q, k, v, g, beta, o=o, ht=ht, n_segments=n_seg, workspace=ws,
                               stream=stream)

        ms = timed_launches(launch, stream, steps, warmup, flush=flush)
        by_count["auto" if n_seg == 0 else str(n_seg)] = sum(ms) / len(ms)
        del ws
        torch.cuda.empty_cache()
    avg = by_count["auto"]
    nbytes = algorithmic_bytes(T, H, dk, dv, 2, 2)
    del inp, q, k, v, g, beta, o
    torch.cuda.empty_cache()
    return {"workload": f"ultralong_256k: B=1, T={T}, H={H}, d_k=d_v={dk}, bf16 q/k/v and "
                        "output, fp32 g/beta/state, automatic segment count",
            "tokens_per_s": T / (avg * 1e-3), "ms_per_call": avg,
            "ms_per_call_by_segments": by_count,
            "achieved_gbs": nbytes / (avg * 1e-3) / 1e9, "peak_gbs": HBM_PEAK_GBS,
            "roofline": hbm_roofline(nbytes, avg, counter_traffic(SEGMENT_COUNTERS, SEGMENT_SRC)),
            "algorithmic_bytes_per_call": nbytes,
            "kernels": "prep pass (chunk kernel), transition walk, ordered scan, replay walk"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--legs",
                    default="prefill,decode,verify_tiny,decode_sweep,segment,varlen,backward,prefill_f32",
                    help="comma-separated legs to run besides the prefill line (decode, "
                         "verify_tiny, decode_sweep, segment, varlen, raw, backward, "
                         "prefill_f32); the "
                         "prefill leg "
                         "always runs")
    ap.add_argument("--segment-counts", default="0,64,256",
                    help="segment counts the segment leg times (0: the library's automatic "
                         "count, whose figure the leg reports; it must come first)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes --steps times (the "
                         "reference for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build measures one GPU: the KDA recurrence path runs "
                          "on a single MI355X and has no multi-GPU mode (run with --gpus 1)"}))
        sys.exit(2)

    import torch
    import linear_attention_recurrence_chunk_amd as kda
    from linear_attention_recurrence_chunk_amd import workloads as wl

    if args.copy_calibration:
        n = args.copy_calibration // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n * 4, "launches": args.steps}))
        return

    cfg = wl.CONFIGS["prefill_8k"]
    T, H, dk, dv = cfg["T"], cfg["H"], cfg["dk"], cfg["dv"]
    scale = 1.0
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = wl.prefill_inputs(T=T, H=H, dk=dk, dv=dv, dtype=cfg["dtype"], seed=cfg["seed"],
                            h0_std=cfg["h0_std"], device=dev)
    q, k, v, g, beta, h0 = (inp[n] for n in ("q", "k", "v", "g", "beta", "h0"))
    o = torch.empty(T, H, dv, dtype=torch.bfloat16, device=dev)
    ht = torch.empty(1, H, dk, dv, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    # the library's recommended path for this shape: two launches (prep pass over every chunk
    # and head, then the serial walk) when its workspace query returns a size, else one
    ws_bytes = kda.chunk_fwd_workspace_size(1, T, 1, H, dk, dv)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None

    def step():
        kda.chunk_fwd(q, k, v, g, beta, h0=h0, o=o, ht=ht, scale=scale, workspace=ws,
                      stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # per-launch durations with events on the launch stream
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    avg_ms = sum(launch_ms) / len(launch_ms)
    ms_per_step = wall * 1e3 / args.steps

    # the one-launch path on the same inputs, for comparison
    one_ms = timed_launches(
        lambda: kda.chunk_fwd(q, k, v, g, beta, h0=h0, o=o, ht=ht, scale=scale, workspace=None,
                              stream=stream), stream, 5, 1) if ws is not None else launch_ms

    nbytes = algorithmic_bytes(T, H, dk, dv, 2, 2)
    nflops = algorithmic_flops(T, H, dk, dv)
    achieved_gbs = nbytes / (avg_ms * 1e-3) / 1e9
    # the committed counters cover the two-launch path
    traffic = counter_traffic() if ws is not None else None
    line = {
        "metric": "KDA prefill tokens/s (kda_chunk_fwd)",
        "value": T / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded: q, k unit-normalised N(0,1), v N(0,1), "
                "beta = sigmoid(N(0,1)), g = max(-softplus(N(0,1)), -5), h0 N(0, 0.02^2))",
        "config": {"workload": "prefill_8k: B=1, T=8192, H=96, d_k=d_v=128, chunk 64, bf16 "
                               "q/k/v and output, fp32 g/beta/state, with h0 and final state",
                   "global_batch": 1, "seq_len": T, "heads": H, "head_dim": dk,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": achieved_gbs, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved_gbs / HBM_PEAK_GBS,
                     "traffic": traffic},
        "mfma": {"achieved_tflops": nflops / (avg_ms * 1e-3) / 1e12,
                 "peak_tflops_bf16": BF16_PEAK_TFLOPS,
                 "frac": nflops / (avg_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                 "flops_per_launch": nflops, "note": "algorithmic FLOPs (triangular-aware)"},
        "kernel": {"name": ("chunk_fwd_kernel (prep pass) + chunk_walk_kernel" if ws is not None
                            else "chunk_fwd_kernel"),
                   "launches_per_step": 2 if ws is not None else 1,
                   "avg_launch_ms": avg_ms, "min_launch_ms": min(launch_ms),
                   "algorithmic_bytes_per_launch": nbytes,
                   "workspace_bytes": ws_bytes,
                   "one_launch_path_ms": sum(one_ms) / len(one_ms),
                   "note": "avg_launch_ms spans the whole kda_chunk_fwd call (both launches "
                           "of the two-launch path), HIP events on the launch stream"},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(inp, scale)
    legs = set(args.legs.split(","))
    if legs & {"decode", "verify_tiny", "decode_sweep", "segment", "varlen", "raw", "backward",
               "prefill_f32"}:
        del inp, q, k, v, g, beta, h0, o, ht, ws
        torch.cuda.empty_cache()
    if "decode" in legs:
        line["decode"] = bench_decode(kda, wl, torch, dev, stream, args.steps, args.warmup,
                                      not args.no_cpu_baseline)
    if "verify_tiny" in legs:
        line["verify_tiny"] = bench_verify_tiny(kda, wl, torch, dev, stream, args.steps,
                                                args.warmup)
    if "decode_sweep" in legs:
        line["decode_sweep"] = bench_decode_sweep(kda, wl, torch, dev, stream,
                                                  max(3, args.steps // 4), min(args.warmup, 2))
    if "segment" in legs:
        counts = tuple(int(x) for x in args.segment_counts.split(","))
        if not counts or counts[0] != 0:
            raise SystemExit("--segment-counts must start with 0 (the automatic count)")
        line["segment_cp"] = bench_segment(kda, wl, torch, dev, stream,
                                           max(3, args.steps // 4), min(args.warmup, 2), counts)
    if "raw" in legs:
        line["raw_prefill"] = bench_raw(kda, wl, torch, dev, stream, args.steps, args.warmup)
    if "backward" in legs:
        line["backward"] = bench_backward(kda, wl, torch, dev, stream, max(3, args.steps // 4),
                                          min(args.warmup, 1))
    if "prefill_f32" in legs:
        line["prefill_f32"] = bench_prefill_f32(kda, wl, torch, dev, stream, args.steps,
                                                args.warmup)
    if "varlen" in legs:
        line["varlen"] = bench_varlen(kda, wl, torch, dev, stream, max(3, args.steps // 4),
                                      min(args.warmup, 1))
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
