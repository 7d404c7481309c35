#!/usr/bin/env python3
"""Benchmark of the chunkwise GLA forward (and the decode step) on one MI355X.

One step = one gla_chunk_fwd call over the training-shape batch B=8, H=16,
T=2048, d_k=d_v=128, bf16 inputs, fp32 final state: all of the forward's
stages run inside that call (gate cumsum, intra-chunk scores, P.V, inter term,
state carry, varlen/tail handling).  Inputs are synthetic (seeded) and resident
in HBM before timing starts.  The decode step (256 sequences x 16 heads,
d=128, 64 consecutive steps) is timed in the same run and reported under
"decode"; the long-context, packed-sequence, backward and Gated DeltaNet
workloads under keys of their own.  The fp64 CPU oracle is timed on the host on the same inputs.

Prints exactly one JSON line on stdout; progress goes to stderr.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GLA fwd tokens/s + TFLOP/s (% MFMA peak), B8 H16 T2048 d128 bf16"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "sub_quadratic_sequence_amd", "csrc")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def fwd_work(B, H, T, dk, dv, C, esz):
    """Algorithmic FLOPs and bytes of one forward call (chunk form).
    FLOPs per token and head: 2C(dk+dv) (scores and P.V over the chunk) +
    4 dk dv (inter term and state update).  Bytes: q, k, g, v read once, o
    written once, the fp32 final state written once."""
    tokens_heads = B * H * T
    flops = tokens_heads * (2 * C * (dk + dv) + 4 * dk * dv)
    bytes_ = tokens_heads * esz * (3 * dk + 2 * dv) + B * H * dk * dv * 4
    return flops, bytes_


def bwd_work(B, H, T, dk, dv, L, esz):
    """FLOPs and bytes of one backward call (gla_chunk_bwd).
    FLOPs, as the two kernels compute them per token and head (16-token
    sub-chunks, L = 16): the score blocks dO V^T and q~ k~^T and the three
    in-sub-chunk products (L (3 dk + 2 dv) multiply-adds), the three inter terms
    of dq, dk, dv and the two carried-state updates (5 dk dv), and the chunk-state
    pass (2 dk dv); times 2.  Bytes, the algorithmic minimum: q, k, g, v, dO read
    once and dq, dk, dg, dv written once (the chunk states the implementation
    stores and re-reads are not counted; the measured traffic shows them)."""
    tokens_heads = B * H * T
    flops = tokens_heads * 2 * (L * (3 * dk + 2 * dv) + 7 * dk * dv)
    bytes_ = tokens_heads * esz * ((3 * dk + 2 * dv) + (3 * dk + dv))
    return flops, bytes_


def gdn_work(B, H, T, dk, dv, C):
    """Gated DeltaNet forward (bf16 q, k, v, o; fp32 g and beta per token).
    FLOPs per token and head, as the chunk form computes them (full C x C
    blocks): Q K^T and K K^T (4 C dk), the triangular solve and P U (2 C dv),
    K S, Q S and the state update (6 dk dv).  Bytes: q, k, v read once, o
    written once, g and beta read once, the fp32 final state written once."""
    tokens_heads = B * H * T
    flops = tokens_heads * (4 * C * dk + 2 * C * dv + 6 * dk * dv)
    bytes_ = tokens_heads * (2 * (2 * dk + 2 * dv) + 8) + B * H * dk * dv * 4
    return flops, bytes_


def decode_work(N, H, dk, dv, esz):
    """Per decode step: 5 dk dv FLOPs per unit; bytes: the fp32 state read and
    written (8 dk dv) plus q, k, g, v in and o out."""
    units = N * H
    return units * 5 * dk * dv, units * (8 * dk * dv + esz * (3 * dk + 2 * dv))


def sources_sha256(csrc=None, header=None):
    """One digest over every source a launch depends on: the HIP kernels, their
    device headers and host-side dispatch (csrc/*.hip, csrc/*.h) and the C
    header, each file's name and bytes in name order."""
    csrc = csrc or CSRC
    header = header or os.path.join(ROOT, "include", "gla.h")
    h = hashlib.sha256()
    files = sorted(f for f in os.listdir(csrc) if f.endswith((".hip", ".h")))
    for p in [os.path.join(csrc, f) for f in files] + [header]:
        h.update(os.path.basename(p).encode() + b"\0")
        with open(p, "rb") as f:
            h.update(f.read())
        h.update(b"\0")
    return h.hexdigest()


def read_summary(name):
    """key = value lines of a committed profile summary (None if absent)."""
    path = os.path.join(PROFILES, name)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        line = line.strip()
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    return kv


def read_traffic(name):
    """HBM traffic per launch measured by rocprofv3 PMC counters, from the
    committed summary, if it was taken on the current sources (null otherwise:
    the counters describe another build)."""
    kv = read_summary(name)
    if kv is None or kv.get("sources_sha256") != sources_sha256():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def read_counters(name):
    """Diagnostic MFMA and instruction counters of the forward kernel from the
    committed rocprofv3 summary, if it was taken on the current sources (null
    otherwise): the MFMA-busy fraction of the SIMDs' cycles, the executed bf16
    MFMA work over the algorithmic FLOPs, and the waves' waiting share."""
    kv = read_summary(name)
    if kv is None or kv.get("sources_sha256") != sources_sha256():
        return None
    try:
        return {"mfma_busy_frac": float(kv["mfma_busy_frac"]),
                "mfma_flop_executed_over_algorithmic": float(kv["executed_over_algorithmic"]),
                "wait_inst_any_over_wave_cycles": float(kv["wait_inst_any_over_wave_cycles"]),
                "lds_bank_conflict_over_active_lds": float(kv["lds_bank_conflict_over_active_lds"]),
                "source": "profiles/" + name}
    except (KeyError, ValueError):
        return None


def time_launches(fn, steps, warmup, torch, preroll_s=0.0):
    """Untimed: fn() repeated for preroll_s seconds (the GPU leaves its idle
    clocks), then `warmup` calls.  Timed: exactly `steps` calls, bracketed by
    device synchronisation, on the wall clock and with HIP events on the
    current stream (the stream the kernels are launched on)."""
    t_end = time.perf_counter() + preroll_s
    while time.perf_counter() < t_end:
        fn()
        torch.cuda.synchronize()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(steps):
        fn()
    ev1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return (t1 - t0) / steps, ev0.elapsed_time(ev1) / 1e3 / steps


def per_launch(fn, n, torch, flush=None, dirty=False):
    """Per-launch HIP-event times (s) of n calls of fn.  With `flush` (an int32
    device buffer four times the size of the 256 MB last-level cache), the buffer
    is read before each call, so that every call starts with its inputs evicted
    from that cache; with dirty=True it is overwritten instead, which also leaves
    the cache full of modified lines that must be written back while the call
    runs."""
    evs = []
    for i in range(n):
        if flush is not None:
            if dirty:
                flush.fill_(i)
            else:
                flush.sum()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        evs.append((e0, e1))
    torch.cuda.synchronize()
    return sorted(a.elapsed_time(b) / 1e3 for a, b in evs)


def bench_forward(args, torch, gla, inputs):
    w = inputs.TRAIN_BF16
    log(f"[bench] forward {w.name}: generating inputs")
    d = inputs.chunk_inputs(w)
    dev = torch.device("cuda:0")
    q, k, v, g = (d[n].to(dev) for n in "qkvg")
    o = torch.empty(w.B, w.H, w.T, w.dv, dtype=torch.bfloat16, device=dev)
    sf = torch.empty(w.B, w.H, w.dk, w.dv, dtype=torch.float32, device=dev)

    def step():
        gla.gla_chunk_fwd(q, k, v, g, out=o, final_state=sf)

    log(f"[bench] forward: {args.preroll:.1f} s pre-roll, {args.warmup} warmup + {args.steps} timed steps")
    wall, gpu = time_launches(step, args.steps, args.warmup, torch, args.preroll)
    flops, nbytes = fwd_work(w.B, w.H, w.T, w.dk, w.dv, 64, 2)
    # launch-time distribution, warm and with the 256 MB last-level cache evicted
    # by a 1 GiB fill before each launch (outside the timed steps above)
    warm = cold = dirty = [gpu]
    if args.only != "pmc":   # counter runs keep to the timed launches
        warm = per_launch(step, 50, torch)
        flush = torch.zeros(1 << 28, dtype=torch.int32, device=dev)
        cold = per_launch(step, 20, torch, flush)
        dirty = per_launch(step, 20, torch, flush, dirty=True)
        del flush
    return dict(w=w, d=d, wall=wall, gpu=gpu, flops=flops, bytes=nbytes, tokens=w.B * w.T,
                warm=warm, cold=cold, dirty=dirty)


def bench_decode(args, torch, gla, inputs):
    w = inputs.DECODE_BF16
    log(f"[bench] decode {w.name}: generating inputs")
    d = inputs.decode_inputs(w)
    dev = torch.device("cuda:0")
    q, k, v, g = (d[n].to(dev) for n in "qkvg")
    st = d["s0"].to(dev)
    o = torch.empty(w.N, w.H, w.dv, dtype=torch.bfloat16, device=dev)
    it = [0]

    def step():
        t = it[0] % w.steps
        gla.gla_recurrent_step(q[t], k[t], v[t], g[t], st, out=o)
        it[0] += 1

    wall, gpu = time_launches(step, w.steps, min(args.warmup, w.steps), torch)
    flops, nbytes = decode_work(w.N, w.H, w.dk, w.dv, 2)
    if args.pmc:   # counter runs keep to the timed steps
        return dict(w=w, wall=wall, gpu=gpu, flops=flops, bytes=nbytes)
    # cold variants: the state evicted from the 256 MB last-level cache before every
    # step, by reading a 1 GiB buffer (clean eviction) or by overwriting it (dirty)
    flush = torch.zeros(1 << 28, dtype=torch.int32, device=dev)

    def cold_run(dirty):
        evs = []
        for t in range(w.steps):
            if dirty:
                flush.fill_(t)
            else:
                flush.sum()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            gla.gla_recurrent_step(q[t], k[t], v[t], g[t], st, out=o)
            e1.record()
            evs.append((e0, e1))
        torch.cuda.synchronize()
        return sorted(a.elapsed_time(b) / 1e3 for a, b in evs)

    cold_steps = cold_run(False)
    dirty_steps = cold_run(True)
    cold = sum(cold_steps) / w.steps
    # reference for a read-modify-write stream of the state's size: a device copy of
    # the same number of bytes (read once, written once), after the same eviction
    src = torch.empty_like(st)
    cps = []
    for t in range(8):
        flush.sum()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        st.copy_(src)
        e1.record()
        cps.append((e0, e1))
    torch.cuda.synchronize()
    copy_t = sum(a.elapsed_time(b) for a, b in cps) / 1e3 / len(cps)
    copy_gbs = 2 * st.numel() * 4 / copy_t / 1e9
    del src, flush
    return dict(w=w, wall=wall, gpu=gpu, cold=cold, cold_median=cold_steps[len(cold_steps) // 2],
                cold_min=cold_steps[0], dirty_median=dirty_steps[len(dirty_steps) // 2],
                flops=flops, bytes=nbytes, copy_gbs=copy_gbs)


def bench_long(args, torch, gla, inputs):
    """The long-context workload (B1 H16 T65536 d128, initial state): 32 work
    items for the whole device unless the sequences are split into segments
    (gla_chunk_fwd_ws), so both paths are timed."""
    w = inputs.LONG_BF16
    log(f"[bench] long context {w.name}: generating inputs")
    d = inputs.chunk_inputs(w)
    dev = torch.device("cuda:0")
    q, k, v, g = (d[n].to(dev) for n in "qkvg")
    s0 = d["s0"].to(dev)
    o = torch.empty(w.B, w.H, w.T, w.dv, dtype=torch.bfloat16, device=dev)
    sf = torch.empty(w.B, w.H, w.dk, w.dv, dtype=torch.float32, device=dev)
    ws = torch.empty(gla.workspace_size(q, v) + 256, dtype=torch.uint8, device=dev)
    res = {False: None}
    for split in ((True,) if args.pmc else (True, False)):
        def step():
            gla.gla_chunk_fwd(q, k, v, g, initial_state=s0, out=o, final_state=sf, split=split,
                              workspace=ws)
        _, t = time_launches(step, 3 if args.pmc else 10, 1 if args.pmc else 2, torch,
                             0.0 if args.pmc else 0.3)
        res[split] = t
    flops, nbytes = fwd_work(w.B, w.H, w.T, w.dk, w.dv, 64, 2)
    nbytes += w.B * w.H * w.dk * w.dv * 4          # the initial state is read too
    return dict(w=w, split=res[True], unsplit=res[False], flops=flops, bytes=nbytes)


def bench_varlen(args, torch, gla, inputs):
    """The packed workload: 16 sequences of 64..4096 tokens (33,280 in all), H16,
    d_k 128, d_v 256, strong gates (most chunks take the sub-chunk pivots)."""
    w = inputs.VARLEN_BF16
    log(f"[bench] packed sequences {w.name}: generating inputs")
    d = inputs.chunk_inputs(w)
    dev = torch.device("cuda:0")
    q, k, v, g = (d[n].to(dev) for n in "qkvg")
    cu = d["cu_seqlens"].to(dev)
    T, nseq = d["T"], d["nseq"]
    o = torch.empty(1, w.H, T, w.dv, dtype=torch.bfloat16, device=dev)
    sf = torch.empty(nseq, w.H, w.dk, w.dv, dtype=torch.float32, device=dev)

    def step():
        gla.gla_chunk_fwd(q, k, v, g, cu_seqlens=cu, out=o, final_state=sf)

    _, t = time_launches(step, 3 if args.pmc else 20, 1 if args.pmc else 3, torch,
                         0.0 if args.pmc else 0.3)
    flops, nbytes = fwd_work(1, w.H, T, w.dk, w.dv, 64, 2)
    nbytes += (nseq - 1) * w.H * w.dk * w.dv * 4   # one final state per sequence
    return dict(w=w, t=t, flops=flops, bytes=nbytes, tokens=T)


def bench_backward(args, torch, gla, inputs, saved=True):
    """The backward pass on the training shape (B8 H16 T2048 d128, no initial
    state, gradient of the outputs only): one gla_chunk_bwd call = the chunk-state
    pass plus the backward kernel."""
    w = inputs.TRAIN_BWD_BF16
    log(f"[bench] backward {w.name}: generating inputs")
    d = inputs.chunk_inputs(w)
    d.update(inputs.upstream_grads(w, d, final=False))
    dev = torch.device("cuda:0")
    q, k, v, g, do = (d[n].to(dev) for n in ("q", "k", "v", "g", "do"))
    outs = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v), torch.empty_like(g))
    ws = torch.empty(gla.bwd_workspace_size(q, v) + 256, dtype=torch.uint8, device=dev)

    def step():
        gla.gla_chunk_bwd(q, k, v, g, do, workspace=ws, out=outs)

    steps = max(1, args.steps // 4)
    wall, gpu = time_launches(step, steps, max(1, args.warmup // 4), torch, args.preroll * 0.5)
    flops, nbytes = bwd_work(w.B, w.H, w.T, w.dk, w.dv, 16, 2)
    res = dict(w=w, wall=wall, gpu=gpu, flops=flops, bytes=nbytes, tokens=w.B * w.T, steps=steps)
    if not saved:
        return res
    # the training step with the forward keeping its chunk states: gla_chunk_fwd_states
    # (the forward plus the states) and gla_chunk_bwd_saved (no state recomputation),
    # against gla_chunk_fwd and gla_chunk_bwd
    o = torch.empty_like(v)
    gla.gla_chunk_fwd_states(q, k, v, g, out=o, chunk_states=ws)

    def fwd_states():
        gla.gla_chunk_fwd_states(q, k, v, g, out=o, chunk_states=ws)

    def bwd_saved():
        gla.gla_chunk_bwd(q, k, v, g, do, workspace=ws, out=outs, states_saved=True)

    def fwd_plain():
        gla.gla_chunk_fwd(q, k, v, g, out=o)

    _, res["fwd_states_gpu"] = time_launches(fwd_states, steps, 2, torch, 0.0)
    _, res["bwd_saved_gpu"] = time_launches(bwd_saved, steps, 2, torch, 0.0)
    _, res["fwd_plain_gpu"] = time_launches(fwd_plain, steps, 2, torch, 0.0)
    return res


def bench_gdn(args, torch, gla, inputs):
    """The Gated DeltaNet chunk forward on the training shape (B8 H16 T2048 d128,
    bf16, fp32 final state): one gdn_chunk_fwd call, one kernel.  The fp64 GDN
    oracle is timed beside it on whole sequences of the same batch (all heads),
    for about 3 s."""
    w = inputs.GDN_TRAIN_BF16
    log(f"[bench] gated deltanet {w.name}: generating inputs")
    d = inputs.gdn_inputs(w)
    dev = torch.device("cuda:0")
    q, k, v, g, beta = (d[n].to(dev) for n in ("q", "k", "v", "g", "beta"))
    o = torch.empty(w.B, w.H, w.T, w.dv, dtype=torch.bfloat16, device=dev)
    sf = torch.empty(w.B, w.H, w.dk, w.dv, dtype=torch.float32, device=dev)

    def step():
        gla.gdn_chunk_fwd(q, k, v, g, beta, out=o, final_state=sf)

    steps = max(1, args.steps // 2)
    wall, gpu = time_launches(step, steps, max(1, args.warmup // 2), torch, args.preroll * 0.5)
    flops, nbytes = gdn_work(w.B, w.H, w.T, w.dk, w.dv, 64)
    res = dict(w=w, wall=wall, gpu=gpu, flops=flops, bytes=nbytes, tokens=w.B * w.T, steps=steps)
    if not args.no_cpu_baseline:
        from oracle import gdn as ogdn

        threads = host_threads()
        el, runs, used = 0.0, 0, 0
        per = w.B if threads > w.H else 1   # whole batch per call when the heads alone leave threads idle
        while el < 3.0 and runs < 8 * w.B // per:   # cycling through the batch
            b = (runs * per) % w.B
            t0 = time.perf_counter()
            _, _, used = ogdn.recurrence(d["q"][b:b + per], d["k"][b:b + per], d["v"][b:b + per],
                                         d["g"][b:b + per], d["beta"][b:b + per], nthreads=threads,
                                         return_threads=True)
            el += time.perf_counter() - t0
            runs += 1
        res["oracle"] = {"value": runs * per * w.T / el, "unit": "tokens/s", "cores": used,
                         "kind": "oracle",
                         "sample": f"{runs} calls x {per} sequences x {w.H} heads x {w.T} tokens of "
                                   "the same batch (fp64 GDN token recurrence, OpenMP over units)",
                         "seconds": round(el, 3), "host": host_info()}
    return res


def host_threads():
    """CPU threads this process may use: the CPUs it is allowed to run on,
    capped by OMP_NUM_THREADS when the environment sets it (the host's share
    of CPUs for this job)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, n)


def host_info():
    """The host CPU model and counts, reported beside the oracle's rate."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = None
    return {"cpu_model": model, "host_cpus": os.cpu_count(), "cpus_allowed": affinity,
            "omp_num_threads_env": os.environ.get("OMP_NUM_THREADS")}


def _time_oracle(oracle, w, d, threads, min_seconds, max_runs, per_call):
    """Groups of per_call whole sequences of the batch (all heads) through the
    fp64 oracle, cycling through the batch, until at least min_seconds of
    oracle time (and one call) have passed."""
    done_tokens, elapsed, used, n = 0, 0.0, 0, 0
    while (elapsed < min_seconds or n == 0) and n < max_runs:
        b = (n * per_call) % w.B
        sl = slice(b, b + per_call)
        t0 = time.perf_counter()
        _, _, used = oracle.recurrence(d["q"][sl], d["k"][sl], d["v"][sl], d["g"][sl],
                                       nthreads=threads, return_threads=True)
        elapsed += time.perf_counter() - t0
        done_tokens += w.T * per_call
        n += 1
    return done_tokens, elapsed, used, n


def cpu_baseline(fwd, min_seconds=12.0, max_passes=64, one_thread_seconds=3.0):
    """The fp64 oracle as it stands, on the host, on the forward workload's own
    inputs: whole sequences (all heads, all tokens) of the batch are run, cycling
    through the batch, until at least min_seconds of oracle time have passed; then
    the same on one thread for at least one_thread_seconds."""
    import oracle

    w, d = fwd["w"], fwd["d"]
    threads = host_threads()
    oracle.build(force=False)
    # the whole batch per call (B x H independent units), so every thread has work
    done_tokens, elapsed, used, n = _time_oracle(oracle, w, d, threads, min_seconds,
                                                 max_passes, w.B)
    sample = (f"{n} passes over the whole batch ({w.B} sequences x {w.H} heads x {w.T} tokens) of "
              f"the same workload (fp64 token recurrence, OpenMP over the {w.B * w.H} units, "
              f"final state kept)")
    t1, e1, u1, n1 = _time_oracle(oracle, w, d, 1, one_thread_seconds, max_passes * w.B, 1)
    return {"value": done_tokens / elapsed, "unit": "tokens/s", "cores": used, "kind": "oracle",
            "sample": sample, "seconds": round(elapsed, 3), "host": host_info(),
            "one_thread": {"value": t1 / e1, "unit": "tokens/s", "cores": u1,
                           "sample": f"{n1} sequence runs x {w.H} heads x {w.T} tokens",
                           "seconds": round(e1, 3)}}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--preroll", type=float, default=1.0,
                    help="seconds of untimed calls before the warm-up steps, so that the GPU "
                         "runs at its working clocks when timing starts")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-long", action="store_true",
                    help="skip the long-context and packed-sequence legs")
    ap.add_argument("--no-bwd", action="store_true", help="skip the backward leg")
    ap.add_argument("--no-gdn", action="store_true", help="skip the Gated DeltaNet leg")
    ap.add_argument("--only", choices=["fwd", "decode", "long", "bwd", "gdn", "copy", "pmc"],
                    default=None,
                    help="profiling runs: launch only this part (copy = 512 MiB calibration "
                         "copy; pmc = copy, then a few launches of every leg: forward, decode, "
                         "long context split, packed sequences, backward, Gated DeltaNet)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); "
              "the library runs on a single GPU and has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch

    from sub_quadratic_sequence_amd import gla, inputs

    gla.load_library()
    args.pmc = args.only == "pmc"
    if args.only in ("copy", "pmc"):
        src = torch.ones(512 << 20, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log("[bench] copy calibration: 5 x 512 MiB device-to-device copies done")
        if args.only == "copy":
            return
        # a few launches of every leg, in order: forward, decode, long context (split),
        # packed sequences, backward, Gated DeltaNet
        args.steps, args.warmup, args.preroll = 5, 1, 0.0
        args.no_cpu_baseline = True
        bench_forward(args, torch, gla, inputs)
        bench_decode(args, torch, gla, inputs)
        bench_long(args, torch, gla, inputs)
        bench_varlen(args, torch, gla, inputs)
        args.steps = 12   # the backward and GDN legs run steps/4 and steps/2 launches
        bench_backward(args, torch, gla, inputs, saved=False)
        bench_gdn(args, torch, gla, inputs)
        log("[bench] pmc launches done")
        return
    if args.only == "long":
        lg = bench_long(args, torch, gla, inputs)
        log(f"[bench] long context: {lg['split'] * 1e6:.1f} us split, {lg['unsplit'] * 1e6:.1f} us unsplit")
        return
    if args.only == "bwd":
        bw = bench_backward(args, torch, gla, inputs)
        log(f"[bench] backward {bw['gpu'] * 1e6:.1f} us/call; saved states: forward "
            f"{bw['fwd_states_gpu'] * 1e6:.1f} us (plain {bw['fwd_plain_gpu'] * 1e6:.1f}), backward "
            f"{bw['bwd_saved_gpu'] * 1e6:.1f} us")
        return
    if args.only == "gdn":
        args.no_cpu_baseline = True
        gd = bench_gdn(args, torch, gla, inputs)
        log(f"[bench] gated deltanet {gd['gpu'] * 1e6:.1f} us/call")
        return
    if args.only == "decode":
        dec = bench_decode(args, torch, gla, inputs)
        log(f"[bench] decode warm {dec['gpu'] * 1e6:.1f} us/step, cold {dec['cold'] * 1e6:.1f} us/step")
        return

    fwd = bench_forward(args, torch, gla, inputs)
    t = fwd["gpu"]
    tflops = fwd["flops"] / t / 1e12
    gbs = fwd["bytes"] / t / 1e9
    log(f"[bench] forward: {t * 1e6:.1f} us/launch (events), {fwd['wall'] * 1e6:.1f} us/step (wall), "
        f"{tflops:.1f} TFLOP/s, {gbs:.0f} GB/s; per launch median {fwd['warm'][len(fwd['warm']) // 2] * 1e6:.1f} us "
        f"warm, {fwd['cold'][len(fwd['cold']) // 2] * 1e6:.1f} us with the last-level cache evicted")
    if args.only == "fwd":
        return
    traffic = read_traffic("chunk_fwd_b8h16t2048d128_bf16_traffic.txt")
    out = {
        "metric": METRIC,
        "value": fwd["tokens"] / fwd["wall"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "preroll_s": args.preroll,
        "ms_per_step": fwd["wall"] * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": fwd["w"].name, "B": 8, "H": 16, "T": 2048, "dk": 128, "dv": 128,
                   "chunk": 64, "final_state": True, "initial_state": False},
        "tflop_s": tflops,
        "mfma_peak_frac": tflops / MFMA_BF16_PEAK_TFLOPS,
        "mfma_counters": read_counters("chunk_fwd_b8h16t2048d128_bf16_counters.txt"),
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "gla::chunk_fwd_pipe_kernel<128, kFull, 1> (64-column d_v slice)",
                     "algorithmic_bytes_per_launch": fwd["bytes"],
                     "algorithmic_flops_per_launch": fwd["flops"],
                     "avg_launch_us": t * 1e6},
        "launch_us": {
            "warm_median": fwd["warm"][len(fwd["warm"]) // 2] * 1e6, "warm_min": fwd["warm"][0] * 1e6,
            "cold_llc_median": fwd["cold"][len(fwd["cold"]) // 2] * 1e6,
            "cold_llc_min": fwd["cold"][0] * 1e6,
            "cold_llc_frac_of_hbm": fwd["bytes"] / fwd["cold"][len(fwd["cold"]) // 2] / 1e9 / HBM_PEAK_GBS,
            "cold_dirty_llc_median": fwd["dirty"][len(fwd["dirty"]) // 2] * 1e6,
            "cold_dirty_llc_min": fwd["dirty"][0] * 1e6,
            "note": "per-launch HIP events: 50 warm launches; 20 launches each after reading a 1 GiB "
                    "buffer (cold_llc: inputs evicted from the 256 MB last-level cache, which holds "
                    "clean lines); 20 launches each after overwriting it (cold_dirty_llc: the cache "
                    "also holds 256 MB of modified lines written back during the launch)"},
    }
    if not args.no_decode:
        dec = bench_decode(args, torch, gla, inputs)
        dgbs = dec["bytes"] / dec["gpu"] / 1e9
        cgbs = dec["bytes"] / dec["cold"] / 1e9
        log(f"[bench] decode: {dec['gpu'] * 1e6:.1f} us/step warm ({dgbs:.0f} GB/s), "
            f"{dec['cold'] * 1e6:.1f} us/step cold ({cgbs:.0f} GB/s)")
        out["decode"] = {
            "workload": dec["w"].name, "tokens_per_s": dec["w"].N / dec["wall"],
            "us_per_step": dec["gpu"] * 1e6, "us_per_step_cold_llc": dec["cold"] * 1e6,
            "us_per_step_cold_llc_median": dec["cold_median"] * 1e6,
            "us_per_step_cold_llc_min": dec["cold_min"] * 1e6,
            "us_per_step_cold_dirty_llc_median": dec["dirty_median"] * 1e6,
            "roofline": {"bound": "hbm", "achieved": dgbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": dgbs / HBM_PEAK_GBS, "achieved_cold_llc": cgbs,
                         "frac_cold_llc": cgbs / HBM_PEAK_GBS,
                         "device_copy_same_bytes_cold_gbs": dec["copy_gbs"],
                         "traffic": read_traffic("recurrent_step_n256h16d128_bf16_traffic.txt"),
                         "kernel": "gla::recurrent_step_kernel<128, 128, BF16>",
                         "algorithmic_bytes_per_launch": dec["bytes"]},
        }
    if not args.no_long:
        lg = bench_long(args, torch, gla, inputs)
        gbs = lg["bytes"] / lg["split"] / 1e9
        log(f"[bench] long context: {lg['split'] * 1e6:.1f} us split, {lg['unsplit'] * 1e6:.1f} us unsplit "
            f"({gbs:.0f} GB/s split)")
        out["long_context"] = {
            "workload": lg["w"].name, "us_per_call_split": lg["split"] * 1e6,
            "us_per_call_unsplit": lg["unsplit"] * 1e6,
            "tokens_per_s": lg["w"].B * lg["w"].T / lg["split"],
            "tflop_s": lg["flops"] / lg["split"] / 1e12,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes_per_call": lg["bytes"],
                         "note": "three kernels per call: segment state pass, segment scan, forward"},
        }
    if not args.no_long:
        vl = bench_varlen(args, torch, gla, inputs)
        gbs = vl["bytes"] / vl["t"] / 1e9
        log(f"[bench] packed sequences: {vl['t'] * 1e6:.1f} us ({gbs:.0f} GB/s)")
        out["packed_sequences"] = {
            "workload": vl["w"].name, "us_per_call": vl["t"] * 1e6,
            "tokens_per_s": vl["tokens"] / vl["t"], "tflop_s": vl["flops"] / vl["t"] / 1e12,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes_per_call": vl["bytes"],
                         "kernel": "gla::chunk_fwd_pipe_kernel<128, kFull, 2> (128-column d_v slice)"},
        }
    if not args.no_bwd:
        bw = bench_backward(args, torch, gla, inputs)
        gbs = bw["bytes"] / bw["gpu"] / 1e9
        tf = bw["flops"] / bw["gpu"] / 1e12
        log(f"[bench] backward: {bw['gpu'] * 1e6:.1f} us/call ({gbs:.0f} GB/s algorithmic, {tf:.1f} TFLOP/s)")
        out["backward"] = {
            "workload": bw["w"].name, "us_per_call": bw["gpu"] * 1e6, "steps": bw["steps"],
            "tokens_per_s": bw["tokens"] / bw["wall"], "tflop_s": tf,
            "mfma_peak_frac": tf / MFMA_BF16_PEAK_TFLOPS,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes_per_call": bw["bytes"],
                         "algorithmic_flops_per_call": bw["flops"],
                         "note": "two kernels per call: chunk-state pass, backward"},
            "saved_states": {
                "note": "training step with the forward keeping its chunk states "
                        "(gla_chunk_fwd_states + gla_chunk_bwd_saved) against recomputing them "
                        "(gla_chunk_fwd + gla_chunk_bwd); HIP-event time per call",
                "fwd_states_us": bw["fwd_states_gpu"] * 1e6, "bwd_saved_us": bw["bwd_saved_gpu"] * 1e6,
                "fwd_us": bw["fwd_plain_gpu"] * 1e6, "bwd_us": bw["gpu"] * 1e6,
                "step_us_saved": (bw["fwd_states_gpu"] + bw["bwd_saved_gpu"]) * 1e6,
                "step_us_recomputed": (bw["fwd_plain_gpu"] + bw["gpu"]) * 1e6},
        }
    if not args.no_gdn:
        gd = bench_gdn(args, torch, gla, inputs)
        gbs = gd["bytes"] / gd["gpu"] / 1e9
        tf = gd["flops"] / gd["gpu"] / 1e12
        log(f"[bench] gated deltanet: {gd['gpu'] * 1e6:.1f} us/call ({gbs:.0f} GB/s, {tf:.1f} TFLOP/s)")
        out["gated_deltanet"] = {
            "workload": gd["w"].name, "us_per_call": gd["gpu"] * 1e6, "steps": gd["steps"],
            "tokens_per_s": gd["tokens"] / gd["wall"], "tflop_s": tf,
            "mfma_peak_frac": tf / MFMA_BF16_PEAK_TFLOPS,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes_per_call": gd["bytes"],
                         "algorithmic_flops_per_call": gd["flops"],
                         "traffic": read_traffic("gdn_fwd_b8h16t2048d128_bf16.txt"),
                         "kernel": "gla::gdn_chunk_fwd_kernel<128>"},
        }
        if "oracle" in gd:
            out["gated_deltanet"]["cpu_baseline"] = gd["oracle"]
    if not args.no_cpu_baseline:
        log("[bench] timing the fp64 oracle on the host")
        out["cpu_baseline"] = cpu_baseline(fwd)
        log(f"[bench] oracle: {out['cpu_baseline']['value']:.3g} tokens/s on "
            f"{out['cpu_baseline']['cores']} threads, "
            f"{out['cpu_baseline']['one_thread']['value']:.3g} tokens/s on one")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
