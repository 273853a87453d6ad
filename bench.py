#!/usr/bin/env python3
"""Throughput of one Medusa draft-and-verify step on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
the heads' residual blocks, their LM projection, shortlists + tree, tree
attention, verify logits, acceptance + KV rollback (six library calls, the
fused call sequence of speculative_decoding_heads_amd/step.py).  Default
workload: the Llama-7B shape at batch 1 (hidden 4096, vocab 32000, 4 heads,
64-candidate tree, 32 heads x 128, prefix 2048, bf16, greedy); the batch-16
typical-acceptance variant ("also") and the 128k-vocabulary, 32k-context,
batch-32 workload ("large") are measured too and reported alongside.

Timing: inputs are resident in HBM; W warmup steps, then K timed steps between
two events on the launch stream (synchronised on both sides).  Each step uses
its own seq_len buffer (preset to P), so no reset work runs inside the timed
region.  When a workload's weights+cache are small enough to sit in the
256 MB Infinity Cache across steps, two copies of every input are rotated.
A second pass of K steps records events between the calls for the per-call
times and the roofline of every call; the dominant call (most time among the
calls that move algorithmic bytes) gives `roofline`.

Algorithmic bytes and flops per call are those of the method (the head
weights once, the LM projection once per pass, the prefix and tree K/V and the
tree queries once); logits written by one call and read by the next are not
counted, since they could be fused away.  The shortlist and acceptance calls
move no algorithmic bytes beyond those and are bound by latency.

With --loop S (default 8) the workload also runs as a steady-state loop: S
consecutive steps with the state carried on the device, captured in one HIP
graph and replayed (reported under "loop"; `value` stays the single-step
figure above).

Prints ONE JSON line (rank 0).  --gpus N > 1 exits with a message: the step
runs on one GPU.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import hashlib

METRIC = "Medusa verify steps/sec at 7B shape (bs1, bs16) + % of HBM/MFMA roofline"
PROFILES = os.path.join(ROOT, "profiles")
HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
RIDGE = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)      # flop per byte
CALLS = ["draft_hidden", "draft_lm", "topk_tree", "tree_attn", "verify_lm", "accept_compact"]


def alg_bytes(c):
    """Algorithmic bytes each call must move (whole batch)."""
    e = 2 if c.dtype == "bf16" else 4
    return {
        "draft_hidden": c.K * c.H * c.H * e,
        "draft_lm": c.V * c.H * e,
        "topk_tree": 0,
        "tree_attn": 2 * c.b * c.nkv * (c.P + c.T) * c.d * e + c.b * c.T * c.nq * c.d * e,
        "verify_lm": c.V * c.H * e,
        "accept_compact": 0,
    }


def alg_flops(c):
    return {
        "draft_hidden": 2 * c.b * c.K * c.H * c.H,
        "draft_lm": 2 * c.b * (c.K + 1) * c.H * c.V,
        "topk_tree": 0,
        "tree_attn": 4 * c.b * c.nq * c.T * (c.P + c.T) * c.d,
        "verify_lm": 2 * c.b * c.T * c.H * c.V,
        "accept_compact": 0,
    }


def _enqueue(st, x, step, M, c, ev=None):
    """The six calls of VerifyStep.run (fused path), with optional events
    ev[0..6] around them."""
    def mark(i):
        if ev is not None:
            ev[i].record()
    mark(0)
    if st.draft in ("hydra", "mtp"):   # the whole draft counts as draft_hidden
        if st.draft == "hydra":
            st.draft_hydra(x, step, st.root_mode, st.root)
        else:
            st.draft_mtp(x, step, st.root_mode, st.root)
        mark(1)
        mark(2)
        mark(3)
    else:
        M.medusa_heads_hidden(x["h"], x["W"], st.u, include_base=1)
        mark(1)
        M.medusa_lm_logits(st.u, x["LM"], st.logits, reverse_k=1)
        mark(2)
        _shortlists(st, x, step, M, c)
        mark(3)
    M.medusa_tree_attn(x["Q"], x["Kc"], x["Vc"], x["seq_len"], st.anc, st.O, ws=st.ws_attn)
    mark(4)
    M.medusa_verify_logits(st.O.view(c.b * c.T, c.nq * c.d), x["LM"],
                           st.base_logits.view(c.b * c.T, c.V), st.mode, c.temperature,
                           st.ws_verify)
    mark(5)
    M.medusa_accept_compact(st.base_logits, st.tokens, st.parent, st.depth, c.K, st.mode,
                            c.temperature, c.eps, c.delta, c.seed, step, st.L, st.path,
                            st.acc_tokens, st.bonus, x["Kc"], x["Vc"], x["seq_len"], st.ws_acc,
                            verify_ws=st.ws_verify)
    mark(6)


def _shortlists(st, x, step, M, c):
    if st.plan is not None:
        M.medusa_topk_tree_tables(st.logits, c.k, c.kmax, st.plan[0], st.plan[1], st.root_mode,
                                  c.temperature, c.seed, step, x["seq_len"], st.root, st.idx,
                                  st.val, st.tokens, st.pos, st.parent, st.depth, st.anc,
                                  st.ws_topk)
    else:
        M.medusa_topk_tree(st.logits, c.k, c.kmax, c.N, c.decay.numerator, c.decay.denominator,
                           st.root_mode, c.temperature, c.seed, step, x["seq_len"], st.root, st.idx,
                           st.val, st.tokens, st.pos, st.parent, st.depth, st.anc, st.ws_topk)


def measure(cfg, steps, warmup, rotate=None, log=print, plan=None, draft="medusa"):
    import torch
    from speculative_decoding_heads_amd import medusa as M
    from speculative_decoding_heads_amd.step import VerifyStep, device_inputs
    from speculative_decoding_heads_amd.synth import make_inputs, make_mtp_inputs

    M.lib()
    c = cfg
    t0 = time.time()
    names = ("h", "W", "LM", "Kc", "Vc", "Q") + (("E",) if draft == "hydra" else ())
    host = make_inputs(c, names)
    mtp = make_mtp_inputs(c) if draft == "mtp" else {}
    ws_bytes = sum(v.numel() * v.element_size() for v in list(host.values()) + list(mtp.values()))
    if rotate is None:
        rotate = 2 if ws_bytes < (1 << 30) else 1
    sets = []
    for r in range(rotate):
        x = device_inputs(c, host)
        if mtp:
            x["mtp"] = {n: t.to("cuda") for n, t in mtp.items()}
        sets.append(x)
    del host, mtp
    log(f"[bench] {c.name}: inputs {ws_bytes / 1e6:.1f} MB x {rotate} copies "
        f"({time.time() - t0:.1f}s)")
    st = VerifyStep(c, plan=plan, draft=draft)
    n = warmup + 2 * steps
    seqs = [torch.full((c.b,), c.P, dtype=torch.int32, device="cuda") for _ in range(n)]

    def inputs(i):
        x = dict(sets[i % rotate])
        x["seq_len"] = seqs[i]
        return x

    for i in range(warmup):
        _enqueue(st, inputs(i), i, M, c)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(warmup, warmup + steps):
        _enqueue(st, inputs(i), i, M, c)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps

    # per-call pass: events on the launch stream (torch's current stream, which
    # every call above enqueues on) between the calls
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(CALLS) + 1)]
           for _ in range(steps)]
    for j in range(steps):
        i = warmup + steps + j
        _enqueue(st, inputs(i), i, M, c, evs[j])
    torch.cuda.synchronize()
    per_call = {}
    for k, name in enumerate(CALLS):
        per_call[name] = 1000.0 * sum(e[k].elapsed_time(e[k + 1]) for e in evs) / steps   # us
    del sets, seqs, st
    torch.cuda.empty_cache()
    return ms, per_call


def call_roofline(c, name, us):
    """Roofline entry of one call: algorithmic bytes and flops per launch over
    its event-timed average duration, against the bound its arithmetic
    intensity selects (HBM below the ridge, bf16 MFMA above)."""
    ab, af = alg_bytes(c)[name], alg_flops(c)[name]
    t = us * 1e-6
    if ab == 0 or t <= 0:
        return {"bound": "latency", "avg_launch_us": round(us, 2)}
    gbps = ab / t / 1e9
    tflops = af / t / 1e12
    out = {"avg_launch_us": round(us, 2), "alg_bytes_per_launch": ab, "alg_flops_per_launch": af,
           "hbm_GBps": round(gbps, 1), "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
           "mfma_TFLOPs": round(tflops, 1), "mfma_frac": round(tflops / BF16_PEAK_TFLOPS, 4)}
    if c.dtype == "bf16" and af / ab > RIDGE:
        out.update({"bound": "mfma", "achieved": round(tflops, 2), "peak": BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": out["mfma_frac"]})
    else:
        out.update({"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
                    "unit": "GB/s", "frac": out["hbm_frac"]})
    return out


def summarise(c, ms, per_call):
    """value, per-call times, every call's roofline, the dominant call's roofline."""
    rl = {k: call_roofline(c, k, per_call[k]) for k in CALLS}
    moving = [k for k in CALLS if alg_bytes(c)[k] > 0]
    dom = max(moving, key=lambda k: per_call[k])
    roof = dict(rl[dom])
    roof["kernel"] = dom
    roof["traffic"] = measured_traffic(c.name, dom)
    step_bytes = sum(alg_bytes(c).values())
    step_flops = sum(alg_flops(c).values())
    return {
        "value": round(1000.0 / ms, 2), "ms_per_step": round(ms, 4),
        "roofline": roof, "rooflines": rl,
        "step_alg_bytes": step_bytes, "step_alg_flops": step_flops,
        "step_effective_GBps": round(step_bytes / (ms * 1e-3) / 1e9, 1),
        "step_hbm_frac": round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "per_call_us": {k: round(v, 2) for k, v in per_call.items()},
    }


def measure_loop(cfg, steps_per_graph, replays, warmup_replays=2, log=print):
    """Steady-state loop (VerifyLoop): steps_per_graph consecutive steps with the
    state carried on the device (tree K/V appended behind the accepted prefix,
    next hidden state and root from the previous step), captured once in a HIP
    graph and replayed; the state keeps advancing across replays, so the cache
    holds every replay's steps.  Returns ms per step."""
    import torch
    from speculative_decoding_heads_amd.step import VerifyLoop, device_inputs, loop_inputs
    from speculative_decoding_heads_amd.synth import make_inputs

    c = cfg
    x = device_inputs(c, make_inputs(c))
    total = (warmup_replays + replays) * steps_per_graph
    cap = c.P + total * (c.K + 1) + c.T
    for name in ("Kc", "Vc"):
        big = torch.zeros(c.b, c.nkv, cap, c.d, dtype=x[name].dtype, device="cuda")
        big[:, :, : c.P] = x[name][:, :, : c.P]
        x[name] = big
    Qs, Kn, Vn = loop_inputs(c, steps_per_graph, seed_base=c.index)
    loop = VerifyLoop(c)
    g = loop.capture(x, Qs, Kn, Vn)
    for _ in range(warmup_replays):
        g.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(replays):
        g.replay()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / (replays * steps_per_graph)
    log(f"[bench] {c.name}: loop of {steps_per_graph} steps x {replays} graph replays, "
        f"{ms * 1e3:.1f} us per step, final seq_len {x['seq_len'].tolist()[:4]}")
    return ms


def budget_rates(k):
    """Per-rank acceptance rates standing in for measured ones (no trained heads
    here): head d+1 holds the accepted token in its shortlist with probability
    0.9 - 0.1 d, spread over the ranks geometrically (ratio 1/2).  The full
    7B-shape tree then expects 3.43 tokens per step."""
    q = []
    for d, s in enumerate(k):
        w = [0.5 ** r for r in range(s)]
        q.append([(0.9 - 0.1 * d) * x / sum(w) for x in w])
    return q


def tree_sweep(cfg, sizes, steps, warmup, log=print):
    """The tree budget on the device: for each candidate count N the tree of most
    expected tokens under budget_rates (medusa_tree_plan_rates), its measured
    step rate, and expected tokens per second = expected tokens x steps/s."""
    from speculative_decoding_heads_amd import medusa as M
    q = budget_rates(cfg.k)
    points = []
    for N in sizes:
        par, _, rk, e = M.medusa_tree_plan_rates(cfg.k, N, q)
        c = cfg.with_(N=N)
        ms, _ = measure(c, steps, warmup, None, log, plan=(par, rk))
        points.append({"candidates": N, "nodes": N + 1, "expected_tokens": round(e, 4),
                       "steps_per_s": round(1000.0 / ms, 1),
                       "tokens_per_s": round(e * 1000.0 / ms, 1)})
        log(f"[bench] tree budget N={N}: {e:.3f} tokens/step x {1000.0 / ms:.0f} steps/s")
    best = max(points, key=lambda p: p["tokens_per_s"])
    return {"workload": cfg.name,
            "rates": "synthetic stand-in: head d+1 holds the accepted token with probability "
                     "0.9 - 0.1 d, geometric over ranks (ratio 1/2)",
            "points": points, "best_candidates": best["candidates"],
            "best_tokens_per_s": best["tokens_per_s"]}


def host_identity():
    """CPU model (from /proc/cpuinfo, as lscpu reports it), logical CPUs and
    the CPUs this process may run on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.lower().startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        allowed = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        allowed = os.cpu_count()
    return {"cpu_model": model, "logical_cpus": os.cpu_count(), "cpus_allowed": allowed}


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        return (max([i.get("num_threads", 1) for i in info] or [1]),
                sorted({i.get("internal_api", "?") for i in info}))
    except Exception:
        return None, []


def _oracle_steps(c, f, P, seconds, log, tag):
    from oracle import oracle_step
    done, t0 = 0, time.perf_counter()
    while True:
        oracle_step(f["h"], f["W"], f["LM"], f["Q"], f["Kc"], f["Vc"], P, c.k, c.N, c.decay,
                    c.mode, bf16=(c.dtype == "bf16"), temperature=c.temperature, eps=c.eps,
                    delta=c.delta, seed=c.seed, step=done)
        done += 1
        el = time.perf_counter() - t0
        log(f"[bench] oracle ({tag}) step {done}: {el:.1f}s")
        if el >= seconds or done >= 100:
            return done, el


def cpu_baseline(cfg, seconds, single_seconds, log=print):
    """The oracle (numpy float64) timed on this host on whole steps of the
    workload: once with numpy's BLAS threads as they come, once pinned to one
    core (process affinity one CPU, BLAS limited to one thread)."""
    import numpy as np
    from speculative_decoding_heads_amd.synth import make_inputs
    c = cfg
    host = make_inputs(c)
    f = {k: v.float().numpy().astype(np.float64) for k, v in host.items()}
    del host
    P = np.full(c.b, c.P)
    threads, apis = _blas_threads()
    done, el = _oracle_steps(c, f, P, seconds, log, f"{threads} BLAS threads")
    out = {"value": done / el, "unit": "verify-steps/s", "cores": threads or os.cpu_count(),
           "kind": "oracle",
           "sample": f"{done} full step(s) of the {c.name} workload, float64 numpy, "
                     f"{el:.1f} s wall, numpy BLAS with {threads} threads",
           "host": host_identity(), "blas": apis}
    if single_seconds > 0:
        single = None
        try:
            from threadpoolctl import threadpool_limits
            old = os.sched_getaffinity(0)
            cpu = min(old)
            os.sched_setaffinity(0, {cpu})
            try:
                with threadpool_limits(limits=1):
                    d1, e1 = _oracle_steps(c, f, P, single_seconds, log, "one core")
            finally:
                os.sched_setaffinity(0, old)
            single = {"value": d1 / e1, "unit": "verify-steps/s", "cores": 1,
                      "sample": f"{d1} full step(s), process pinned to CPU {cpu}, "
                                f"BLAS limited to one thread, {e1:.1f} s wall"}
        except Exception as ex:            # affinity or threadpoolctl unavailable
            single = {"error": str(ex)}
        out["single_core"] = single
    return out


def kernel_source_hash(name):
    path = os.path.join(ROOT, "speculative_decoding_heads_amd", "csrc", name)
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic(workload, call):
    """HBM bytes per launch of a call's kernel(s) from the committed counter
    summary (two rocprofv3 --pmc runs, FETCH_SIZE and WRITE_SIZE, scaled by a
    copy of known size), or None when absent or when a kernel source it names
    has changed since."""
    path = os.path.join(PROFILES, f"traffic_{call}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    srcs = t.get("sources") or {t["source"]: t["source_sha256"]}
    if any(kernel_source_hash(s) != h for s, h in srcs.items()):
        return None
    return t["traffic_bytes_per_launch"]


def copy_calibration(mib):
    """One device copy of a known size, for scaling the HBM byte counters."""
    import torch
    n = mib * (1 << 20)
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def stream_read_rates(sizes, copies=3, iters=30, log=print):
    """The library's plain-read yardstick (medusa_stream_read) on buffers of the
    given byte counts: median rate over `iters` calls, each call timed by
    events on the launch stream, `copies` buffers rotated so the last-level
    cache cannot serve a repeat.  Returns {bytes: GB/s}."""
    import torch
    from speculative_decoding_heads_amd import medusa as M
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = {}
    for nbytes in sorted(set(sizes)):
        n16 = (nbytes + 15) // 16
        bufs = [torch.ones(n16 * 4, dtype=torch.int32, device="cuda") for _ in range(copies)]
        for i in range(6):
            M.medusa_stream_read(bufs[i % copies], sink)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(iters)]
        for i, (a, b) in enumerate(ev):
            a.record()
            M.medusa_stream_read(bufs[i % copies], sink)
            b.record()
        torch.cuda.synchronize()
        ts = sorted(a.elapsed_time(b) * 1e-3 for a, b in ev)
        out[nbytes] = round(n16 * 16 / ts[len(ts) // 2] / 1e9, 1)
        del bufs
        torch.cuda.empty_cache()
    log(f"stream read yardstick (GB/s by bytes): {out}")
    return out


def attach_read_yardstick(block, rates):
    """Each HBM-bound roofline entry gets the yardstick's rate for a read of its
    algorithmic bytes and its achieved rate as a fraction of that."""
    for entry in [block.get("roofline")] + list((block.get("rooflines") or {}).values()):
        if not entry or entry.get("bound") != "hbm":
            continue
        r = rates.get(entry["alg_bytes_per_launch"])
        if r:
            entry["read_yardstick_GBps"] = r
            entry["frac_of_read_yardstick"] = round(entry["achieved"] / r, 4)


def measured_peaks(log=print):
    """Achievable reference rates on this GPU, reported next to the spec-sheet
    peaks: a 1 GiB device copy (read + write bytes), a 1 GiB reduction (read
    bytes), a vendor bf16 GEMM (8192 x 8192 x 8192, library call), and the
    library's plain-read yardstick at 1 GiB.  The torch and vendor kernels are
    yardsticks only; no part of the step uses them."""
    import torch
    def timed(fn, iters):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(iters):
            fn()
        b.record()
        b.synchronize()
        return a.elapsed_time(b) / iters * 1e-3
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    t_copy = timed(lambda: dst.copy_(src), 10)
    words = src.view(torch.float32)
    t_read = timed(lambda: words.sum(), 10)
    del src, dst, words
    m = 8192
    a = torch.randn(m, m, device="cuda").to(torch.bfloat16)
    b = torch.randn(m, m, device="cuda").to(torch.bfloat16)
    t_mm = timed(lambda: torch.matmul(a, b), 10)
    del a, b
    out = {"copy_GBps": round(2 * n / t_copy / 1e9, 1), "read_GBps": round(n / t_read / 1e9, 1),
           "stream_read_1GiB_GBps": stream_read_rates([1 << 30], log=log)[1 << 30],
           "vendor_bf16_gemm_TFLOPs": round(2 * m ** 3 / t_mm / 1e12, 1),
           "spec_hbm_GBps": HBM_PEAK_GBPS, "spec_bf16_TFLOPs": BF16_PEAK_TFLOPS}
    log(f"measured peaks: {out}")
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama7b_bs1")
    ap.add_argument("--also", default="llama7b_bs16",
                    help="second workload reported alongside ('' to skip)")
    ap.add_argument("--large", default="vocab128k_ctx32k_bs32",
                    help="large workload reported alongside, fewer steps ('' to skip)")
    ap.add_argument("--large-steps", type=int, default=10)
    ap.add_argument("--rotate", type=int, default=None)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--cpu-single-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--loop", type=int, default=8,
                    help="steps per captured graph for the steady-state loop (0 to skip)")
    ap.add_argument("--loop-replays", type=int, default=10)
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the measured copy / read / vendor-GEMM reference rates")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one device copy of this many MiB first (counter calibration)")
    ap.add_argument("--mode", default="", choices=["", "greedy", "typical", "reject"],
                    help="override the workloads' acceptance mode")
    ap.add_argument("--hydra", action="store_true",
                    help="also time the step with the Hydra-style draft (medusa_hydra_draft: "
                         "one LM pass per tree depth) on the same workload")
    ap.add_argument("--mtp", action="store_true",
                    help="also time the step with MTP-style draft heads (medusa_mtp_draft: one "
                         "transformer layer of the Llama layer shape per head) on the same workload")
    ap.add_argument("--tree-sweep", default="",
                    help="comma-separated candidate counts: measure the tree budget "
                         "(expected tokens per second per tree size) on the workload")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: the verify step runs on one GPU; --gpus {args.gpus} "
              f"(WORLD_SIZE={world}) is not supported.", file=sys.stderr)
        sys.exit(2)

    import torch
    from speculative_decoding_heads_amd import configs as C

    log = lambda m: print(m, file=sys.stderr, flush=True)
    if args.copy_calibration_mib:
        copy_calibration(args.copy_calibration_mib)

    def cfg_of(name):
        c = C.BY_NAME[name]
        return c.with_(mode=args.mode) if args.mode else c

    cfg = cfg_of(args.workload)
    ms, per_call = measure(cfg, args.steps, args.warmup, args.rotate, log)
    main_block = summarise(cfg, ms, per_call)
    out = {
        "metric": METRIC, "value": main_block["value"], "unit": "verify-steps/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": main_block["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": cfg.name, "batch": cfg.b, "hidden": cfg.H, "vocab": cfg.V,
                   "medusa_heads": cfg.K, "shortlist": list(cfg.k), "tree_candidates": cfg.N,
                   "q_heads": cfg.nq, "kv_heads": cfg.nkv, "head_dim": cfg.d, "prefix": cfg.P,
                   "acceptance": cfg.mode, "parallelism": "single-gpu"},
    }
    out.update({k: v for k, v in main_block.items() if k not in ("value", "ms_per_step")})
    for key, name, steps, warm in (("also", args.also, args.steps, args.warmup),
                                   ("large", args.large, min(args.steps, args.large_steps),
                                    min(args.warmup, 3))):
        if not name:
            continue
        c2 = cfg_of(name)
        ms2, pc2 = measure(c2, steps, warm, None, log)
        blk = {"workload": c2.name, "unit": "verify-steps/s", "steps": steps, "warmup": warm}
        blk.update(summarise(c2, ms2, pc2))
        out[key] = blk
    if args.hydra:
        ms_h, pch = measure(cfg, args.steps, args.warmup, args.rotate, log, draft="hydra")
        out["hydra"] = {"workload": cfg.name, "draft": "hydra", "value": round(1000.0 / ms_h, 2),
                        "unit": "verify-steps/s", "ms_per_step": round(ms_h, 4),
                        "per_call_us": {k: round(v, 2) for k, v in pch.items()}}
    if args.mtp:
        from speculative_decoding_heads_amd.synth import mtp_width
        ms_m, pcm = measure(cfg, args.steps, args.warmup, args.rotate, log, draft="mtp")
        F = mtp_width(cfg.H)
        e = 2
        layer = (cfg.nq + 2 * cfg.nkv) * cfg.d * cfg.H + cfg.H * cfg.nq * cfg.d + 3 * F * cfg.H
        draft_bytes = cfg.K * layer * e + cfg.V * cfg.H * e \
            + cfg.K * 2 * cfg.b * cfg.nkv * cfg.P * cfg.d * e
        t = pcm["draft_hidden"] * 1e-6
        out["mtp"] = {"workload": cfg.name, "draft": "mtp", "value": round(1000.0 / ms_m, 2),
                      "unit": "verify-steps/s", "ms_per_step": round(ms_m, 4),
                      "mlp_width": F, "draft_alg_bytes": draft_bytes,
                      "draft_hbm_frac": round(draft_bytes / t / 1e9 / HBM_PEAK_GBPS, 4),
                      "per_call_us": {k: round(v, 2) for k, v in pcm.items()}}
    if args.loop > 0:
        ms_l = measure_loop(cfg, args.loop, args.loop_replays, log=log)
        out["loop"] = {"workload": cfg.name, "value": round(1000.0 / ms_l, 2),
                       "unit": "verify-steps/s", "ms_per_step": round(ms_l, 4),
                       "steps_per_graph": args.loop, "replays": args.loop_replays,
                       "hip_graph": True}
    if args.tree_sweep:
        sizes = [int(v) for v in args.tree_sweep.split(",") if v.strip()]
        out["tree_sweep"] = tree_sweep(cfg, sizes, args.steps, args.warmup, log)
    torch.cuda.synchronize()
    out["measured_peaks"] = None if args.no_peaks else measured_peaks(log)
    if not args.no_peaks:
        # the plain-read yardstick at the byte counts of every HBM-bound call
        blocks = [out] + [out[k] for k in ("also", "large") if k in out]
        sizes = [e["alg_bytes_per_launch"] for blk in blocks
                 for e in (blk.get("rooflines") or {}).values() if e.get("bound") == "hbm"]
        rates = stream_read_rates(sizes, log=log)
        out["measured_peaks"]["stream_read_GBps_by_bytes"] = {str(k): v for k, v in rates.items()}
        for blk in blocks:
            attach_read_yardstick(blk, rates)
    out["cpu_baseline"] = None if args.no_cpu_baseline else \
        cpu_baseline(cfg, args.cpu_seconds, args.cpu_single_seconds, log)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
