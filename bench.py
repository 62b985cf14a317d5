#!/usr/bin/env python3
"""Benchmark of the batched speculative-sampling verify step on one MI355X.

One step = one rs_verify call over a whole batch (row statistics, accept
tests, first rejection, sampling race, output rows).  The default workload is
B=256 requests, K=8 drafts each, V=151936, bf16 target logits, fp32 draft
probabilities, per-request temperature ~U[0.3, 1.2], mean acceptance ~0.75.
Inputs are built on the GPU before the timed region (three independent
copies, rotated so consecutive calls do not hit the 256 MB Infinity Cache);
the timed region holds exactly --steps calls bracketed by a device
synchronize.

Prints ONE JSON line on stdout:
  value           verified draft positions per second (D per call / time)
  effective_GBps  every logits row once + gathers + resampled q rows +
                  metadata, over the call time (rows skipped behind a first
                  rejection still count)
  achieved_GBps   the bytes the call's kernels must move (rows 0 .. n_b of
                  each request on the stream path) over the call time
  roofline        the longest kernel of the call: its algorithmic bytes /
                  its average duration, measured with HIP events recorded on
                  the launch stream after every kernel.  On the stream path
                  that kernel runs the whole hot path and is charged with the
                  call's algorithmic bytes (every logits row once, as
                  effective_GBps); `traffic` is the HBM bytes rocprofv3
                  counted for it (profiles/), `moved_GBps` that over its
                  duration
  cpu_baseline    the CPU oracle timed on this host on a bounded sample
Diagnostics go to stderr.
"""
import argparse
import gc
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verified draft positions/s + achieved HBM GB/s (% of peak), B=256 K=8 V=152k"
HBM_PEAK_GBPS = 8000.0  # MI355X published HBM3E bandwidth


def log(*a):
    print(*a, file=sys.stderr, flush=True)




def phase_bounds(max_k, ends=()):
    """Phase boundaries of the library's split path: its automatic rule (with
    L = max_k + 1 >= 3, phases [0, ceil(L/3)) and [ceil(L/3), L); one phase
    otherwise), (-1,) for one phase, or explicit phase ends."""
    L = max_k + 1
    ends = tuple(ends)
    if ends and ends[0] < 0:
        return [0, L]
    if not ends or ends[0] == 0:
        ends = ((L + 2) // 3,) if L >= 3 else ()
    bounds = [0]
    for e in ends[:3]:
        if e <= bounds[-1] or e >= L:
            break
        bounds.append(e)
    return bounds + [L]


def outcome_bytes(w, num_accepted, bounds, path=2):
    """Bytes each kernel's tasks must move for one call, given the outcome.

    Phased split path (2): per phase i a row kernel (phase1: rows; phase2..:
    rows + the race of the previous phase's decisions) and its scan (accept
    tests), then race<last> (the race of the last phase's decisions) and emit
    (output rows of random requests).  Row
    statistics of phase i read every logits row of that phase's positions
    for the requests still active (all requests in phase 1); a race reads the
    q row of a request resampled with draft probabilities (the logits row it
    re-reads is not counted: it is an implementation re-read, and usually an
    Infinity Cache hit).
    Per-request path (1): one kernel, charged with the 'needed' bytes.
    Stream path (3): init (per-request set-up), stream (charged with all the
    'needed' bytes; rows it reads speculatively are not counted) and
    race_tail (race chunks left to after the stream kernel, charged nothing).
    Also returned: 'needed' = only rows 0 .. n_b of each request (the least
    any implementation of the rule must read) and 'every_row' = every logits
    row once (what a single phase reads).
    """
    import numpy as np
    B, D, V = w.B, w.D, w.V
    sl = w.logits.element_size()
    ks = np.asarray(w.num_draft)
    T = w.temperature.cpu().numpy()
    has_q = w.draft_probs is not None
    n = np.asarray(num_accepted)
    rnd = T > 0
    qrow = np.where(rnd & (n < ks) & has_q, V * 4, 0)  # q row of each resampled request
    gather = 4 + (4 if has_q else 0)
    meta = 4 * B + 4 * (B + 1) + 4 * B * (w.max_k + 2)
    rows_needed = int((n + 1).sum())
    evaluated = int(np.minimum(n + 1, ks).sum())
    needed = rows_needed * V * sl + evaluated * gather + int(qrow.sum()) + meta
    every = (D + B) * V * sl + D * gather + int(qrow.sum()) + meta
    kernels = []
    if path == 1:
        kernels = [("request", needed)]
    elif path == 3:
        kernels = [("init", 0), ("stream", needed), ("race_tail", 0)]
    else:
        nph = len(bounds) - 1
        for i in range(nph):
            jb, je = bounds[i], bounds[i + 1]
            active = np.ones(B, bool) if i == 0 else (n >= jb)
            rows = int((active * np.clip(np.minimum(je, ks + 1) - jb, 0, None)).sum())
            race_q = 0
            if i >= 1:
                dec = (n >= bounds[i - 1]) & (n < bounds[i]) & rnd
                race_q = int(qrow[dec].sum())
            gathers = int((active * np.clip(np.minimum(je, ks) - jb, 0, None)).sum()) * gather
            kernels.append(("phase%d" % (i + 1), rows * V * sl + race_q + gathers))
            kernels.append(("scan%d" % (i + 1), 0))
        last = (n >= bounds[nph - 1]) & rnd
        kernels.append(("race%d" % nph, int(qrow[last].sum())))
        kernels.append(("emit", meta))
    return {"kernels": kernels, "total": sum(k[1] for k in kernels), "needed": needed, "every_row": every,
            "rows_needed": rows_needed, "n_res": int((qrow > 0).sum())}


def profiled_traffic(kernel):
    """HBM bytes per dispatch of `kernel` from the committed rocprofv3 counter
    summary (FETCH_SIZE / WRITE_SIZE scaled by a known-size copy kernel), or
    None if the summary is missing or the kernel sources changed since."""
    import glob
    import hashlib
    path = os.path.join(ROOT, "profiles", "rs_verify_B256_K8_V151936_hbm_bytes.md")
    if not os.path.exists(path):
        return None
    traffic, sha = None, None
    for line in open(path):
        if line.startswith("traffic_bytes_per_dispatch:"):
            traffic = json.loads(line.split(":", 1)[1])
        elif line.startswith("kernel_source_sha256:"):
            sha = line.split(":", 1)[1].strip()
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "rejection_sampling_verify_rs_amd", "csrc", "*"))):
        h.update(open(p, "rb").read())
    if traffic is None or sha != h.hexdigest():
        return None
    return traffic.get(kernel)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--workload", type=int, default=4, help="1..5 (4 = B=256 K=8 V=151936)")
    ap.add_argument("--copies", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU oracle sample budget (0 = skip)")
    ap.add_argument("--phases", default="", help="phase ends, e.g. '3' or '2,5' (default: the library's rule)")
    ap.add_argument("--sweep", action="store_true", help="also time a set of phase splits (stderr)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 512 MiB device copy (known bytes) to scale HBM byte counters")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures the verify step on one GPU only (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE={world}); requests are independent, so N GPUs would each run this same "
              f"call on B/N requests.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import rejection_sampling_verify_rs_amd as rs
    import rs_workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a HIP device", file=sys.stderr)
        sys.exit(1)
    rs.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    t0 = time.time()
    copies = [W.config(args.workload, device=dev, copy=i) for i in range(args.copies)]
    torch.cuda.synchronize()
    w0 = copies[0]
    log(f"inputs: {args.copies} x {w0.name}: B={w0.B} D={w0.D} V={w0.V} "
        f"({w0.logits.numel() * w0.logits.element_size() / 1e6:.1f} MB logits"
        f"{'' if w0.draft_probs is None else f', {w0.draft_probs.numel() * 4 / 1e6:.1f} MB q'}) "
        f"built in {time.time() - t0:.1f}s")

    ws = torch.zeros(max(rs.workspace_size(w.B, w.D, w.max_k, w.V, w.logits.dtype) for w in copies),
                     dtype=torch.uint8, device=dev)
    outs = [torch.empty((w.B, w.max_k + 1), dtype=torch.int32, device=dev) for w in copies]
    naccs = [torch.empty((w.B,), dtype=torch.int32, device=dev) for w in copies]
    stream = torch.cuda.current_stream(dev)

    ends = tuple(int(x) for x in args.phases.split(",") if x.strip())

    filt = {"top_k": None, "top_p": None}  # set while timing the filtered variants
    ws_f = None

    def call(i, debug=None):
        w = copies[i]
        if debug is None and ends:
            debug = rs.Debug(phase_ends=ends)
        elif debug is not None and ends and not debug.phase_ends:
            debug.phase_ends = ends
        tk, tp = filt["top_k"], filt["top_p"]
        rs.verify(w.logits, w.draft_probs, w.draft_token_ids, w.cu_num_draft_tokens, w.temperature,
                  seed=w.seed, max_k=w.max_k, out=outs[i], num_accepted=naccs[i],
                  workspace=ws if tk is None and tp is None else ws_f, debug=debug, stream=stream,
                  top_k=tk, top_p=tp)

    # Warm-up runs straight into the timed region (the GPU's clocks drop after
    # even a few milliseconds idle), with no garbage-collection pauses on the
    # launching thread meanwhile.
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    gc.collect()
    gc.disable()
    for k in range(args.warmup):
        call(k % args.copies)

    # ---- timed region: exactly --steps calls
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record(stream)
    for k in range(args.steps):
        call(k % args.copies)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    gc.enable()
    ms_per_step = start.elapsed_time(end) / args.steps
    log(f"timed {args.steps} steps: {ms_per_step * 1e3:.1f} us/step (host wall {wall / args.steps * 1e6:.1f} us/step)")


    # ---- outcome of each copy (deterministic) -> bytes each kernel must move
    bounds = phase_bounds(w0.max_k, ends)
    probe = rs.Debug()
    call(0, debug=probe)
    path = probe.path_taken
    path_name = {1: "per-request", 2: "phased split", 3: "stream"}[path]
    outcomes, acc = [], []
    for i, w in enumerate(copies):
        call(i)
        torch.cuda.synchronize()
        n = naccs[i].cpu().numpy()
        outcomes.append(outcome_bytes(w, n, bounds, path))
        acc.append(float(n.mean()))
    rot = [outcomes[k % args.copies] for k in range(args.steps)]
    alg_total = float(np.mean([o["total"] for o in rot]))
    alg_needed = float(np.mean([o["needed"] for o in rot]))
    alg_every = float(np.mean([o["every_row"] for o in rot]))
    step_s = ms_per_step / 1e3
    positions_per_s = w0.D / step_s
    eff_gbps = alg_total / step_s / 1e9
    # The method's algorithmic bytes (every logits row once, gathers, the q row
    # of every resampled request, metadata) over the call time: rows skipped
    # behind a first rejection still count, so this "effective" rate can
    # exceed what the call physically moves.
    every_gbps = alg_every / step_s / 1e9

    # ---- per-kernel durations: events recorded on the launch stream after every kernel
    def kernel_times(**knobs):
        nk = max(10, min(args.steps, 40))
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(16)] for _ in range(nk)]
        launched = []
        for k in range(args.warmup):
            call(k % args.copies, debug=rs.Debug(**knobs))
        for k in range(nk):
            dbg = rs.Debug(events=evs[k], **knobs)
            call(k % args.copies, debug=dbg)
            launched.append(dbg.kernels_launched)
        torch.cuda.synchronize()
        nl = launched[0]
        assert all(x == nl for x in launched)
        return [float(np.mean([e[a].elapsed_time(e[a + 1]) for e in evs])) for a in range(nl)]

    def timed_steps(**knobs):
        dbg = rs.Debug(**knobs)
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        gc.disable()
        for k in range(args.warmup):
            call(k % args.copies, debug=dbg)
        torch.cuda.synchronize()
        s0.record(stream)
        for k in range(args.steps):
            call(k % args.copies, debug=dbg)
        s1.record(stream)
        torch.cuda.synchronize()
        gc.enable()
        return s0.elapsed_time(s1) / args.steps

    t = kernel_times()
    names = [k[0] for k in outcomes[0]["kernels"]]
    if len(t) != len(names):
        raise RuntimeError(f"library launched {len(t)} kernels, expected {names}")
    kbytes = [float(np.mean([o["kernels"][i][1] for o in rot])) for i in range(len(names))]
    kernels = {nm: {"us": ms * 1e3, "task_bytes": by, "GBps": by / (ms / 1e3) / 1e9}
               for nm, ms, by in zip(names, t, kbytes)}
    dom = max(range(len(t)), key=lambda i: t[i])
    dom_name, dom_ms, dom_bytes = names[dom], t[dom], kbytes[dom]
    if dom_name == "stream":
        # The stream kernel is the whole hot path (every row is either
        # streamed or skipped behind a first rejection, and it runs all but a
        # few race chunks), so it is charged with the method's algorithmic
        # bytes for the call: every logits row once + gathers + the q row of
        # each resampled request + metadata.
        dom_bytes = alg_every
    dom_gbps = dom_bytes / (dom_ms / 1e3) / 1e9
    dom_traffic = profiled_traffic(dom_name) if w0.name.startswith("B=256 K=8 V=151936") else None
    log("kernels (event-timed): " + ", ".join(f"{k} {v['us']:.1f} us ({v['GBps']:.0f} GB/s)"
                                              for k, v in kernels.items()))
    log(f"path: {path_name}; effective {every_gbps:.0f} GB/s (every row once, {every_gbps / HBM_PEAK_GBPS:.1%} of "
        f"peak); {eff_gbps:.0f} GB/s of needed / task bytes; rows needed per call "
        f"{[o['rows_needed'] for o in outcomes]} of {w0.D + w0.B}; resampled rows {[o['n_res'] for o in outcomes]}; "
        f"mean accepted {np.mean(acc):.3f}")

    # other configurations of the same call, for reference
    variants = {}
    for name, knobs in (("phased_split", {"sampling_path": 2}),
                        ("stream", {"sampling_path": 3}),
                        ("one_phase_every_row", {"sampling_path": 2, "phase_ends": (-1,)}),
                        ("per_request", {"sampling_path": 1})):
        ms_v = timed_steps(**knobs)
        variants[name] = {"ms_per_step": ms_v, "positions_per_s": w0.D / (ms_v / 1e3),
                          "algorithmic_GBps": alg_every / (ms_v / 1e3) / 1e9}
        log(f"{name}: {ms_v * 1e3:.1f} us/step, {w0.D / (ms_v / 1e3):.3g} positions/s, "
            f"{variants[name]['algorithmic_GBps'] / HBM_PEAK_GBPS:.1%} of the HBM roofline on algorithmic bytes")
    if args.sweep:
        for split in ((1,), (2,), (3,), (4,), (5,), (1, 3), (2, 4), (2, 5), (3, 5), (1, 2, 4), (1, 3, 5), (2, 3, 5)):
            ms_v = timed_steps(phase_ends=split)
            log(f"phase ends {split}: {ms_v * 1e3:.1f} us/step, {w0.D / (ms_v / 1e3):.3g} positions/s")
    # top-k / top-p filtered verify (rs_verify_filtered) on the same inputs:
    # every request with top_k = 50 and top_p = 0.9, or one of them
    ws_f = torch.zeros(max(rs.workspace_size(w.B, w.D, w.max_k, w.V, w.logits.dtype, filtered=True) for w in copies),
                       dtype=torch.uint8, device=dev)
    for name, k, p in (("filtered_topk50_topp0.9", 50, 0.9), ("filtered_topk50", 50, None),
                       ("filtered_topp0.9", None, 0.9)):
        filt["top_k"] = None if k is None else torch.full((w0.B,), k, dtype=torch.int32, device=dev)
        filt["top_p"] = None if p is None else torch.full((w0.B,), p, dtype=torch.float32, device=dev)
        ms_v = timed_steps()
        tk = kernel_times()
        variants[name] = {"ms_per_step": ms_v, "positions_per_s": w0.D / (ms_v / 1e3),
                          "algorithmic_GBps": alg_every / (ms_v / 1e3) / 1e9,
                          "kernel_us": [round(x * 1e3, 1) for x in tk]}
        log(f"{name}: {ms_v * 1e3:.1f} us/step, {w0.D / (ms_v / 1e3):.3g} positions/s, "
            f"{variants[name]['algorithmic_GBps'] / HBM_PEAK_GBPS:.1%} of the HBM roofline on algorithmic bytes; "
            f"kernels (us) {variants[name]['kernel_us']}")
    filt["top_k"] = filt["top_p"] = None
    for i in range(args.copies):  # the unfiltered outcome of every copy again
        call(i)
    # acceptance counters after each call (rs_accept_stats_accumulate), one launch per step
    counters = torch.zeros(rs.STATS_COUNTERS, dtype=torch.int64, device=dev)
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s0.record(stream)
    for k in range(args.steps):
        rs.accept_stats_accumulate(naccs[k % args.copies], copies[k % args.copies].cu_num_draft_tokens, counters,
                                   stream=stream)
    s1.record(stream)
    torch.cuda.synchronize()
    variants["accept_stats"] = {"us_per_step": s0.elapsed_time(s1) / args.steps * 1e3,
                                "accept_rate": rs.accept_rate(counters), "accept_length": rs.accept_length(counters)}
    log(f"accept_stats: {variants['accept_stats']['us_per_step']:.1f} us/step; alpha "
        f"{variants['accept_stats']['accept_rate']:.4f}, tau {variants['accept_stats']['accept_length']:.4f}")
    # tree verify (rs_verify_tree): B=64 EAGLE-style draft trees of 60 nodes
    # (branching 4, 2, 2, 1, 1; depth 5) at the same V, T ~ U[0.5, 1.2]
    trees = [W.make_tree(64, w0.V, temperature=("uniform", 0.5, 1.2), seed=7, gen_seed=5000 + i, device=dev)
             for i in range(args.copies)]
    tw = trees[0]
    tws = torch.empty((rs.load_library().rs_verify_tree_workspace_size(tw.B, tw.V),), dtype=torch.uint8, device=dev)
    tout = torch.empty((tw.B, tw.max_depth + 1), dtype=torch.int32, device=dev)
    tpath = torch.empty((tw.B, tw.max_depth), dtype=torch.int32, device=dev)
    tn = torch.empty((tw.B,), dtype=torch.int32, device=dev)

    def tree_call(i):
        t = trees[i % args.copies]
        rs.verify_tree(t.logits, t.node_tokens, t.node_parents, t.cu_num_nodes, t.temperature, seed=t.seed,
                       max_nodes=t.max_nodes, max_depth=t.max_depth, out=tout, accepted_nodes=tpath,
                       num_accepted=tn, workspace=tws, stream=stream)

    for k in range(args.warmup):
        tree_call(k)
    torch.cuda.synchronize()
    s0.record(stream)
    for k in range(args.steps):
        tree_call(k)
    s1.record(stream)
    torch.cuda.synchronize()
    tms = s0.elapsed_time(s1) / args.steps
    rows_read = []
    for i in range(args.copies):
        tree_call(i)
        torch.cuda.synchronize()
        rows_read.append(int((tn.cpu().numpy() + 1).sum()))
    dense = (tw.N + tw.B) * tw.V * tw.logits.element_size()
    variants["tree_eagle_B64"] = {
        "us_per_step": tms * 1e3, "nodes_per_s": tw.N / (tms / 1e3), "nodes": tw.N, "rows": tw.N + tw.B,
        "rows_streamed": float(np.mean(rows_read)),
        "effective_GBps": dense / (tms / 1e3) / 1e9}
    log(f"tree (B=64, {tw.max_nodes} nodes, depth {tw.max_depth}): {tms * 1e3:.1f} us/step, "
        f"{tw.N / (tms / 1e3):.3g} nodes/s, {np.mean(rows_read):.0f} of {tw.N + tw.B} rows streamed, "
        f"{dense / (tms / 1e3) / 1e9:.0f} GB/s effective (every row once)")
    del trees
    # n-gram proposer (rs_ngram_propose): B=64 contexts of 4096 tokens,
    # min_n 3, max_n 8, k 5 (the pages' example settings)
    ctx, ccu = W.make_contexts(64, 4096, w0.V, seed=3, device=dev)
    for _ in range(args.warmup):
        rs.ngram_propose(ctx, ccu, min_n=3, max_n=8, k=5, stream=stream)
    torch.cuda.synchronize()
    s0.record(stream)
    for _ in range(args.steps):
        _, nprop, _ = rs.ngram_propose(ctx, ccu, min_n=3, max_n=8, k=5, stream=stream)
    s1.record(stream)
    torch.cuda.synchronize()
    nms = s0.elapsed_time(s1) / args.steps
    variants["ngram_B64_ctx4096"] = {"us_per_step": nms * 1e3, "context_tokens_per_s": ctx.numel() / (nms / 1e3),
                                     "mean_drafts": float(nprop.float().mean())}
    log(f"ngram (B=64, 4096-token contexts): {nms * 1e3:.1f} us/step, {ctx.numel() / (nms / 1e3):.3g} context "
        f"tokens/s, {float(nprop.float().mean()):.2f} drafts/request")
    tv = kernel_times(sampling_path=2, phase_ends=(-1,))
    lg = (w0.D + w0.B) * w0.V * w0.logits.element_size()
    variants["one_phase_every_row"]["row_pass_us"] = tv[0] * 1e3
    variants["one_phase_every_row"]["row_pass_GBps"] = lg / (tv[0] / 1e3) / 1e9
    log(f"one-phase row pass: {tv[0] * 1e3:.1f} us, {lg / (tv[0] / 1e3) / 1e9:.0f} GB/s of logits")

    if args.copy_calibration:
        # a plain elementwise copy kernel of known size (torch.mul by 1 on fp32;
        # a same-device copy_ would go to the DMA engine, which the counters
        # do not see): 512 MiB read + 512 MiB written per launch
        a = torch.ones(128 << 20, dtype=torch.float32, device=dev)
        c = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(3):
            torch.mul(a, 1.0, out=c)
        torch.cuda.synchronize()
        log("copy calibration: 3 x elementwise copy kernel of 536870912 bytes read + written")
        del a, c

    # ---- CPU oracle on a bounded sample of the same workload
    cpu = None
    if args.cpu_seconds > 0:
        import oracle
        threads = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
        threads = max(1, min(threads, len(os.sched_getaffinity(0))))
        hc = w0.to("cpu")
        calls, t_cpu = 0, 0.0
        while calls == 0 or t_cpu < args.cpu_seconds:
            t1 = time.perf_counter()
            oracle.verify(hc.logits, hc.draft_probs, hc.draft_token_ids, hc.cu_num_draft_tokens, hc.temperature,
                          hc.seed, hc.max_k, threads=threads)
            t_cpu += time.perf_counter() - t1
            calls += 1
        cpu_rate = hc.D * calls / t_cpu
        model = ""
        try:
            with open("/proc/cpuinfo") as f:
                model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
        except OSError:
            pass
        cpu = {"value": cpu_rate, "unit": "positions/s", "cores": threads, "kind": "oracle",
               "sample": f"{calls} full call(s) of the same workload (copy 0, all {hc.B} requests), "
                         f"{t_cpu:.1f} s, fp64 C oracle with OpenMP over requests on {model}"}
        log(f"cpu oracle: {cpu_rate:.3g} positions/s on {threads} threads ({calls} calls, {t_cpu:.1f}s)")

    line = {
        "metric": METRIC,
        "value": positions_per_s,
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w0.name, "B": w0.B, "K": w0.max_k, "V": w0.V, "total_draft_tokens": w0.D,
                   "logits_dtype": str(w0.logits.dtype).replace("torch.", ""),
                   "draft_probs": w0.draft_probs is not None, "input_copies": args.copies,
                   "path": path_name, "phases": bounds if path == 2 else None, "parallelism": "single GPU"},
        "effective_GBps": every_gbps,
        "effective_frac": every_gbps / HBM_PEAK_GBPS,
        "achieved_GBps": eff_gbps,
        "hbm_frac": eff_gbps / HBM_PEAK_GBPS,
        "bytes_per_step": {"tasks": alg_total, "needed": alg_needed, "every_row": alg_every},
        "kernels": kernels,
        "mean_accepted": float(np.mean(acc)),
        "roofline": {"bound": "hbm", "achieved": dom_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": dom_gbps / HBM_PEAK_GBPS, "traffic": dom_traffic,
                     "kernel": dom_name, "kernel_us": dom_ms * 1e3, "algorithmic_bytes": dom_bytes,
                     # what the kernel physically moved per the HBM byte counters, over its duration
                     "moved_GBps": (dom_traffic / (dom_ms / 1e3) / 1e9) if dom_traffic else None},
        "variants": variants,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
