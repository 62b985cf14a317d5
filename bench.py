#!/usr/bin/env python3
"""Benchmark of the batched speculative-sampling verify step on one MI355X.

One step = one rs_verify call over a whole batch (row statistics, accept
tests, first rejection, sampling race, output rows).  The default workload is
B=256 requests, K=8 drafts each, V=151936, bf16 target logits, fp32 draft
probabilities, per-request temperature ~U[0.3, 1.2], mean acceptance ~0.75.
Inputs are built on the GPU before the timed region (three independent
copies, rotated so consecutive calls do not hit the 256 MB Infinity Cache);
the timed region holds exactly --steps calls bracketed by a device
synchronize, with an event between consecutive calls for per-call statistics.

Prints ONE JSON line on stdout:
  value           verified draft positions per second (D per call / time)
  trials          per-call times over the timed region: median, p10, p90
  roofline        the longest kernel of the call, measured with HIP events
                  recorded on the launch stream around every kernel:
                    achieved / frac    the call's algorithmic bytes given its
                                       outcome (every logits row a request
                                       needs: rows 0 .. n_b, the drafts behind
                                       a first rejection being discarded; the
                                       q row of each resampled request; the
                                       gathers and metadata) over the
                                       kernel's duration
                    every_row_*        the same with every logits row charged
                                       (what a method without early exit
                                       reads): an effective rate
                    traffic / moved_*  the HBM bytes rocprofv3 counted for the
                                       kernel (profiles/), over its duration
  variants        other paths and entry points on the same inputs, and the
                  other workloads (1, 2, 3, 5), each with its own statistics
  cpu_baseline    the CPU oracle timed on this host on a bounded sample, with
                  every host thread and with one
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


def profiled_traffic(kernel, tag="B256_K8_V151936"):
    """HBM bytes per dispatch of `kernel` from the committed rocprofv3 counter
    summary of the workload `tag` (FETCH_SIZE / WRITE_SIZE scaled by a
    known-size copy kernel), or None if the summary is missing or the kernel
    sources changed since."""
    import glob
    import hashlib
    path = os.path.join(ROOT, "profiles", f"rs_verify_{tag}_hbm_bytes.md")
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


def per_step_stats(events, steps):
    """Per-call statistics (ms) from events recorded before the first call
    and after every call of a timed region."""
    import numpy as np
    d = np.array([events[i].elapsed_time(events[i + 1]) for i in range(steps)])
    return {"ms_per_step": events[0].elapsed_time(events[steps]) / steps, "median_ms": float(np.median(d)),
            "p10_ms": float(np.percentile(d, 10)), "p90_ms": float(np.percentile(d, 90)), "trials": int(steps)}


def timed_region(fn, steps, warmup, stream):
    """warmup untimed calls running straight into exactly `steps` timed calls
    (the GPU's clocks drop after a few idle milliseconds), an event between
    consecutive calls, bracketed by device synchronisations."""
    import torch
    events = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    gc.collect()
    gc.disable()
    try:
        for k in range(warmup):
            fn(k)
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        events[0].record(stream)
        for k in range(steps):
            fn(k)
            events[k + 1].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
    finally:
        gc.enable()
    st = per_step_stats(events, steps)
    st["host_wall_ms_per_step"] = wall / steps * 1e3
    return st


def cache_resident(w, copies):
    """Do all input copies fit the 256 MB Infinity Cache together?"""
    b = w.logits.numel() * w.logits.element_size() + (0 if w.draft_probs is None else w.draft_probs.numel() * 4)
    return b * copies <= (256 << 20)


def workload_tag(w):
    return f"B{w.B}_K{w.max_k}_V{w.V}"


def cpu_oracle_rate(w, seconds, threads):
    """Full oracle calls of the workload on `threads` host threads until
    `seconds` of CPU work: positions/s, calls, time."""
    import oracle
    calls, t = 0, 0.0
    while calls == 0 or t < seconds:
        t1 = time.perf_counter()
        oracle.verify(w.logits, w.draft_probs, w.draft_token_ids, w.cu_num_draft_tokens, w.temperature, w.seed,
                      w.max_k, threads=threads)
        t += time.perf_counter() - t1
        calls += 1
    return w.D * calls / t, calls, t


class Bench:
    def __init__(self, args, dev, stream):
        self.args, self.dev, self.stream = args, dev, stream

    def workload(self, n):
        """Input copies, workspace and outputs of workload n."""
        import torch
        import rejection_sampling_verify_rs_amd as rs
        import rs_workloads as W
        a = self.args
        t0 = time.time()
        copies = [W.config(n, device=self.dev, copy=i) for i in range(a.copies)]
        torch.cuda.synchronize()
        w0 = copies[0]
        log(f"inputs: {a.copies} x {w0.name}: B={w0.B} D={w0.D} V={w0.V} "
            f"({w0.logits.numel() * w0.logits.element_size() / 1e6:.1f} MB logits"
            f"{'' if w0.draft_probs is None else f', {w0.draft_probs.numel() * 4 / 1e6:.1f} MB q'}) "
            f"built in {time.time() - t0:.1f}s")
        ws = torch.zeros(max(max(rs.workspace_size(w.B, w.D, w.max_k, w.V, w.logits.dtype) for w in copies), 1),
                         dtype=torch.uint8, device=self.dev)
        outs = [torch.empty((w.B, w.max_k + 1), dtype=torch.int32, device=self.dev) for w in copies]
        naccs = [torch.empty((w.B,), dtype=torch.int32, device=self.dev) for w in copies]
        return copies, ws, outs, naccs

    def measure(self, n, greedy_entry=False, ends=()):
        """Time workload n (rs_verify, or rs_verify_greedy) and attribute its
        bytes; returns (report, state for further variants)."""
        import numpy as np
        import torch
        import rejection_sampling_verify_rs_amd as rs
        a = self.args
        copies, ws, outs, naccs = self.workload(n)
        w0 = copies[0]
        stream = self.stream

        def call(i, debug=None):
            w = copies[i % a.copies]
            if greedy_entry:
                rs.verify_greedy(w.logits, w.draft_token_ids, w.cu_num_draft_tokens, max_k=w.max_k,
                                 out=outs[i % a.copies], num_accepted=naccs[i % a.copies], workspace=ws,
                                 stream=stream)
                return
            if debug is None and ends:
                debug = rs.Debug(phase_ends=ends)
            rs.verify(w.logits, w.draft_probs, w.draft_token_ids, w.cu_num_draft_tokens, w.temperature,
                      seed=w.seed, max_k=w.max_k, out=outs[i % a.copies], num_accepted=naccs[i % a.copies],
                      workspace=ws, debug=debug, stream=stream)

        st = timed_region(call, a.steps, a.warmup, stream)
        # outcome of each copy (deterministic) -> the bytes each kernel must move
        bounds = phase_bounds(w0.max_k, ends)
        path = 2
        if not greedy_entry:
            probe = rs.Debug()
            call(0, debug=probe)
            path = probe.path_taken
        outcomes, acc = [], []
        for i, w in enumerate(copies):
            call(i)
            torch.cuda.synchronize()
            nacc = naccs[i].cpu().numpy()
            if greedy_entry:  # every request greedy: no gathers, no q rows
                wg = w.to(self.dev)
                wg.temperature = torch.zeros_like(w.temperature)
                wg.draft_probs = None
                outcomes.append(outcome_bytes(wg, nacc, bounds, path))
            else:
                outcomes.append(outcome_bytes(w, nacc, bounds, path))
            acc.append(float(nacc.mean()))
        rot = [outcomes[k % a.copies] for k in range(a.steps)]
        needed = float(np.mean([o["needed"] for o in rot]))
        every = float(np.mean([o["every_row"] for o in rot]))
        step_s = st["ms_per_step"] / 1e3
        rep = {"config": w0.name, "B": w0.B, "K": w0.max_k, "V": w0.V, "total_draft_tokens": w0.D,
               "path": {1: "per-request", 2: "phased split", 3: "stream"}[path] if not greedy_entry else "greedy",
               **st, "positions_per_s": w0.D / step_s,
               "needed_bytes": needed, "every_row_bytes": every,
               "needed_GBps": needed / step_s / 1e9, "needed_frac": needed / step_s / 1e9 / HBM_PEAK_GBPS,
               "every_row_GBps": every / step_s / 1e9, "every_row_frac": every / step_s / 1e9 / HBM_PEAK_GBPS,
               "cache_resident": cache_resident(w0, a.copies), "mean_accepted": float(np.mean(acc)),
               "rows_needed": [o["rows_needed"] for o in outcomes], "rows": w0.D + w0.B,
               "resampled_rows": [o["n_res"] for o in outcomes]}
        if not greedy_entry:
            rep["roofline"] = self.roofline(call, outcomes, rot, path, needed, every, workload_tag(w0))
        log(f"{w0.name}{' (greedy entry)' if greedy_entry else ''}: {rep['path']}; "
            f"{st['ms_per_step'] * 1e3:.1f} us/step (median {st['median_ms'] * 1e3:.1f}, p10 {st['p10_ms'] * 1e3:.1f}, "
            f"p90 {st['p90_ms'] * 1e3:.1f}); {rep['positions_per_s']:.3g} positions/s; needed bytes "
            f"{needed / 1e6:.1f} MB -> {rep['needed_frac']:.1%} of HBM peak; every row {every / 1e6:.1f} MB -> "
            f"{rep['every_row_frac']:.1%}; mean accepted {rep['mean_accepted']:.3f}"
            f"{'; cache-resident inputs' if rep['cache_resident'] else ''}")
        return rep, {"copies": copies, "ws": ws, "outs": outs, "naccs": naccs, "call": call, "rot": rot,
                     "every": every, "needed": needed, "path": path, "outcomes": outcomes}

    def kernel_times(self, call, **knobs):
        """Mean and median duration (ms) of each kernel of a call: events
        recorded on the launch stream before the first kernel and after every
        kernel, over calls rotated like the timed region."""
        import numpy as np
        import torch
        import rejection_sampling_verify_rs_amd as rs
        a = self.args
        nk = max(20, min(a.steps, 40))
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(16)] for _ in range(nk)]
        launched = []
        for k in range(a.warmup):
            call(k, debug=rs.Debug(**knobs))
        for k in range(nk):
            dbg = rs.Debug(events=evs[k], **knobs)
            call(k, debug=dbg)
            launched.append(dbg.kernels_launched)
        torch.cuda.synchronize()
        nl = launched[0]
        assert all(x == nl for x in launched)
        d = np.array([[e[i].elapsed_time(e[i + 1]) for i in range(nl)] for e in evs])
        return [float(x) for x in d.mean(0)], [float(x) for x in np.median(d, 0)]

    def roofline(self, call, outcomes, rot, path, needed, every, tag):
        import numpy as np
        t, tmed = self.kernel_times(call)
        names = [k[0] for k in outcomes[0]["kernels"]]
        if len(t) != len(names):
            raise RuntimeError(f"library launched {len(t)} kernels, expected {names}")
        kbytes = [float(np.mean([o["kernels"][i][1] for o in rot])) for i in range(len(names))]
        kernels = {nm: {"us": ms * 1e3, "median_us": md * 1e3, "task_bytes": by, "GBps": by / (ms / 1e3) / 1e9}
                   for nm, ms, md, by in zip(names, t, tmed, kbytes)}
        dom = max(range(len(t)), key=lambda i: t[i])
        name, ms, by = names[dom], t[dom], kbytes[dom]
        sec = ms / 1e3
        traffic = profiled_traffic(name, tag)
        whole = name in ("stream", "request")  # the kernel that runs the whole hot path
        r = {"bound": "hbm", "achieved": by / sec / 1e9, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
             "frac": by / sec / 1e9 / HBM_PEAK_GBPS, "traffic": traffic, "kernel": name, "kernel_us": ms * 1e3,
             "kernel_median_us": tmed[dom] * 1e3, "algorithmic_bytes": by,
             "every_row_bytes": every if whole else None,
             "every_row_GBps": every / sec / 1e9 if whole else None,
             "every_row_frac": every / sec / 1e9 / HBM_PEAK_GBPS if whole else None,
             "moved_GBps": traffic / sec / 1e9 if traffic else None,
             "moved_frac": traffic / sec / 1e9 / HBM_PEAK_GBPS if traffic else None,
             "kernels": kernels}
        log("kernels (event-timed): " + ", ".join(f"{k} {v['us']:.1f} us ({v['GBps']:.0f} GB/s)"
                                                  for k, v in kernels.items()))
        log(f"roofline: {name} {ms * 1e3:.1f} us; {by / 1e6:.1f} MB algorithmic (needed) -> {r['frac']:.1%}"
            + (f"; every row {every / 1e6:.1f} MB -> {r['every_row_frac']:.1%}" if whole else "")
            + (f"; {traffic / 1e6:.1f} MB counted -> {r['moved_frac']:.1%}" if traffic else ""))
        return r


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--workload", type=int, default=4, help="1..5 (4 = B=256 K=8 V=151936)")
    ap.add_argument("--copies", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU oracle sample budget per thread count (0 = skip)")
    ap.add_argument("--phases", default="", help="phase ends, e.g. '3' or '2,5' (default: the library's rule)")
    ap.add_argument("--only", action="store_true", help="the headline workload only (no variants)")
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
    stream = torch.cuda.current_stream(dev)
    bench = Bench(args, dev, stream)
    ends = tuple(int(x) for x in args.phases.split(",") if x.strip())

    # ---- the headline workload: exactly --steps timed calls
    head, state = bench.measure(args.workload, ends=ends)
    copies, call = state["copies"], state["call"]
    w0 = copies[0]
    every = state["every"]

    variants = {}
    if not args.only:
        def timed_knobs(**knobs):
            dbg = rs.Debug(**knobs)
            return timed_region(lambda k: call(k, debug=dbg), args.steps, args.warmup, stream)

        # other paths of the same call
        for name, knobs in (("phased_split", {"sampling_path": 2}),
                            ("stream", {"sampling_path": 3}),
                            ("one_phase_every_row", {"sampling_path": 2, "phase_ends": (-1,)}),
                            ("per_request", {"sampling_path": 1})):
            st = timed_knobs(**knobs)
            variants[name] = {**st, "positions_per_s": w0.D / (st["ms_per_step"] / 1e3),
                              "every_row_frac": every / (st["ms_per_step"] / 1e3) / 1e9 / HBM_PEAK_GBPS}
            log(f"{name}: {st['ms_per_step'] * 1e3:.1f} us/step (median {st['median_ms'] * 1e3:.1f}), "
                f"{variants[name]['positions_per_s']:.3g} positions/s")
        tv, _ = bench.kernel_times(call, sampling_path=2, phase_ends=(-1,))
        lg = (w0.D + w0.B) * w0.V * w0.logits.element_size()
        variants["one_phase_every_row"]["row_pass_us"] = tv[0] * 1e3
        variants["one_phase_every_row"]["row_pass_GBps"] = lg / (tv[0] / 1e3) / 1e9
        log(f"one-phase row pass: {tv[0] * 1e3:.1f} us, {lg / (tv[0] / 1e3) / 1e9:.0f} GB/s of logits")
        if args.sweep:
            for split in ((1,), (2,), (3,), (4,), (5,), (1, 3), (2, 4), (2, 5), (3, 5), (1, 2, 4), (1, 3, 5)):
                st = timed_knobs(phase_ends=split)
                log(f"phase ends {split}: {st['ms_per_step'] * 1e3:.1f} us/step")

        # rs_verify_noalloc on the same inputs (the library's own scratch)
        def call_noalloc(k):
            i = k % args.copies
            w = copies[i]
            rs.verify_noalloc(w.logits, w.draft_probs, w.draft_token_ids, w.cu_num_draft_tokens, w.temperature,
                              seed=w.seed, max_k=w.max_k, out=state["outs"][i], num_accepted=state["naccs"][i],
                              stream=stream)
        if rs.workspace_size(w0.B, w0.D, w0.max_k, w0.V, w0.logits.dtype) <= rs.NOALLOC_SCRATCH_BYTES:
            st = timed_region(call_noalloc, args.steps, args.warmup, stream)
            variants["noalloc"] = {**st, "positions_per_s": w0.D / (st["ms_per_step"] / 1e3)}
            log(f"noalloc: {st['ms_per_step'] * 1e3:.1f} us/step")

        # top-k / top-p filtered verify (rs_verify_filtered) on the same inputs
        ws_f = torch.zeros(max(rs.workspace_size(w.B, w.D, w.max_k, w.V, w.logits.dtype, filtered=True)
                               for w in copies), dtype=torch.uint8, device=dev)
        for name, kk, pp in (("filtered_topk50_topp0.9", 50, 0.9), ("filtered_topk50", 50, None),
                             ("filtered_topp0.9", None, 0.9)):
            tk = None if kk is None else torch.full((w0.B,), kk, dtype=torch.int32, device=dev)
            tp = None if pp is None else torch.full((w0.B,), pp, dtype=torch.float32, device=dev)

            def call_f(k, debug=None, tk=tk, tp=tp):
                i = k % args.copies
                w = copies[i]
                rs.verify(w.logits, w.draft_probs, w.draft_token_ids, w.cu_num_draft_tokens, w.temperature,
                          seed=w.seed, max_k=w.max_k, out=state["outs"][i], num_accepted=state["naccs"][i],
                          workspace=ws_f, debug=debug, stream=stream, top_k=tk, top_p=tp)
            st = timed_region(call_f, args.steps, args.warmup, stream)
            kt, _ = bench.kernel_times(call_f)
            variants[name] = {**st, "positions_per_s": w0.D / (st["ms_per_step"] / 1e3),
                              "every_row_frac": every / (st["ms_per_step"] / 1e3) / 1e9 / HBM_PEAK_GBPS,
                              "kernel_us": [round(x * 1e3, 1) for x in kt]}
            log(f"{name}: {st['ms_per_step'] * 1e3:.1f} us/step (median {st['median_ms'] * 1e3:.1f}); "
                f"kernels (us) {variants[name]['kernel_us']}")
        del ws_f
        for i in range(args.copies):  # the unfiltered outcome of every copy again
            call(i)

        # acceptance counters after each call (rs_accept_stats_accumulate), one launch per step
        counters = torch.zeros(rs.STATS_COUNTERS, dtype=torch.int64, device=dev)
        st = timed_region(lambda k: rs.accept_stats_accumulate(state["naccs"][k % args.copies],
                                                               copies[k % args.copies].cu_num_draft_tokens,
                                                               counters, stream=stream),
                          args.steps, 0, stream)
        variants["accept_stats"] = {**st, "accept_rate": rs.accept_rate(counters),
                                    "accept_length": rs.accept_length(counters)}
        log(f"accept_stats: {st['ms_per_step'] * 1e3:.1f} us/step; alpha {variants['accept_stats']['accept_rate']:.4f}, "
            f"tau {variants['accept_stats']['accept_length']:.4f}")

        # tree verify (rs_verify_tree): B=64 EAGLE-style draft trees of 60 nodes
        # (branching 4, 2, 2, 1, 1; depth 5) at the same V, T ~ U[0.5, 1.2];
        # then the same with the draft distributions (fp32, every tree position)
        for with_q, key in ((False, "tree_eagle_B64"), (True, "tree_eagle_B64_draft_probs")):
            trees = [W.make_tree(64, w0.V, temperature=("uniform", 0.5, 1.2), seed=7, gen_seed=5000 + i, device=dev,
                                 with_q=with_q) for i in range(args.copies)]
            tw = trees[0]
            tws = torch.empty((rs.load_library().rs_verify_tree_workspace_size(tw.B, tw.V),), dtype=torch.uint8,
                              device=dev)
            tout = torch.empty((tw.B, tw.max_depth + 1), dtype=torch.int32, device=dev)
            tpath = torch.empty((tw.B, tw.max_depth), dtype=torch.int32, device=dev)
            tn = torch.empty((tw.B,), dtype=torch.int32, device=dev)

            def tree_call(k):
                t = trees[k % args.copies]
                rs.verify_tree(t.logits, t.node_tokens, t.node_parents, t.cu_num_nodes, t.temperature, seed=t.seed,
                               max_nodes=t.max_nodes, max_depth=t.max_depth, draft_probs=t.draft_probs, out=tout,
                               accepted_nodes=tpath, num_accepted=tn, workspace=tws, stream=stream)

            st = timed_region(tree_call, args.steps, args.warmup, stream)
            rows_read = []
            for i in range(args.copies):
                tree_call(i)
                torch.cuda.synchronize()
                rows_read.append(int((tn.cpu().numpy() + 1).sum()))
            tsec = st["ms_per_step"] / 1e3
            dense = (tw.N + tw.B) * tw.V * tw.logits.element_size()
            needed_t = float(np.mean(rows_read)) * tw.V * tw.logits.element_size()
            variants[key] = {
                **st, "nodes_per_s": tw.N / tsec, "nodes": tw.N, "rows": tw.N + tw.B,
                "rows_streamed": float(np.mean(rows_read)), "needed_frac": needed_t / tsec / 1e9 / HBM_PEAK_GBPS,
                "every_row_GBps": dense / tsec / 1e9}
            log(f"{key} (B=64, {tw.max_nodes} nodes, depth {tw.max_depth}): {st['ms_per_step'] * 1e3:.1f} us/step "
                f"(median {st['median_ms'] * 1e3:.1f}), {tw.N / tsec:.3g} nodes/s, {np.mean(rows_read):.0f} of "
                f"{tw.N + tw.B} rows streamed")
            del trees, tree_call

        # n-gram proposer (rs_ngram_propose): B=64 contexts of 4096 tokens,
        # min_n 3, max_n 8, k 5 (the pages' example settings)
        ctx, ccu = W.make_contexts(64, 4096, w0.V, seed=3, device=dev)
        holder = {}
        nb = int(ccu.numel()) - 1
        ng_out = (torch.empty(nb * 5, dtype=torch.int32, device=dev), torch.empty(nb, dtype=torch.int32, device=dev),
                  torch.empty(nb + 1, dtype=torch.int32, device=dev))
        ng_ws = torch.empty(nb * 5, dtype=torch.int32, device=dev)

        def ngram_call(k):  # outputs and workspace allocated once, as a serving loop would
            holder["r"] = rs.ngram_propose(ctx, ccu, min_n=3, max_n=8, k=5, out=ng_out, workspace=ng_ws,
                                           stream=stream)

        st = timed_region(ngram_call, args.steps, args.warmup, stream)
        variants["ngram_B64_ctx4096"] = {**st, "context_tokens_per_s": ctx.numel() / (st["ms_per_step"] / 1e3),
                                         "mean_drafts": float(holder["r"][1].float().mean())}
        log(f"ngram (B=64, 4096-token contexts): {st['ms_per_step'] * 1e3:.1f} us/step")

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

    # ---- CPU oracle on a bounded sample of the headline workload (copy 0)
    cpu = None
    if args.cpu_seconds > 0:
        hc = w0.to("cpu")
        threads = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
        threads = max(1, min(threads, len(os.sched_getaffinity(0))))
        model = ""
        try:
            with open("/proc/cpuinfo") as f:
                model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
        except OSError:
            pass
        rate, calls, t_cpu = cpu_oracle_rate(hc, args.cpu_seconds, threads)
        rate1, calls1, t1 = cpu_oracle_rate(hc, args.cpu_seconds, 1)
        cpu = {"value": rate, "unit": "positions/s", "cores": threads, "kind": "oracle",
               "sample": f"{calls} full call(s) of the same workload (copy 0, all {hc.B} requests), {t_cpu:.1f} s, "
                         f"fp64 C oracle with OpenMP over requests on {threads} threads of {model}",
               "single_thread": {"value": rate1, "unit": "positions/s", "cores": 1,
                                 "sample": f"{calls1} full call(s), {t1:.1f} s, one thread"}}
        log(f"cpu oracle: {rate:.3g} positions/s on {threads} threads ({calls} calls, {t_cpu:.1f}s); "
            f"{rate1:.3g} on 1 thread ({calls1} calls, {t1:.1f}s)")
    del copies, state, call

    # ---- the other workloads, each measured the same way (after the headline's CPU leg)
    if not args.only:
        for n in (1, 2, 3, 4, 5):
            if n == args.workload:
                continue
            rep, st_n = bench.measure(n)
            variants[f"workload_{n}"] = rep
            del st_n
            if n == 2:
                rep, st_n = bench.measure(2, greedy_entry=True)
                variants["workload_2_greedy_entry"] = rep
                del st_n
            torch.cuda.empty_cache()

    step_s = head["ms_per_step"] / 1e3
    line = {
        "metric": METRIC,
        "value": head["positions_per_s"],
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": head["config"], "B": head["B"], "K": head["K"], "V": head["V"],
                   "total_draft_tokens": head["total_draft_tokens"],
                   "logits_dtype": str(w0.logits.dtype).replace("torch.", ""),
                   "draft_probs": w0.draft_probs is not None, "input_copies": args.copies,
                   "path": head["path"], "parallelism": "single GPU"},
        "trials": {k: head[k] for k in ("median_ms", "p10_ms", "p90_ms", "trials", "host_wall_ms_per_step")},
        "needed_GBps": head["needed_GBps"],
        "needed_frac": head["needed_frac"],
        "every_row_GBps": head["every_row_GBps"],
        "every_row_frac": head["every_row_frac"],
        "bytes_per_step": {"needed": head["needed_bytes"], "every_row": head["every_row_bytes"]},
        "mean_accepted": head["mean_accepted"],
        "rows_needed": head["rows_needed"],
        "roofline": head["roofline"],
        "variants": variants,
        "cpu_baseline": cpu,
    }
    log(f"headline: {head['ms_per_step'] * 1e3:.1f} us/step, {head['positions_per_s']:.4g} positions/s, "
        f"whole call {head['needed_frac']:.1%} of HBM peak on needed bytes ({step_s * 1e6:.1f} us)")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
