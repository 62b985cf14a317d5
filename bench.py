#!/usr/bin/env python3
"""Benchmark of the batched speculative-sampling verify step on one MI355X.

One step = one rs_verify call over a whole batch (row pass, scan, sampling
race).  The default workload is B=256 requests, K=8 drafts each, V=151936,
bf16 target logits, fp32 draft probabilities, per-request temperature
~U[0.3, 1.2], mean acceptance ~0.75.  Inputs are built on the GPU before the
timed region (three independent copies, rotated so consecutive calls do not
hit the 256 MB Infinity Cache); the timed region holds exactly --steps calls
bracketed by a device synchronize.

Prints ONE JSON line on stdout:
  value      verified draft positions per second (D per call / time per call)
  roofline   the row pass (the dominant kernel): algorithmic bytes (every logits
             row once) / its average duration, measured with HIP events
             recorded on the launch stream around that kernel
  cpu_baseline  the CPU oracle timed on this host on a bounded sample
Diagnostics go to stderr.
"""
import argparse
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




def algorithmic_bytes(w, num_accepted):
    """Bytes the method must move for one call, given its outcome.

    every_row: every logits row once (the full-pass definition), plus the
      q(x*) gathers and draft ids of every position, the q row at every
      resampled position, temperatures, cu and the outputs.
    needed: only the rows the verify rule reads -- rows 0 .. n_b of request b
      (a draft behind the first rejection is discarded unread) -- with the
      gathers of those positions, plus the same q rows and metadata.
    logits_every_row / logits_needed: the logits part of each.
    """
    import numpy as np
    B, D, V = w.B, w.D, w.V
    sl = w.logits.element_size()
    ks = np.asarray(w.num_draft)
    T = w.temperature.cpu().numpy()
    random_req = T > 0
    has_q = w.draft_probs is not None
    n = np.asarray(num_accepted)
    n_res = int(((n < ks) & random_req).sum()) if has_q else 0
    gather = 4 + (4 if has_q else 0)
    meta = 4 * B + 4 * (B + 1) + 4 * B * (w.max_k + 2)
    rows_needed = int((n + 1).sum())
    evaluated = int(np.minimum(n + 1, ks).sum())
    every = (D + B) * V * sl + D * gather + n_res * V * 4 + meta
    needed = rows_needed * V * sl + evaluated * gather + n_res * V * 4 + meta
    return {"every_row": every, "needed": needed, "logits_every_row": (D + B) * V * sl,
            "logits_needed": rows_needed * V * sl, "n_res": n_res, "rows_needed": rows_needed}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=4, help="1..5 (4 = B=256 K=8 V=151936)")
    ap.add_argument("--copies", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU oracle sample budget (0 = skip)")
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

    ws = torch.empty(rs.workspace_size(w0.B, w0.D, w0.max_k, w0.V, w0.logits.dtype), dtype=torch.uint8, device=dev)
    outs = [torch.empty((w.B, w.max_k + 1), dtype=torch.int32, device=dev) for w in copies]
    naccs = [torch.empty((w.B,), dtype=torch.int32, device=dev) for w in copies]
    stream = torch.cuda.current_stream(dev)

    def call(i, debug=None):
        w = copies[i]
        rs.verify(w.logits, w.draft_probs, w.draft_token_ids, w.cu_num_draft_tokens, w.temperature,
                  seed=w.seed, max_k=w.max_k, out=outs[i], num_accepted=naccs[i], workspace=ws, debug=debug,
                  stream=stream)

    for k in range(args.warmup):
        call(k % args.copies)
    torch.cuda.synchronize()

    # ---- timed region: exactly --steps calls
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record(stream)
    for k in range(args.steps):
        call(k % args.copies)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = start.elapsed_time(end) / args.steps
    log(f"timed {args.steps} steps: {ms_per_step * 1e3:.1f} us/step (host wall {wall / args.steps * 1e6:.1f} us/step)")


    # ---- outcome of each copy (deterministic) -> algorithmic bytes
    outcomes, acc = [], []
    for i, w in enumerate(copies):
        call(i)
        torch.cuda.synchronize()
        n = naccs[i].cpu().numpy()
        outcomes.append(algorithmic_bytes(w, n))
        acc.append(float(n.mean()))
    rot = [outcomes[k % args.copies] for k in range(args.steps)]
    alg_needed = float(np.mean([o["needed"] for o in rot]))
    alg_every = float(np.mean([o["every_row"] for o in rot]))
    step_s = ms_per_step / 1e3
    positions_per_s = w0.D / step_s
    per_request = False  # the library's default is the split path
    alg_path = alg_needed if per_request else alg_every
    eff_gbps = alg_path / step_s / 1e9

    # ---- per-kernel durations with events recorded around each kernel
    def kernel_times(path):
        nk = max(10, min(args.steps, 50))
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(nk)]
        for k in range(nk):
            call(k % args.copies, debug=rs.Debug(events=evs[k], sampling_path=path))
        torch.cuda.synchronize()
        return [float(np.mean([e[a].elapsed_time(e[a + 1]) for e in evs])) for a in range(3)]

    def timed_steps(path):
        dbg = rs.Debug(sampling_path=path)
        for k in range(args.warmup):
            call(k % args.copies, debug=dbg)
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        s0.record(stream)
        for k in range(args.steps):
            call(k % args.copies, debug=dbg)
        s1.record(stream)
        torch.cuda.synchronize()
        return s0.elapsed_time(s1) / args.steps

    t = kernel_times(0)
    if per_request:
        kernels = {"request_kernel": t[0] * 1e3}
        dom_name, dom_ms, dom_bytes = "request_kernel", t[0], alg_needed
    else:
        kernels = {"row_pass": t[0] * 1e3, "scan": t[1] * 1e3, "race_emit": t[2] * 1e3}
        dom_name, dom_ms = "row_pass_kernel", t[0]
        dom_bytes = float(np.mean([o["logits_every_row"] for o in rot]))
    dom_gbps = dom_bytes / (dom_ms / 1e3) / 1e9
    log(f"kernels (event-timed): " + ", ".join(f"{k} {v:.1f} us" for k, v in kernels.items()))
    log(f"{dom_name}: {dom_gbps:.0f} GB/s algorithmic ({dom_gbps / HBM_PEAK_GBPS:.1%} of 8 TB/s); "
        f"whole call {eff_gbps:.0f} GB/s; rows needed per call {[o['rows_needed'] for o in outcomes]} "
        f"of {w0.D + w0.B}; resampled rows {[o['n_res'] for o in outcomes]}; mean accepted {np.mean(acc):.3f}")

    # the split path (every row's statistics across the GPU, then scan, race, emit) for reference
    split = None
    if per_request:
        ms_split = timed_steps(2)
        ts = kernel_times(2)
        lg = float(np.mean([o["logits_every_row"] for o in rot]))
        split = {"ms_per_step": ms_split, "positions_per_s": w0.D / (ms_split / 1e3),
                 "achieved_GBps_every_row": alg_every / (ms_split / 1e3) / 1e9,
                 "kernel_us": {"row_pass": ts[0] * 1e3, "scan": ts[1] * 1e3, "race_emit": ts[2] * 1e3},
                 "row_pass_GBps": lg / (ts[0] / 1e3) / 1e9}
        log(f"split path: {ms_split * 1e3:.1f} us/step, {split['positions_per_s']:.3g} positions/s, row pass "
            f"{split['row_pass_GBps']:.0f} GB/s, kernels {split['kernel_us']}")

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
                   "path": "per-request" if per_request else "split", "parallelism": "single GPU"},
        "achieved_GBps": eff_gbps,
        "hbm_frac": eff_gbps / HBM_PEAK_GBPS,
        "algorithmic_bytes_per_step": {"path": alg_path, "needed": alg_needed, "every_row": alg_every},
        "kernel_us": kernels,
        "mean_accepted": float(np.mean(acc)),
        "roofline": {"bound": "hbm", "achieved": dom_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": dom_gbps / HBM_PEAK_GBPS, "traffic": None, "kernel": dom_name},
        "split_path": split,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
