#!/usr/bin/env python3
"""Decode-step throughput on one MI355X: positions/s of dlm_decode_step.

One step = LM head over every row of the block + confidence/candidate +
commit policy + state update: one launch of the fused kernel.  The
default workload is B=1, L=32, H=2048, V=126464, bf16, threshold 0.9.

Inputs are seeded and synthetic and already resident in HBM when the timed
region starts.  An untimed pass first records the trajectory: which
(block, iteration) each sequence sits at, step by step, with automatic
block advance.  The timed pass replays the same inputs from the same
initial state.  The kernels are deterministic, so it follows the same
trajectory without a host round trip between steps.

Prints ONE JSON line (rank 0).  Extra keys: ``roofline`` for the step kernel
(algorithmic bytes / measured time, against 8 TB/s HBM or 2.5 PFLOP/s
bf16 MFMA) and ``cpu_baseline`` (the CPU oracle on a bounded sample).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16
MFMA_FP32_PEAK_TFLOPS = 157.3
METRIC = "decode-step positions/sec (LM head+confidence+commit), B=1 L=32; % HBM/MFMA peak"


def algorithmic_work(wl, topk=0):
    """Bytes the step must move and flops it must do (the [M][V] logits are never stored)."""
    es = 2 if wl.dtype == "bf16" else 4
    M = wl.B * wl.L
    any_credit = any(p.kind == 2 for p in wl.policies)
    state = M * (1 + 1 + 4 + 1 + 4 + 4)            # mask in/out, tokens, commit, conf, gap
    if any_credit:
        state += 2 * M * 4 * 8                     # credit slots in/out
    state += M * topk * 8                          # top-k tokens and probabilities
    bytes_ = wl.V * wl.H * es + M * wl.H * es + state
    flops = 2.0 * M * wl.V * wl.H
    return bytes_, flops


def measured_traffic(workload):
    """HBM bytes per launch from the committed counter summary, if it matches these kernel sources."""
    from decoding_step_amd.traffic import kernel_source_hash
    path = os.path.join(ROOT, "profiles", f"{workload}_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def record_trajectory(wl, W, Wd, steps, dev, topk=0):
    """Untimed: step once per input with host sync, recording the inputs each step consumed."""
    import numpy as np
    import torch
    from decoding_step_amd import _native as nat
    from decoding_step_amd.device import Decoder, new_credit, to_device
    from decoding_step_amd.synth import BlockStream

    seq = [(p.kind, p.threshold, p.decay, p.max_depth) for p in wl.policies]
    dec = Decoder(Wd, wl.B, wl.L, seq, flags=nat.DLM_AUTO_ADVANCE, topk=topk)
    streams = [BlockStream(W, wl.L, s, wl.a_max, rp) for s, rp in zip(wl.seeds, wl.redraw_p)]
    pos = [[0, 0] for _ in range(wl.B)]
    mask = torch.ones((wl.B, wl.L), dtype=torch.uint8, device=dev)
    credit = new_credit(wl.B, wl.L, dev)
    hidden = torch.empty((steps, wl.B, wl.L, wl.H), dtype=Wd.dtype, device=dev)
    commits = 0
    for s in range(steps):
        h = np.stack([streams[b].hidden(*pos[b]) for b in range(wl.B)])
        hidden[s].copy_(to_device(h, dev))
        dec.step(hidden[s], mask, credit)
        m = mask.cpu().numpy()
        commits += int(dec.out_commit.sum().item())
        for b in range(wl.B):
            pos[b] = [pos[b][0] + 1, 0] if not m[b].any() else [pos[b][0], pos[b][1] + 1]
    blocks_done = sum(p[0] for p in pos)
    return hidden, seq, commits, blocks_done


def time_steps_device_loop(wl, Wd, hidden, seq, warmup, steps, dev, graph, topk=0):
    """All timed steps in one dlm_decode_steps call (optionally captured once as a graph and replayed)."""
    import torch
    from decoding_step_amd import _native as nat
    from decoding_step_amd.device import Decoder, new_credit

    stream = torch.cuda.Stream(dev) if graph else torch.cuda.current_stream(dev)
    dec = Decoder(Wd, wl.B, wl.L, seq, flags=nat.DLM_AUTO_ADVANCE, stream=stream, topk=topk)
    mask = torch.ones((wl.B, wl.L), dtype=torch.uint8, device=dev)
    credit = new_credit(wl.B, wl.L, dev)
    credit0 = credit.clone()
    tok = torch.empty((steps, wl.B, wl.L), dtype=torch.int32, device=dev)
    com = torch.empty((steps, wl.B, wl.L), dtype=torch.uint8, device=dev)
    tk_tok = torch.empty((steps, wl.B, wl.L, topk), dtype=torch.int32, device=dev) if topk else None
    tk_prob = torch.empty((steps, wl.B, wl.L, topk), dtype=torch.float32, device=dev) if topk else None
    run = lambda: dec.steps(hidden[:steps], mask, credit, tok, com, tk_tok, tk_prob)
    with torch.cuda.stream(stream):
        for _ in range(max(1, warmup // max(1, steps))):
            run()
    torch.cuda.synchronize()
    if graph:
        g = torch.cuda.CUDAGraph()
        mask.fill_(1)
        credit.copy_(credit0)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=stream):
            run()
        run = g.replay
        stream = torch.cuda.current_stream(dev)
        dec.policy.set_stream(stream)
    mask.fill_(1)
    credit.copy_(credit0)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    with torch.cuda.stream(stream):
        run()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return ev0.elapsed_time(ev1) / 1e3, wall, None


def time_steps(wl, Wd, hidden, seq, warmup, steps, dev, topk=0, time_head=False):
    """One dlm_decode_step call per step.  The region is timed with two events only; a second
    pass over the same steps records an event between consecutive steps for the per-step
    distribution (those events add ~3 us to each step, so the rate comes from the first pass).
    With time_head, a third pass has the library record an event pair around the vocabulary-head
    kernel of every step (dlm_policy.head_events): that kernel's own durations, in us."""
    import torch
    from decoding_step_amd import _native as nat
    from decoding_step_amd.device import Decoder, new_credit

    stream = torch.cuda.current_stream(dev)
    dec = Decoder(Wd, wl.B, wl.L, seq, flags=nat.DLM_AUTO_ADVANCE, stream=stream, topk=topk)
    mask = torch.ones((wl.B, wl.L), dtype=torch.uint8, device=dev)
    credit = new_credit(wl.B, wl.L, dev)
    credit0 = credit.clone()
    for s in range(warmup):                      # warm-up on the first inputs, then reset the state
        dec.step(hidden[s % hidden.shape[0]], mask, credit)
    torch.cuda.synchronize()

    def reset():
        mask.fill_(1)
        credit.copy_(credit0)
        torch.cuda.synchronize()

    reset()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for s in range(steps):
        dec.step(hidden[s], mask, credit)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total = start.elapsed_time(end) / 1e3
    reset()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for s in range(steps):
        dec.step(hidden[s], mask, credit)
        ev[s + 1].record(stream)
    torch.cuda.synchronize()
    per_step = [ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(steps)]   # us
    head = None
    if time_head:
        reset()
        hb = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        he = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        for s in range(steps):
            dec.policy.set_head_events(hb[s], he[s])
            dec.step(hidden[s], mask, credit)
        dec.policy.set_head_events(None, None)
        torch.cuda.synchronize()
        head = [hb[i].elapsed_time(he[i]) * 1e3 for i in range(steps)]
    return total, wall, per_step, head


def time_shard_share(wl, W, hidden, seq, warmup, steps, dev, G):
    """One GPU's share of a step of the head split over G vocabulary shards: dlm_shard_stats on a
    V/G-row shard, then dlm_merge_commit over G record sets (the other G-1 sets come from the other
    shards on the first input; the exchange that would deliver them is not part of this timing).
    Returns (total seconds, shard-kernel seconds, merge seconds) from HIP events on the stream."""
    import numpy as np
    import torch
    from decoding_step_amd import _native as nat
    from decoding_step_amd.device import new_credit, to_device, torch_dtype_code

    cuts = [wl.V * g // G for g in range(G + 1)]
    M = wl.B * wl.L
    stream = torch.cuda.current_stream(dev)
    W_sh = [to_device(np.ascontiguousarray(W[a:b]), dev) for a, b in zip(cuts[:-1], cuts[1:])]
    code = torch_dtype_code(W_sh[0])
    pols = []
    for (a, b), w in zip(zip(cuts[:-1], cuts[1:]), W_sh):
        ws = torch.zeros(nat.dlm_workspace_bytes(wl.B, wl.L, wl.H, b - a, code), dtype=torch.uint8, device=dev)
        pols.append(nat.StepPolicy(wl.B, wl.L, wl.H, b - a, code, seq, ws, stream=stream))
    records = torch.empty((G, M, 4), dtype=torch.float32, device=dev)
    for g in range(G):                                  # the records the exchange would deliver
        nat.dlm_shard_stats(hidden[0], W_sh[g], cuts[g], pols[g], records[g])
    merge = nat.StepPolicy(wl.B, wl.L, wl.H, wl.V, code, seq, flags=nat.DLM_AUTO_ADVANCE, stream=stream)
    tok = torch.empty((wl.B, wl.L), dtype=torch.int32, device=dev)
    com = torch.empty((wl.B, wl.L), dtype=torch.uint8, device=dev)
    mask = torch.ones((wl.B, wl.L), dtype=torch.uint8, device=dev)
    credit = new_credit(wl.B, wl.L, dev)

    def one(s):
        nat.dlm_shard_stats(hidden[s], W_sh[0], 0, pols[0], records[0])
        nat.dlm_merge_commit(records, G, mask, credit, merge, tok, com)

    for s in range(warmup):
        one(s % hidden.shape[0])
    mask.fill_(1)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    ev[0].record(stream)
    for s in range(steps):
        one(s)
    ev[1].record(stream)
    torch.cuda.synchronize()
    total = ev[0].elapsed_time(ev[1]) / 1e3
    # the two kernels apart: the shard kernel alone over the same inputs, then the merge alone
    ev[0].record(stream)
    for s in range(steps):
        nat.dlm_shard_stats(hidden[s], W_sh[0], 0, pols[0], records[0])
    ev[1].record(stream)
    for s in range(steps):
        nat.dlm_merge_commit(records, G, mask, credit, merge, tok, com)
    ev[2].record(stream)
    torch.cuda.synchronize()
    return total, ev[0].elapsed_time(ev[1]) / 1e3, ev[1].elapsed_time(ev[2]) / 1e3, cuts[1] - cuts[0]


def time_vendor_gemm(Wd, hidden, warmup, steps):
    """The bare contraction of the same rows with the same W by the vendor library: torch.mm,
    which ROCm's torch hands to hipBLASLt, writing the [B*L][V] logits to HBM in bf16 and
    computing no statistics.  A reference point for the fused head, not part of the step."""
    import torch
    n, B, L, H = hidden.shape
    x = hidden.reshape(n, B * L, H)
    out = torch.empty((B * L, Wd.shape[0]), dtype=Wd.dtype, device=Wd.device)
    for i in range(warmup):
        torch.mm(x[i % n], Wd.t(), out=out)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(steps):
        torch.mm(x[i % n], Wd.t(), out=out)
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps * 1e3          # us per call


def measure_ceilings(dev):
    """Practical ceilings of this GPU by vendor routines, beside the published peaks: a 2 GiB
    device-to-device copy (HBM read + write), a float32-accumulated sum over 2 GiB of bf16 (HBM
    read), and torch.mm of two 8192 x 8192 bf16 matrices (hipBLASLt)."""
    import torch

    def per_call(f, n, warm=5):
        for _ in range(warm):
            f()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(n):
            f()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / n * 1e-3

    nbytes = 1 << 31
    a = torch.ones(nbytes // 2, dtype=torch.bfloat16, device=dev)
    b = torch.empty_like(a)
    s_copy = per_call(lambda: b.copy_(a), 20)
    s_sum = per_call(lambda: a.sum(dtype=torch.float32), 20)
    del b
    n = 8192
    x = torch.randn(n, n, dtype=torch.bfloat16, device=dev)
    y = torch.randn(n, n, dtype=torch.bfloat16, device=dev)
    z = torch.empty(n, n, dtype=torch.bfloat16, device=dev)
    s_mm = per_call(lambda: torch.mm(x, y, out=z), 20)
    return {
        "copy_GBps": 2 * nbytes / s_copy / 1e9, "copy_frac_of_hbm_peak": 2 * nbytes / s_copy / 1e9 / HBM_PEAK_GBS,
        "read_sum_GBps": nbytes / s_sum / 1e9, "read_sum_frac_of_hbm_peak": nbytes / s_sum / 1e9 / HBM_PEAK_GBS,
        "mm8192_bf16_TFLOPs": 2 * n ** 3 / s_mm / 1e12,
        "mm8192_frac_of_mfma_peak": 2 * n ** 3 / s_mm / 1e12 / MFMA_BF16_PEAK_TFLOPS,
        "note": "torch copy_, sum(dtype=float32) and mm (hipBLASLt) on this GPU; 20 calls after 5 untimed",
    }


def cpu_baseline(wl, W, budget_s=20.0, topk=0):
    """The oracle as it stands, on the first steps of the same workload, on this host's cores
    (with the top-k export, the oracle's topk_candidates over the same rows is part of a step)."""
    import numpy as np
    import oracle
    from decoding_step_amd.synth import BlockStream

    from threadpoolctl import threadpool_info, threadpool_limits
    threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    seq = [(p.kind, p.threshold, p.decay, p.max_depth) for p in wl.policies]
    # the oracle's exact float64 values of W, widened once before any timing (as the parity tests
    # do): a weight conversion per step would be timed as oracle work
    W64 = oracle.as_f64(W)
    streams = [BlockStream(W, wl.L, s, wl.a_max, rp) for s, rp in zip(wl.seeds, wl.redraw_p)]
    mask = np.ones((wl.B, wl.L), np.uint8)
    ctok = np.full((wl.B, wl.L, 4), -1, np.int32)
    cval = np.zeros((wl.B, wl.L, 4), np.float32)
    pos = [[0, 0] for _ in range(wl.B)]
    n, t = 0, 0.0
    while t < budget_s and n < 4096:
        h = np.stack([streams[b].hidden(*pos[b]) for b in range(wl.B)])
        t0 = time.perf_counter()
        out = oracle.decode_step(h, W64, mask, seq, ctok, cval, auto_advance=True)
        if topk:
            oracle.topk_candidates(h, W64, topk)
        t += time.perf_counter() - t0
        mask, ctok, cval = out["mask"], out["credit_tok"], out["credit_val"]
        for b in range(wl.B):
            pos[b] = [pos[b][0] + 1, 0] if not mask[b].any() else [pos[b][0], pos[b][1] + 1]
        n += 1
    # the same oracle on one thread, on the first step only
    h = np.stack([BlockStream(W, wl.L, sd, wl.a_max, rp).hidden(0, 0) for sd, rp in zip(wl.seeds, wl.redraw_p)])
    with threadpool_limits(limits=1, user_api="blas"):
        t1 = time.perf_counter()
        oracle.decode_step(h, W64, np.ones((wl.B, wl.L), np.uint8), seq, np.full((wl.B, wl.L, 4), -1, np.int32),
                           np.zeros((wl.B, wl.L, 4), np.float32), auto_advance=True)
        if topk:
            oracle.topk_candidates(h, W64, topk)
        t1 = time.perf_counter() - t1
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:  # pragma: no cover
        pass
    return {"value": wl.B * wl.L * n / t, "unit": "positions/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {n} steps of {wl.name} (whole steps, all {wl.B * wl.L} rows), {t:.1f} s; "
                      f"W widened to float64 once, before the timed steps",
            "one_thread_value": wl.B * wl.L / t1, "affinity_cpus": len(os.sched_getaffinity(0)), "cpu_model": model}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # Sustained back-to-back steps meet a clock transient: a few milliseconds into a burst the
    # step slows (by up to ~40% for the 512-row head) and recovers over ~20 ms.  300 warm-up
    # steps (26 ms at B=1 L=32, ~90 ms at 512 rows) put the timed steps in the settled state.
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--workload", default="threshold_b1_l32")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--loop", choices=["calls", "steps", "graph"], default="calls",
                    help="one dlm_decode_step call per step (default), all timed steps in one "
                         "dlm_decode_steps call, or that call captured as a graph and replayed")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle time")
    ap.add_argument("--topk", type=int, default=0,
                    help="also export the k best candidates of every row (0 = off, at most 8)")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="also time the vendor library's plain GEMM (torch.mm -> hipBLASLt) on the same "
                         "rows and W, bf16 logits out, no statistics (GEMM-shaped workloads only)")
    ap.add_argument("--ceilings", action="store_true",
                    help="only measure this GPU's practical ceilings with vendor routines (HBM copy and read, "
                         "an 8192^3 bf16 GEMM) and print them as one JSON line")
    ap.add_argument("--shards", type=int, default=1,
                    help="time one GPU's share of a head split over this many vocabulary shards "
                         "(shard kernel + merge of the shards' records; the exchange is not timed)")
    args = ap.parse_args()
    if not 0 <= args.topk <= 8:
        ap.error("--topk must be in 0..8")
    if not 1 <= args.shards <= 256 or (args.shards > 1 and args.topk):
        ap.error("--shards must be in 1..256, and the shard calls have no top-k export")
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the step shards by sequence or by vocabulary range; see the design notes).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from decoding_step_amd import _native as nat
    from decoding_step_amd.device import to_device
    from decoding_step_amd.synth import make_weights
    from decoding_step_amd.workloads import WORKLOADS

    nat.load()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.ceilings:
        print(json.dumps({"ceilings": measure_ceilings(dev), "hbm_peak_GBps": HBM_PEAK_GBS,
                          "mfma_bf16_peak_TFLOPs": MFMA_BF16_PEAK_TFLOPS}), flush=True)
        return
    wl = WORKLOADS[args.workload]
    if args.vendor_gemm and (args.shards > 1 or not (wl.dtype == "bf16" and wl.B * wl.L > 64 and wl.H % 256 == 0)):
        ap.error("--vendor-gemm needs a GEMM-shaped workload (bf16, B*L > 64) and no --shards")
    print(f"[bench] workload {wl.name}: generating W ({wl.V}x{wl.H} {wl.dtype})", file=sys.stderr, flush=True)
    W = make_weights(wl.V, wl.H, wl.dtype)
    Wd = to_device(W, dev)
    n_in = max(args.steps, 1)
    print(f"[bench] recording {n_in} steps", file=sys.stderr, flush=True)
    hidden, seq, commits, blocks = record_trajectory(wl, W, Wd, n_in, dev, args.topk)
    print(f"[bench] timing {args.steps} steps after {args.warmup} warm-up", file=sys.stderr, flush=True)
    if args.shards > 1:
        total, t_shard, t_merge, v_shard = time_shard_share(wl, W, hidden, seq, args.warmup, args.steps, dev,
                                                             args.shards)
        es = 2 if wl.dtype == "bf16" else 4
        M = wl.B * wl.L
        shard_bytes = v_shard * wl.H * es + M * wl.H * es + M * 16
        per = total / args.steps
        out = {
            "metric": METRIC + " -- one GPU's share of a vocabulary-sharded step",
            "value": M / per, "unit": "positions/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": per * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": wl.dtype, "data": "synthetic (seeded generator: W ~ N(0,0.02), planted-peak hidden states)",
            "config": {"workload": wl.name, "B": wl.B, "L": wl.L, "H": wl.H, "V": wl.V, "shards": args.shards,
                       "shard_rows": v_shard,
                       "share": "dlm_shard_stats on one shard + dlm_merge_commit over all shards' records; "
                                "the all-gather between them is not timed"},
            "roofline": {"bound": "hbm", "kernel": "dlm_shard_stats (shard-shaped LM head)",
                         "achieved": shard_bytes / (t_shard / args.steps) / 1e9, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": shard_bytes / (t_shard / args.steps) / 1e9 / HBM_PEAK_GBS,
                         "traffic": measured_traffic(f"{wl.name}_shard{args.shards}"),
                         "algorithmic_bytes_per_launch": shard_bytes},
            "shard_us": t_shard / args.steps * 1e6, "merge_commit_us": t_merge / args.steps * 1e6,
            "cpu_baseline": None,
        }
        print(json.dumps(out), flush=True)
        return
    gemm_path = wl.dtype == "bf16" and wl.B * wl.L > 64 and wl.H % 256 == 0
    one_kernel = not gemm_path                            # the step is the head kernel itself
    head = None
    if args.loop == "calls":
        t, wall, per_step, head = time_steps(wl, Wd, hidden, seq, args.warmup, args.steps, dev, args.topk,
                                             time_head=not one_kernel)
    else:
        t, wall, per_step = time_steps_device_loop(wl, Wd, hidden, seq, args.warmup, args.steps, dev,
                                                   graph=args.loop == "graph", topk=args.topk)
    ms = t / args.steps * 1e3
    bytes_, flops = algorithmic_work(wl, args.topk)
    sec_per_step = t / args.steps
    # the head kernel's average duration: the step itself when it is one kernel, else the
    # event pair the library records around that kernel (third pass over the same steps)
    sec_head = sec_per_step if head is None else float(np.mean(head)) * 1e-6
    if flops / bytes_ > 312 and wl.dtype == "bf16":
        roof = {"bound": "mfma", "achieved": flops / sec_head / 1e12, "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": bytes_ / sec_head / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(wl.name + (f"_topk{args.topk}" if args.topk else ""))
    if args.topk and one_kernel:
        roof["kernel"] = "dlm::step_kernel with the top-k fold (one launch per step)"
    elif gemm_path:
        gemm = ("dlm::gemm_r512_topk_kernel" if args.topk else
                "dlm::gemm_r512_kernel" if wl.B * wl.L > 256 else "dlm::gemm_r256_kernel")
        roof["kernel"] = gemm + " (the step also holds pack_hidden_kernel and finalize_parts_kernel)"
    else:
        roof["kernel"] = "dlm::step_kernel (one launch per step)"
    if head is not None:
        roof["kernel_us"] = float(np.mean(head))
        roof["timing"] = ("head kernel alone: mean of per-step event pairs the library records around it "
                          "(a pass over the same steps after the timed one)")
        roof["step_frac"] = (flops / sec_per_step / 1e12 if roof["bound"] == "mfma"
                             else bytes_ / sec_per_step / 1e9) / roof["peak"]
    elif one_kernel or args.loop != "calls":
        roof["timing"] = ("whole step over the timed region" + (" (one kernel per step)" if one_kernel else
                          " (the step's other kernels included)"))
    roof["algorithmic_bytes_per_launch"] = bytes_
    roof["algorithmic_flops_per_launch"] = flops
    out = {
        "metric": METRIC, "value": wl.B * wl.L / sec_per_step, "unit": "positions/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype,
        "data": "synthetic (seeded generator: W ~ N(0,0.02), planted-peak hidden states)",
        "config": {"workload": wl.name, "B": wl.B, "L": wl.L, "H": wl.H, "V": wl.V,
                   "policies": sorted(set(f"{['threshold', 'hierarchical', 'credit'][p.kind]} {p.threshold}"
                                          for p in wl.policies)),
                   "topk": args.topk},
        "roofline": roof,
        "step_us": None if per_step is None else {
            "median": float(np.median(per_step)), "p10": float(np.percentile(per_step, 10)),
            "p90": float(np.percentile(per_step, 90)),
            "note": "second pass with an event between steps (each event adds ~3 us)"},
        "loop": args.loop,
        "committed_tok_per_s": commits / args.steps / sec_per_step,
        "per_sequence_tok_per_s": commits / args.steps / sec_per_step / wl.B,
        "blocks_completed": blocks,
        "host_wall_s": wall,
    }
    if args.vendor_gemm:
        print("[bench] timing the vendor GEMM on the same operands", file=sys.stderr, flush=True)
        us = time_vendor_gemm(Wd, hidden, args.warmup, args.steps)
        out["vendor_gemm"] = {
            "kernel": "torch.mm (hipBLASLt): [B*L][H] x [H][V] -> bf16 logits in HBM, no statistics",
            "us": us, "tflops": flops / (us * 1e-6) / 1e12, "frac": flops / (us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
            "fused_head_speedup": None if head is None else us / float(np.mean(head))}
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(wl, W, args.cpu_budget, args.topk)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
