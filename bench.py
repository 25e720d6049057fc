"""Benchmark of the KDA forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps 200] [--warmup 30] [--repeats 5]
                    [--workload c3] [--extra c4,c5] [--path auto]

One step = one full forward over the whole seeded synthetic batch, with inputs
already resident in HBM: the chunk map plus the single-pass kernel (path
"fused"), the single pass over time segments plus the segment scan and output
correction ("segmented"), or the chunk-parallel and recurrence kernels
("split"); "auto" is the library's own rule. Protocol of the FlashKDA
benchmarks (review page, section 3): W untimed warmup steps, then R repeats of
K timed steps (one kda_fwd call each), each repeat between two device
synchronisations; ms_per_step is the median over the repeats. After each
repeat the same K steps run again with HIP events recorded on the launch stream
around each stage call, which give each kernel's duration per step (a call's
interval also holds the few-microsecond chunk map and the launch gap); per
kernel the line reports the median over repeats of the per-repeat mean, and the
median and minimum over all instrumented steps. The events stay out of the
wall-clock repeats, since each lengthens a short step. The other path is then timed
the same way for comparison, and the extra workloads (default c4 and c5) get
sub-records of the same form. Prints ONE JSON line. Headline workload c3 (8
packed sequences x 8192 tokens, H=32, D=128, bf16), the metric's head count.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KDA fwd tokens/sec at H=32, D=128 bf16; % of MFMA/HBM roofline"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E peak
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 matrix peak
UNIT_BYTES = 18944           # workspace bytes per (chunk, head) unit, bf16 path
KET_BYTES = 4096             # K_end in K_b order per unit, look-ahead recurrence only
LOOK_MAX_PAIRS = 96          # fewer (sequence, head) pairs: look-ahead recurrence
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
# the chunked method's matrix work per token-head (D = 128, C = 16): the dense state
# contractions 6 D^2 (K_b S^T and Q_b S^T, 4 D^2; the update K_end^T E, 2 D^2), the 16 x 16
# block work 10 C D (K K^T, Q K^T, the factors, A^qk E) and the state decay D^2 / C
METHOD_FLOPS_PER_TOKEN_HEAD = 10 * 16 * 128 + 6 * 128 * 128 + 128 * 128 // 16  # 119808


def algorithmic_work(w, bf16_resident_state=False):
    """Bytes each kernel must move and the recurrence's matrix flops, per launch.

    Per (chunk, head) unit, 16 token rows of 128 channels:
      chunk-parallel kernel: reads q, k, g_raw (3 x 256 B per token-head) and
        beta_raw (2 B per token-head), writes one 18944 B workspace unit;
      recurrence kernel: reads the unit and v (256 B per token-head), writes o
        (256 B per token-head); per (sequence, head) it reads the 64 KiB fp32
        initial state (when given) and writes the 64 KiB final state;
      single-pass and token-by-token kernels: read q, k, g_raw, v and beta_raw
        (4 x 256 + 2 B per token-head), write o (256 B per token-head), and the
        states as above.
    Recurrence flops per unit (both paths): K_b S^T and Q_b S^T
    (2 x 2*16*128*128), the state update K_end^T E (2*128*16*128), A^kk E and
    A^qk E (2 x 2*16*16*128) and the decay (128*128).
    With fewer than 96 (sequence, head) pairs the two-kernel path runs the
    look-ahead recurrence: the chunk kernel also writes K_end in K_b order
    (4096 B per unit), the recurrence reads it and forms M = K_b K_end^T of the
    previous chunk (2*16*16*128 flops per unit).
    """
    H = w.H
    units = sum((L + 15) // 16 for L in w.seq_lens) * H
    th = w.T_tot * H
    st = w.N * H * 128 * 128 * 4 * (2 if w.initial_state is not None else 1)
    look = w.N * H < LOOK_MAX_PAIRS and not bf16_resident_state
    unit = UNIT_BYTES + (KET_BYTES if look else 0)
    k1 = th * (3 * 256 + 2) + units * unit
    k2 = units * unit + th * 512 + st
    kf = th * (4 * 256 + 2 + 256) + st
    flops = units * (3 * 2 * 16 * 128 * 128 + 2 * 2 * 16 * 16 * 128 + 128 * 128)
    flops_split = flops + (units * 2 * 16 * 16 * 128 if look else 0)
    # segmented pass: the single pass's inputs and outputs (the initial state read, if
    # given; the final state comes from the finish stage, whose only algorithmic bytes
    # are that write: its segment-state, transfer and y traffic is the price of the split)
    fin = w.N * H * 128 * 128 * 4
    seg = kf - fin
    return dict(units=units, k1_bytes=k1, k2_bytes=k2, kf_bytes=kf, flops=flops, flops_split=flops_split,
                seg_bytes=seg, fin_bytes=fin, method_flops=th * METHOD_FLOPS_PER_TOKEN_HEAD)


def traffic_for(kernel, workload):
    """Counter-measured HBM bytes per launch, if taken on the kernel's current sources."""
    from kimi_delta_attention_k1_amd.profsum import src_hash
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    ent = rec.get(workload, {}).get(kernel)
    if not ent or ent.get("src_sha256") != src_hash(kernel):
        return None
    return ent.get("bytes_per_launch")


def host_cpu():
    """Logical CPUs this process may use and the host CPU's model name."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count()
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return n, model


def cpu_baseline(w, nseq):
    """The fp64 oracle, untuned, on the first nseq sequences (all heads)."""
    import numpy as np  # noqa: F401
    import oracle
    offs = w.offsets()
    e = offs[nseq]
    f = lambda t: t[:e].float().numpy()  # noqa: E731
    s0 = None if w.initial_state is None else w.initial_state[:nseq].numpy()
    threads = min(nseq * w.H, oracle.max_threads())
    t = time.perf_counter()
    oracle.token_forward(f(w.q), f(w.k), f(w.v), f(w.g_raw), f(w.beta_raw), offs[:nseq + 1], s0,
                         lower_bound=w.lower_bound, threads=threads)
    dt = time.perf_counter() - t
    nproc, model = host_cpu()
    return {"value": e / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "nproc": nproc, "cpu_model": model,
            "sample": f"{w.name}: first {nseq} of {w.N} sequences ({e} tokens x {w.H} heads), fp64 token "
                      f"recurrence, OpenMP over the {nseq * w.H} (sequence, head) pairs, {dt:.2f} s wall"}


def _median(xs):
    xs = sorted(xs)
    n = len(xs)
    return xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])


def time_path(call, path, steps, warmup, repeats):
    """Warm up, then per repeat: `steps` plain forwards (one kda_fwd call each)
    between two device synchronisations, then as many again with HIP events
    around each stage call. Returns the wall ms per step of each plain run and,
    per kernel call, its event-measured ms of every instrumented step (grouped by
    repeat). The events stay out of the wall-clock runs: each is a timestamp the
    stream stops for, which lengthens a short step by up to ~12% (C2)."""
    import torch
    if path in ("fused", "recurrent"):
        stages = [("kf_fused" if path == "fused" else "kr_recurrent", call.run)]
    elif path == "segmented":  # chunk map + single pass over segments; segment scan + output correction
        stages = [("kf_fused_seg", call.seg_pass), ("kseg_finish", call.seg_finish)]
    else:
        stages = [("k1_mfma", call.prepare), ("k2_mfma", call.recur)]
    for _ in range(warmup):
        call.run()
    stream = torch.cuda.current_stream()
    walls, kern = [], {name: [] for name, _ in stages}
    for _ in range(repeats):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            call.run()
        torch.cuda.synchronize()
        walls.append((time.perf_counter() - t0) * 1e3 / steps)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(steps)]
        for i in range(steps):
            ev[i][0].record(stream)
            for j, (_, fn) in enumerate(stages):
                fn()
                ev[i][j + 1].record(stream)
        torch.cuda.synchronize()
        for j, (name, _) in enumerate(stages):
            kern[name].append([e[j].elapsed_time(e[j + 1]) for e in ev])
    return walls, kern


def pick_path(kda, w, path):
    """The library's rule (include/kda.h) for an unforced call."""
    if path != "auto":
        return path
    if w.T_tot <= kda.RECURRENT_MAX_AVG_TOKENS * w.N:
        return "recurrent"
    n_c = sum((L + 15) // 16 for L in w.seq_lens) if not w.packed else (w.T_tot + 15 * w.N) // 16
    pairs = w.N * w.H
    seg_min = kda.SEGMENTED_MIN_AVG_CHUNKS_FEW_PAIRS if pairs <= kda.SEGMENTED_FEW_PAIRS else kda.SEGMENTED_MIN_AVG_CHUNKS
    if pairs <= kda.SEGMENTED_MAX_PAIRS and n_c >= seg_min * w.N:
        return "segmented"
    if w.N * w.H >= kda.FUSED_MIN_PAIRS or n_c <= kda.FUSED_MAX_AVG_CHUNKS * w.N:
        return "fused"
    return "split"


def to_device(w, dev):
    q, k, v, g, b = (t.to(dev) for t in (w.q, w.k, w.v, w.g_raw, w.beta_raw))
    s0 = None if w.initial_state is None else w.initial_state.to(dev)
    cu = w.cu_seqlens().to(dev) if w.packed else None
    if not w.packed:
        shp = (w.N, w.seq_lens[0], w.H, 128)
        q, k, v, g = (t.view(shp) for t in (q, k, v, g))
        b = b.view(shp[:3])
    return q, k, v, g, b, s0, cu


def kernel_records(w, name, kern, bf16_resident_state=False):
    """Per-kernel figures from the event times, against the algorithmic work."""
    work = algorithmic_work(w, bf16_resident_state=bf16_resident_state)
    bytes_of = {"k1_mfma": work["k1_bytes"], "k2_mfma": work["k2_bytes"], "kf_fused": work["kf_bytes"],
                "kr_recurrent": work["kf_bytes"], "kf_fused_seg": work["seg_bytes"],
                "kseg_finish": work["fin_bytes"]}
    flops_of = {"k2_mfma": work["flops_split"], "kf_fused": work["method_flops"],
                "kf_fused_seg": work["method_flops"]}
    per_kernel, avg = {}, {}
    for kname, reps in kern.items():
        ms = _median([sum(r) / len(r) for r in reps])  # median over repeats of the per-repeat mean
        steps = [x for r in reps for x in r]
        avg[kname] = ms
        gbs = bytes_of[kname] / (ms * 1e-3) / 1e9
        ent = {"avg_ms": round(ms, 4), "step_median_ms": round(_median(steps), 4),
               "step_min_ms": round(min(steps), 4), "algorithmic_bytes": bytes_of[kname],
               "achieved_GBps": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
        if kname in flops_of:
            fl = flops_of[kname]
            tf = fl / (ms * 1e-3) / 1e12
            ent.update({"algorithmic_flops": fl, "achieved_TFLOPs": round(tf, 2),
                        "mfma_frac": round(tf / BF16_PEAK_TFLOPS, 4)})
        per_kernel[kname] = ent
    dom = max(avg, key=avg.get)
    d = per_kernel[dom]
    roofline = {"bound": "hbm", "kernel": dom, "achieved": d["achieved_GBps"], "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": d["hbm_frac"], "traffic": traffic_for(dom, name)}
    return per_kernel, roofline, work


def bench_workload(kda, workloads, name, path, args, dev, compare_other=False):
    """Time one workload; returns (record, workload)."""
    import torch
    w = workloads.CONFIGS[name]()
    path = "split" if args.bf16_resident_state else pick_path(kda, w, path)
    q, k, v, g, b, s0, cu = to_device(w, dev)
    call = kda.prepare_call(q, k, v, g, b, lower_bound=w.lower_bound, initial_state=s0, cu_seqlens=cu, path=path,
                            bf16_resident_state=args.bf16_resident_state)
    torch.cuda.synchronize()
    walls, kern = time_path(call, path, args.steps, args.warmup, args.repeats)
    ms = _median(walls)
    per_kernel, roofline, work = kernel_records(w, name, kern, args.bf16_resident_state)
    step_ev = [sum(x) for x in zip(*[[t for r in reps for t in r] for reps in kern.values()])]
    e2e = work["kf_bytes"] / (ms * 1e-3) / 1e9
    rec = {"path": path + (" (bf16-resident state)" if args.bf16_resident_state else ""),
           "tokens": w.T_tot, "heads": w.H, "sequences": w.N,
           "ms_per_step": round(ms, 4), "tokens_per_s": round(w.T_tot / (ms * 1e-3), 1),
           "repeat_ms_per_step": [round(x, 4) for x in walls],
           "event_ms_per_step": {"median": round(_median(step_ev), 4), "min": round(min(step_ev), 4)},
           "e2e_algorithmic_hbm_frac": round(e2e / HBM_PEAK_GBS, 4),
           "kernels": per_kernel, "roofline": roofline}
    if compare_other and args.compare_steps > 0:
        other = "split" if path != "split" else "fused"
        oc = kda.prepare_call(q, k, v, g, b, lower_bound=w.lower_bound, initial_state=s0, cu_seqlens=cu,
                              path=other)
        o_walls, o_kern = time_path(oc, other, args.compare_steps, min(args.warmup, 10), 1)
        rec["path_compare"] = {"path": other, "steps": args.compare_steps, "ms_per_step": round(o_walls[0], 4),
                               "tokens_per_s": round(w.T_tot / (o_walls[0] * 1e-3), 1),
                               "kernels_avg_ms": {n: round(sum(r[0]) / len(r[0]), 4) for n, r in o_kern.items()}}
        del oc
    del call, q, k, v, g, b, s0, cu
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec, w


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--repeats", type=int, default=5, help="timed repeats of --steps steps; the median is reported")
    ap.add_argument("--workload", default="c3", choices=["c2", "c3", "c4", "c5", "d1"])
    ap.add_argument("--extra", default="c4,c5",
                    help="comma-separated workloads timed after the headline one, as sub-records ('' skips)")
    ap.add_argument("--path", default="auto", choices=["auto", "fused", "split", "recurrent", "segmented"],
                    help="kernels of the headline workload's step (auto: the library's rule)")
    ap.add_argument("--bf16-resident-state", action="store_true",
                    help="two-kernel path with the recurrence's state rounded to bf16 between chunks")
    ap.add_argument("--compare-steps", type=int, default=100,
                    help="steps of the other path, timed afterwards for comparison (0: skip)")
    ap.add_argument("--cpu-seqs", type=int, default=2, help="sequences in the CPU-baseline sample (0: skip)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run a plain device copy of this size (counter calibration)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: the KDA forward runs on a single GPU; multi-GPU runs are not supported (--gpus must be 1)",
              file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.repeats < 1 or args.warmup < 0:
        print("bench.py: --steps and --repeats must be >= 1, --warmup >= 0", file=sys.stderr)
        sys.exit(2)

    import torch
    import kimi_delta_attention_k1_amd as kda
    from kimi_delta_attention_k1_amd import workloads

    dev = torch.device("cuda:0")
    head, w = bench_workload(kda, workloads, args.workload, args.path, args, dev, compare_other=True)
    extra = {}
    for name in [x for x in args.extra.split(",") if x and x != args.workload]:
        extra[name], _ = bench_workload(kda, workloads, name, "auto", args, dev)
        extra[name]["workload"] = f"{name}: {workloads.DESCRIPTIONS[name]}"

    if args.copy_probe_mib:
        src = torch.empty(args.copy_probe_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    ms = head["ms_per_step"]
    line = {
        "metric": METRIC, "value": head["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "repeats": args.repeats, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded CPU torch.Generator, N(0,1) family; see workloads.py)",
        "config": {"workload": f"{args.workload}: {workloads.DESCRIPTIONS[args.workload]}",
                   "tokens": w.T_tot, "heads": w.H, "head_dim": 128, "sequences": w.N, "chunk": 16,
                   "lower_bound": w.lower_bound, "path": head["path"]},
        "repeat_ms_per_step": head["repeat_ms_per_step"],
        "event_ms_per_step": head["event_ms_per_step"],
        "e2e_algorithmic_hbm_frac": head["e2e_algorithmic_hbm_frac"],
        "kernels": head["kernels"],
        "roofline": head["roofline"],
    }
    if "path_compare" in head:
        line["path_compare"] = head["path_compare"]
    if extra:
        line["workloads"] = extra
    if args.cpu_seqs > 0:
        line["cpu_baseline"] = cpu_baseline(w, min(args.cpu_seqs, w.N))
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
