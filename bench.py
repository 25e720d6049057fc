"""Benchmark of the KDA forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps 200] [--warmup 30] [--workload c3] [--path auto]

One step = one full forward over the whole seeded synthetic batch, with inputs
already resident in HBM: the chunk map plus either the single-pass kernel
(path "fused") or the chunk-parallel and recurrence kernels (path "split");
"auto" is the library's own rule. W untimed warmup steps, then K timed steps
between two device synchronisations; HIP events recorded on the launch stream
around each kernel call give each kernel's average duration inside the same
timed region (the fused call's interval also holds the few-microsecond chunk
map). The other path is then timed the same way for comparison. Prints ONE
JSON line. Default workload c3 (8 packed sequences x 8192 tokens, H=32,
D=128, bf16), the headline metric's head count.
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
UNIT_BYTES = 14848           # workspace bytes per (chunk, head) unit, bf16 path
KET_BYTES = 4096             # K_end in K_b order per unit, look-ahead recurrence only
LOOK_MAX_PAIRS = 96          # fewer (sequence, head) pairs: look-ahead recurrence
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")


def algorithmic_work(w, bf16_resident_state=False):
    """Bytes each kernel must move and the recurrence's matrix flops, per launch.

    Per (chunk, head) unit, 16 token rows of 128 channels:
      chunk-parallel kernel: reads q, k, g_raw (3 x 256 B per token-head) and
        beta_raw (2 B per token-head), writes one 14848 B workspace unit;
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
                seg_bytes=seg, fin_bytes=fin)


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
    return {"value": e / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{w.name}: first {nseq} of {w.N} sequences ({e} tokens x {w.H} heads), fp64 token "
                      f"recurrence, {dt:.2f} s wall"}


def time_path(call, path, steps, warmup):
    """Run `steps` timed forwards on `path`; returns wall ms per step and the
    event-measured average ms of each kernel call."""
    import torch
    if path in ("fused", "recurrent"):
        stages = [("kf_fused" if path == "fused" else "kr_recurrent", call.run)]
    elif path == "segmented":  # chunk map + single pass over segments; segment scan + output correction
        stages = [("kf_fused_seg", call.seg_pass), ("kseg_finish", call.seg_finish)]
    else:
        stages = [("k1_mfma", call.prepare), ("k2_mfma", call.recur)]
    for _ in range(warmup):
        for _, fn in stages:
            fn()
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record(stream)
        for j, (_, fn) in enumerate(stages):
            fn()
            ev[i][j + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern = {name: sum(e[j].elapsed_time(e[j + 1]) for e in ev) / steps for j, (name, _) in enumerate(stages)}
    return wall * 1e3 / steps, kern


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="c3", choices=["c2", "c3", "c4", "c5", "d1"])
    ap.add_argument("--path", default="auto", choices=["auto", "fused", "split", "recurrent", "segmented"],
                    help="kernels of the timed step (auto: the library's rule)")
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

    import torch
    import kimi_delta_attention_k1_amd as kda
    from kimi_delta_attention_k1_amd import workloads

    dev = torch.device("cuda:0")
    w = workloads.CONFIGS[args.workload]()
    q, k, v, g, b = (t.to(dev) for t in (w.q, w.k, w.v, w.g_raw, w.beta_raw))
    s0 = None if w.initial_state is None else w.initial_state.to(dev)
    cu = w.cu_seqlens().to(dev) if w.packed else None
    if not w.packed:
        shp = (w.N, w.seq_lens[0], w.H, 128)
        q, k, v, g = (t.view(shp) for t in (q, k, v, g))
        b = b.view(shp[:3])
    path = args.path
    if args.bf16_resident_state:
        path = "split"
    if path == "auto":  # the library's rule, include/kda.h
        if w.T_tot <= kda.RECURRENT_MAX_AVG_TOKENS * w.N:
            path = "recurrent"
        else:
            n_c = sum((L + 15) // 16 for L in w.seq_lens) if not w.packed else (w.T_tot + 15 * w.N) // 16
            if w.N * w.H <= kda.SEGMENTED_MAX_PAIRS and n_c >= kda.SEGMENTED_MIN_AVG_CHUNKS * w.N:
                path = "segmented"
            else:
                path = "fused" if w.N * w.H >= kda.FUSED_MIN_PAIRS else "split"
    other = "split" if path != "split" else "fused"
    calls = {p: kda.prepare_call(q, k, v, g, b, lower_bound=w.lower_bound, initial_state=s0, cu_seqlens=cu, path=p,
                                 bf16_resident_state=args.bf16_resident_state and p == "split")
             for p in (path, other)}
    torch.cuda.synchronize()

    ms_per_step, kern_ms = time_path(calls[path], path, args.steps, args.warmup)
    compare = None
    if args.compare_steps > 0:
        o_ms, o_kern = time_path(calls[other], other, args.compare_steps, min(args.warmup, 10))
        compare = {"path": other, "steps": args.compare_steps, "ms_per_step": round(o_ms, 4),
                   "tokens_per_s": round(w.T_tot / (o_ms * 1e-3), 1),
                   "kernels_avg_ms": {n: round(x, 4) for n, x in o_kern.items()}}

    if args.copy_probe_mib:
        src = torch.empty(args.copy_probe_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    work = algorithmic_work(w, bf16_resident_state=args.bf16_resident_state)
    bytes_of = {"k1_mfma": work["k1_bytes"], "k2_mfma": work["k2_bytes"], "kf_fused": work["kf_bytes"],
                "kr_recurrent": work["kf_bytes"], "kf_fused_seg": work["seg_bytes"],
                "kseg_finish": work["fin_bytes"]}
    per_kernel = {}
    for name, ms in kern_ms.items():
        gbs = bytes_of[name] / (ms * 1e-3) / 1e9
        ent = {"avg_ms": round(ms, 4), "algorithmic_bytes": bytes_of[name], "achieved_GBps": round(gbs, 1),
               "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
        if name in ("k2_mfma", "kf_fused", "kf_fused_seg"):
            fl = work["flops_split"] if name == "k2_mfma" else work["flops"]
            tf = fl / (ms * 1e-3) / 1e12
            ent.update({"algorithmic_flops": fl, "achieved_TFLOPs": round(tf, 2),
                        "mfma_frac": round(tf / BF16_PEAK_TFLOPS, 4)})
        per_kernel[name] = ent
    dom = max(kern_ms, key=kern_ms.get)
    d = per_kernel[dom]
    roofline = {"bound": "hbm", "kernel": dom, "achieved": d["achieved_GBps"], "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": d["hbm_frac"], "traffic": traffic_for(dom, args.workload)}

    tokens_per_s = w.T_tot / (ms_per_step * 1e-3)
    line = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded CPU torch.Generator, N(0,1) family; see workloads.py)",
        "config": {"workload": f"{args.workload}: {workloads.DESCRIPTIONS[args.workload]}",
                   "tokens": w.T_tot, "heads": w.H, "head_dim": 128, "sequences": w.N, "chunk": 16,
                   "lower_bound": w.lower_bound,
                   "path": path + (" (bf16-resident state)" if args.bf16_resident_state else "")},
        "event_ms_per_step": round(sum(kern_ms.values()), 4),
        "kernels": per_kernel,
        "roofline": roofline,
    }
    if compare is not None:
        line["path_compare"] = compare
    if args.cpu_seqs > 0:
        line["cpu_baseline"] = cpu_baseline(w, min(args.cpu_seqs, w.N))
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
