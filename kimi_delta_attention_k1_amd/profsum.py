"""Summaries of rocprofv3 output for the KDA kernels.

    python -m kimi_delta_attention_k1_amd.profsum stats  <kernel_stats.csv> <command...>
    python -m kimi_delta_attention_k1_amd.profsum traffic <fetch_counter_collection.csv>
           <write_counter_collection.csv> <workload> <copy_probe_mib>
    python -m kimi_delta_attention_k1_amd.profsum util <counter_collection.csv>

`stats` prints a Markdown table of per-kernel call counts and durations.
`traffic` turns FETCH_SIZE / WRITE_SIZE (KiB per dispatch) into HBM bytes per
launch. Both counters are scaled by what they read for the plain device copy
of known size that bench.py --copy-probe-mib runs in the same process
(the runtime's copy kernel; its last dispatches are the probe). The result is
merged into profiles/traffic_counters.json, keyed by workload and kernel, with
the SHA-256 of the kernel's sources so bench.py reports null once they change.
`util` prints, per kernel, the matrix-core and vector-ALU utilisation from one
counter pass (SQ_VALU_MFMA_BUSY_CYCLES, SQ_BUSY_CU_CYCLES, SQ_INSTS_VALU_MFMA_MOPS_BF16,
SQ_INSTS_VALU, SQ_ACTIVE_INST_VALU, SQ_INSTS_MFMA, SQ_WAVES, SQ_BUSY_CYCLES,
GRBM_GUI_ACTIVE), averaged over the kernel's dispatches.
"""
from __future__ import annotations

import csv
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TRAFFIC = os.path.join(ROOT, "profiles", "traffic_counters.json")
CSRC = os.path.join(ROOT, "kimi_delta_attention_k1_amd", "csrc")
# the sources each kernel is compiled from (a change to any of them voids its counters)
KERNEL_SOURCES = {
    "k1_mfma": ("kda_mfma.hip", "kda_mfma_common.h", "kda_internal.h"),
    "k2_mfma": ("kda_mfma.hip", "kda_mfma_common.h", "kda_internal.h"),
    "kf_fused": ("kda_fused.hip", "kda_mfma_common.h", "kda_internal.h"),
    "kr_recurrent": ("kda_recurrent.hip", "kda_internal.h"),
    "kf_fused_seg": ("kda_fused.hip", "kda_mfma_common.h", "kda_internal.h"),
    "kseg_scan": ("kda_seg.hip", "kda_mfma_common.h", "kda_internal.h"),
    "kseg_correct": ("kda_seg.hip", "kda_mfma_common.h", "kda_internal.h"),
}
# kernel-name fragments per reported kernel; the recurrence stage of the two-kernel
# path is k2_mfma, or k2_look (its look-ahead form) when few pairs run
SHORT = {"k1_mfma": ("kda::k1_mfma",), "k2_mfma": ("kda::k2_mfma", "kda::k2_look"),
         "kf_fused": ("kda::kf_fused",), "kr_recurrent": ("kda::kr_recurrent",),
         "k0_chunk_map": ("kda::k0_chunk_map",), "kseg_scan": ("kda::kseg_scan",),
         "kseg_correct": ("kda::kseg_correct",), "copy": ("__amd_rocclr_copyBuffer",)}


def src_hash(kernel: str) -> str:
    """SHA-256 over the kernel's source files, in a fixed order."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def short_name(kernel_name: str) -> str:
    # the single pass's template arguments are <state type, scalar gate, segmented, chunk-start
    # reference>: the segmented instantiations have "true" third
    if "kda::kf_fused<" in kernel_name:
        targs = kernel_name.split("(")[0].split("kda::kf_fused<", 1)[1].rstrip(">").split(",")
        return "kf_fused_seg" if len(targs) > 2 and targs[2].strip() == "true" else "kf_fused"
    for short, keys in SHORT.items():
        if any(key in kernel_name for key in keys):
            return short
    return kernel_name.split("(")[0][:40]


def stats(path: str, command: str) -> str:
    rows = list(csv.DictReader(open(path)))
    out = [f"Command: `{command}`", "", "| kernel | calls | avg us | min us | max us | % time |",
           "|---|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| {short_name(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                   f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f} |")
    return "\n".join(out)


def _per_kernel(path):
    per = {}
    for r in csv.DictReader(open(path)):
        per.setdefault(short_name(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
    return per


def traffic(fetch_csv, write_csv, workload, probe_mib):
    f, w = _per_kernel(fetch_csv), _per_kernel(write_csv)
    probe_kib = probe_mib * 1024.0
    # the probe copies are the last copy dispatches (three of them)
    ff = probe_kib / (sum(f["copy"][-3:]) / 3)
    fw = probe_kib / (sum(w["copy"][-3:]) / 3)
    rec = {}
    if os.path.exists(TRAFFIC):
        rec = json.load(open(TRAFFIC))
    ent = rec.setdefault(workload, {})
    for k in KERNEL_SOURCES:
        if k not in f or k not in w:
            continue
        fk = sum(f[k]) / len(f[k])
        wk = sum(w[k]) / len(w[k])
        ent[k] = {"fetch_kib_raw": round(fk, 1), "write_kib_raw": round(wk, 1),
                  "fetch_scale": round(ff, 4), "write_scale": round(fw, 4),
                  "bytes_per_launch": int(round((fk * ff + wk * fw) * 1024)),
                  "dispatches": len(f[k]), "src_sha256": src_hash(k)}
    os.makedirs(os.path.dirname(TRAFFIC), exist_ok=True)
    with open(TRAFFIC, "w") as fh:
        json.dump(rec, fh, indent=1, sort_keys=True)
    return ent


def util(path: str) -> str:
    """Counter-derived utilisation per kernel. SQ cycle counters are summed over
    compute units (SQ_BUSY_CU_CYCLES) or SIMDs (SQ_VALU_MFMA_BUSY_CYCLES); a CU has
    4 SIMDs and SQ_ACTIVE_INST_VALU counts in units of 4 cycles per wave
    instruction, so both busy fractions divide by 4 x SQ_BUSY_CU_CYCLES.
    SQ_INSTS_VALU_MFMA_MOPS_BF16 counts 512-flop units of bf16 matrix work."""
    per = {}
    for r in csv.DictReader(open(path)):
        k = short_name(r["Kernel_Name"])
        per.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    out = ["| kernel | dispatches | CU busy cycles | MFMA busy | VALU busy | VALU instr / wave | bf16 MFMA flop / dispatch |",
           "|---|---|---|---|---|---|---|"]
    for k, d in per.items():
        if k in ("copy", "k0_chunk_map"):
            continue
        m = {c: sum(v) / len(v) for c, v in d.items()}
        cu = m.get("SQ_BUSY_CU_CYCLES", 0.0)
        if cu <= 0:
            continue
        mfma = m.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (4 * cu)
        valu = m.get("SQ_ACTIVE_INST_VALU", 0.0) * 4 / (4 * cu)
        per_wave = m.get("SQ_INSTS_VALU", 0.0) / max(m.get("SQ_WAVES", 1.0), 1.0)
        flops = m.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) * 512
        out.append(f"| {k} | {len(next(iter(d.values())))} | {cu:.3e} | {100 * mfma:.1f}% | {100 * valu:.1f}% | "
                   f"{per_wave:.0f} | {flops:.3e} |")
    return "\n".join(out)


if __name__ == "__main__":
    if sys.argv[1] == "stats":
        print(stats(sys.argv[2], " ".join(sys.argv[3:])))
    elif sys.argv[1] == "traffic":
        print(json.dumps(traffic(sys.argv[2], sys.argv[3], sys.argv[4], float(sys.argv[5])), indent=1))
    elif sys.argv[1] == "util":
        print(util(sys.argv[2]))
