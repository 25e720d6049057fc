"""Seeded random combinations of the call's options against the fp64 oracle.

The other GPU tests vary one option at a time around the five workloads; here
each case draws every option at once from a fixed seed: the path, the number of
sequences and their lengths (empty, one token, chunk edges, and arbitrary
lengths), the head count, packed or batch layout, lower_bound from -10 to 0,
gate and beta_raw means, a per-channel or scalar gate, the read scale, an
initial state or none, fp32 or bf16 states, fp32 I/O or the fp32-compute flag
where the path takes them, and whether the final state is written. Every
(sequence, head) pair is compared with the oracle (Doubleword "You Could Have
Come Up With Kimi Delta Attention", section 4, token recurrence) under the
bf16 or fp32 bound of the build's specification.
"""
import random

import pytest
import torch

from kimi_delta_attention_k1_amd import workloads
from tests.gpu_helpers import bf16_tol, compare, f32_tol, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

PATHS = ["auto", "split", "fused", "segmented", "recurrent"]
EDGE_LENGTHS = [0, 1, 15, 16, 17, 31, 33, 128, 129]


def _draw_case(i, r):
    path = PATHS[i % len(PATHS)]
    N = r.randint(1, 5)
    H = r.randint(1, 5)
    longest = 900 if path == "segmented" else 400
    batch = r.random() < 0.25
    if batch:
        lens = [r.randint(1, longest)] * N
    else:
        lens = [r.choice(EDGE_LENGTHS) if r.random() < 0.35 else r.randint(1, longest) for _ in range(N)]
        if sum(lens) == 0:
            lens[0] = r.randint(1, longest)
    fp32_ok = path in ("auto", "split", "recurrent")
    mode = r.choice(["bf16", "bf16", "fp32_io", "fp32_compute"]) if fp32_ok else "bf16"
    return dict(
        path=path, lens=lens, H=H, batch=batch, mode=mode,
        lb=r.choice([-10.0, -5.0, -3.0, -1.0, -0.25, 0.0]),
        g_mean=r.choice([-1.0, 0.0, 1.0]), beta_mean=r.choice([0.0, 1.0]),
        scalar_gate=r.random() < 0.25, scale=r.choice([None, None, 0.05, 0.5]),
        init_std=r.choice([0.0, 0.02, 0.1]), bf16_state=r.random() < 0.3,
        final=r.random() < 0.85, seed=1000 + i)


_R = random.Random(20261203)
CASES = [_draw_case(i, _R) for i in range(40)]


def _id(c):
    return (f"{c['path']}-N{len(c['lens'])}-H{c['H']}-{'batch' if c['batch'] else 'packed'}-{c['mode']}"
            f"-lb{c['lb']:g}{'-scalar' if c['scalar_gate'] else ''}")


@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
def test_random_option_mix(gpu, case):
    c = case
    print(f"\n[case] random mix: {c}", flush=True)
    dtype = torch.float32 if c["mode"] == "fp32_io" else torch.bfloat16
    w = workloads.make(c["lens"], c["H"], seed=c["seed"], dtype=dtype, packed=not c["batch"],
                       g_mean=c["g_mean"], beta_mean=c["beta_mean"], init_std=c["init_std"],
                       lower_bound=c["lb"], scalar_gate=c["scalar_gate"])
    state_dtype = torch.bfloat16 if c["bf16_state"] else torch.float32
    if w.initial_state is not None and c["bf16_state"]:
        # the call reads a bf16 state: give the oracle the same values
        w.initial_state = w.initial_state.to(torch.bfloat16).to(torch.float32)
    fin = None
    if c["final"] and w.initial_state is None:
        # without an initial state the final state's dtype comes from the buffer passed
        fin = torch.empty((w.N, w.H, 128, 128), dtype=state_dtype, device=gpu)
    o, s = run_gpu(w, gpu, path=c["path"], state_dtype=state_dtype, fp32_compute=c["mode"] == "fp32_compute",
                   final=c["final"], final_state=fin, scale=c["scale"])
    if s is not None:
        assert s.dtype == state_dtype
    assert torch.isfinite(o.float()).all()
    tol = f32_tol if c["mode"] == "fp32_io" and not c["bf16_state"] else bf16_tol
    compare(w, o, s if c["final"] else None, run_oracle(w, scale=c["scale"]), tol, f"random {_id(c)}")
