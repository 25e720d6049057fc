"""Shared plumbing for the GPU parity tests: move a seeded workload to the GPU,
run it through the C ABI, run the fp64 oracle on all or some (sequence, head)
pairs, and compare with the tolerances of the build's specification.
"""
from __future__ import annotations

import numpy as np
import torch

import kimi_delta_attention_k1_amd as kda
import oracle


def bf16_tol(ref: np.ndarray) -> float:
    """max|x_gpu - x_ref| <= 1e-2 * max|x_ref| + 1e-3 (bf16 I/O)."""
    return 1e-2 * float(np.max(np.abs(ref))) + 1e-3


def f32_tol(ref: np.ndarray) -> float:
    """max|x_gpu - x_ref| <= 1e-5 * max|x_ref| (fp32 debug path)."""
    return 1e-5 * float(np.max(np.abs(ref)))


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def run_gpu(w, dev, *, state_dtype=torch.float32, fp32_compute=False, workspace=None, final=True,
            initial_state="from_workload", out=None, final_state=None, path="auto", beta=None,
            bf16_resident_state=False, scale=None):
    """Run workload w on the GPU; returns (out [T_tot,H,128] tensor, final_state tensor or None).
    `path` selects the kernels ("auto", "split", "fused"); `beta` replaces the
    device copy of beta_raw (same shape and values, e.g. at an odd address);
    `scale` is the read scale (None: 128^-1/2)."""
    q, k, v, g, b = (t.to(dev) for t in (w.q, w.k, w.v, w.g_raw, w.beta_raw))
    if beta is not None:
        b = beta
    s0 = w.initial_state if initial_state == "from_workload" else initial_state
    if s0 is not None:
        s0 = s0.to(dev, state_dtype)
    if w.packed:
        cu = w.cu_seqlens().to(dev)
        o, s = kda.fwd(q, k, v, g, b, lower_bound=w.lower_bound, scale=scale, initial_state=s0,
                       output_final_state=final,
                       cu_seqlens=cu, fp32_compute=fp32_compute, workspace=workspace, out=out,
                       final_state=final_state, path=path, bf16_resident_state=bf16_resident_state)
    else:
        B, T = w.N, w.seq_lens[0]
        shp = (B, T, w.H, 128)
        gshp = shp if g.dim() == 3 else shp[:3]
        o, s = kda.fwd(q.view(shp), k.view(shp), v.view(shp), g.view(gshp), b.view(B, T, w.H),
                       lower_bound=w.lower_bound, scale=scale, initial_state=s0, output_final_state=final,
                       fp32_compute=fp32_compute, workspace=workspace,
                       out=None if out is None else out.view(shp), final_state=final_state, path=path,
                       bf16_resident_state=bf16_resident_state)
        o = o.view(B * T, w.H, 128)
    torch.cuda.synchronize(dev)
    return o, s


def _gate(w):
    """g_raw as the oracle takes it, [T, H, 128]: a scalar per-head gate is the
    same value on every key channel (the Gated DeltaNet case of the recurrence)."""
    g = w.g_raw
    return g[..., None].expand(*g.shape, 128) if g.dim() == 2 else g


def run_oracle(w, pairs=None, threads=0, scale=None):
    """fp64 token oracle on the whole workload (pairs=None) or on the listed
    (sequence, head) pairs, with read scale `scale` (None: 128^-1/2).
    Returns {(n, h): (o [L,128], S [128,128])}."""
    offs = w.offsets()
    f = lambda t: t.to(torch.float32).numpy()  # noqa: E731  exact widening of bf16/fp32
    res = {}
    if pairs is None:
        o, S = oracle.token_forward(f(w.q), f(w.k), f(w.v), f(_gate(w)), f(w.beta_raw), offs,
                                    None if w.initial_state is None else w.initial_state.numpy(),
                                    lower_bound=w.lower_bound, scale=scale, threads=threads)
        for n in range(w.N):
            for h in range(w.H):
                res[(n, h)] = (o[offs[n]:offs[n + 1], h], S[n, h])
        return res
    # group by sequence so one oracle call covers several heads of it
    by_seq = {}
    for n, h in pairs:
        by_seq.setdefault(n, []).append(h)
    for n, hs in by_seq.items():
        a, e = offs[n], offs[n + 1]
        sl = lambda t: f(t[a:e][:, hs])  # noqa: E731
        s0 = None if w.initial_state is None else w.initial_state[n][hs].numpy()[None]
        o, S = oracle.token_forward(sl(w.q), sl(w.k), sl(w.v), sl(_gate(w)), sl(w.beta_raw), [0, e - a], s0,
                                    lower_bound=w.lower_bound, scale=scale, threads=threads)
        for i, h in enumerate(hs):
            res[(n, h)] = (o[:, i], S[0, i])
    return res


# (what, pairs compared, worst output err/tol, worst state err/tol) of every comparison in
# this session, printed at the end of the run (tests/conftest.py)
RESULTS = []


def compare(w, o_gpu, s_gpu, ref, tol_fn, what=""):
    """Check every pair in ref; returns (worst o ratio, worst state ratio) of err/tol."""
    offs = w.offsets()
    o_all = np.concatenate([r[0].reshape(-1) for r in ref.values()])
    s_all = np.concatenate([r[1].reshape(-1) for r in ref.values()])
    tol_o, tol_s = tol_fn(o_all), tol_fn(s_all)
    worst_o = worst_s = 0.0
    og = o_gpu.detach().to("cpu", torch.float32)
    sg = None if s_gpu is None else s_gpu.detach().to("cpu", torch.float32)
    for (n, h), (ro, rs) in ref.items():
        go = og[offs[n]:offs[n + 1], h].numpy().astype(np.float64)
        eo = float(np.max(np.abs(go - ro))) if ro.size else 0.0
        worst_o = max(worst_o, eo / tol_o if tol_o > 0 else eo)
        if sg is not None:
            es = float(np.max(np.abs(sg[n, h].numpy().astype(np.float64) - rs)))
            worst_s = max(worst_s, es / tol_s if tol_s > 0 else es)
    print(f"{what}: err/tol o {worst_o:.3f} state {worst_s:.3f} (tol o {tol_o:.3e}, state {tol_s:.3e})",
          flush=True)
    RESULTS.append((what, len(ref), worst_o, worst_s if sg is not None else None))
    assert worst_o <= 1.0, f"{what}: output error {worst_o:.3f} x tolerance"
    assert worst_s <= 1.0, f"{what}: state error {worst_s:.3f} x tolerance"
    return worst_o, worst_s
