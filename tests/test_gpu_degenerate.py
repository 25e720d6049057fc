"""Degenerate and boundary inputs on every GPU path, against the fp64 oracle:
infinite gate and beta inputs (sigmoid exactly 0 or 1), no decay, the pages'
own head counts (H = 64, 96), and NULL vs explicit-zero initial states.

beta_raw = -inf gives beta = 0: no write, so the state only decays and the
output reads the decayed initial state (Doubleword section 3); g_raw = +inf
gives the strongest decay alpha = e^lb on every channel, g_raw = -inf none.
"""
import pytest
import torch

from kimi_delta_attention_k1_amd import workloads
from tests.gpu_helpers import bf16_tol, compare, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

PATHS = ["split", "fused", "recurrent"]


def _banner(name):
    print(f"\n[case] degenerate: {name}", flush=True)


def _with(w, **kw):
    d = dict(q=w.q, k=w.k, v=w.v, g_raw=w.g_raw, beta_raw=w.beta_raw, initial_state=w.initial_state)
    d.update(kw)
    return workloads.Workload(w.name, d["q"], d["k"], d["v"], d["g_raw"], d["beta_raw"], w.seq_lens, w.packed,
                              d["initial_state"], w.lower_bound)


@pytest.mark.parametrize("path", PATHS)
def test_no_write_when_beta_is_zero(gpu, path):
    _banner(f"beta_raw = -inf (beta = 0), {path}")
    w = workloads.make([40, 17], 2, seed=81, init_std=0.05)
    w = _with(w, beta_raw=torch.full_like(w.beta_raw, float("-inf")))
    compare(w, *run_gpu(w, gpu, path=path), run_oracle(w), bf16_tol, f"beta=0 {path}")


@pytest.mark.parametrize("path", PATHS)
def test_full_write_and_extreme_gates(gpu, path):
    """beta_raw = +inf (beta = 1); g_raw alternating +inf / -inf per channel
    (alpha = e^lb or 1); with lower_bound -10 the strongest decays reach e^-160
    within one chunk."""
    _banner(f"beta = 1, gates +-inf, lower_bound -10, {path}")
    w = workloads.make([33, 64], 2, seed=82, init_std=0.05, lower_bound=-10.0)
    g = torch.full_like(w.g_raw, float("inf"))
    g[..., 1::2] = float("-inf")
    w = _with(w, g_raw=g, beta_raw=torch.full_like(w.beta_raw, float("inf")))
    o, s = run_gpu(w, gpu, path=path)
    assert torch.isfinite(o.float()).all() and torch.isfinite(s.float()).all()
    compare(w, o, s, run_oracle(w), bf16_tol, f"extreme gates {path}")


@pytest.mark.parametrize("path", PATHS)
def test_no_decay(gpu, path):
    _banner(f"g_raw = -inf (alpha = 1, DeltaNet), {path}")
    w = workloads.make([50, 70], 2, seed=83, init_std=0.02)
    w = _with(w, g_raw=torch.full_like(w.g_raw, float("-inf")))
    compare(w, *run_gpu(w, gpu, path=path), run_oracle(w), bf16_tol, f"no decay {path}")


@pytest.mark.parametrize("H", [64, 96])
def test_page_head_counts(gpu, H):
    """The head counts of the pages' benchmarks; 4 x 512 tokens (256 or 384
    pairs: the automatic rule picks the single pass), plus the split path."""
    _banner(f"H={H}, 4 x 512 tokens")
    w = workloads.make([512] * 4, H, seed=84 + H, init_std=0.02)
    ref = run_oracle(w, pairs=[(0, 0), (1, H // 2), (3, H - 1)])
    for path in ("auto", "split"):
        compare(w, *run_gpu(w, gpu, path=path), ref, bf16_tol, f"H={H} {path}")


@pytest.mark.parametrize("path", PATHS)
def test_null_and_zero_initial_state_agree(gpu, path):
    _banner(f"NULL vs explicit zero initial state, {path}")
    w = workloads.make([30, 45], 3, seed=85)
    o1, s1 = run_gpu(w, gpu, path=path)  # workload has no initial state: NULL
    o2, s2 = run_gpu(w, gpu, path=path, initial_state=torch.zeros(2, 3, 128, 128))
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    compare(w, o1, s1, run_oracle(w), bf16_tol, f"null state {path}")
