"""Degenerate and boundary inputs on every GPU path, against the fp64 oracle:
infinite gate and beta inputs (sigmoid exactly 0 or 1), no decay, keys that
point almost the same way, the pages' own head counts (H = 64, 96), and NULL
vs explicit-zero initial states. The segmented pass gets sequences long enough
for three segments or more (its segments are at least 8 chunks, the first 12), next to
a one-chunk sequence.

beta_raw = -inf gives beta = 0: no write, so the state only decays and the
output reads the decayed initial state (Doubleword section 3); g_raw = +inf
gives the strongest decay alpha = e^lb on every channel, g_raw = -inf none.
"""
import pytest
import torch

from kimi_delta_attention_k1_amd import workloads
from tests.gpu_helpers import bf16_tol, compare, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

PATHS = ["split", "fused", "segmented", "recurrent"]


def _lens(path, lens):
    """The case's own lengths, or for the segmented pass 3, 1 and 2 segments."""
    return [700, 17, 433] if path == "segmented" else lens


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
    w = workloads.make(_lens(path, [40, 17]), 2, seed=81, init_std=0.05)
    w = _with(w, beta_raw=torch.full_like(w.beta_raw, float("-inf")))
    compare(w, *run_gpu(w, gpu, path=path), run_oracle(w), bf16_tol, f"beta=0 {path}")


@pytest.mark.parametrize("path", PATHS)
def test_full_write_and_extreme_gates(gpu, path):
    """beta_raw = +inf (beta = 1); g_raw alternating +inf / -inf per channel
    (alpha = e^lb or 1); with lower_bound -10 the strongest decays reach e^-160
    within one chunk."""
    _banner(f"beta = 1, gates +-inf, lower_bound -10, {path}")
    w = workloads.make(_lens(path, [33, 64]), 2, seed=82, init_std=0.05, lower_bound=-10.0)
    g = torch.full_like(w.g_raw, float("inf"))
    g[..., 1::2] = float("-inf")
    w = _with(w, g_raw=g, beta_raw=torch.full_like(w.beta_raw, float("inf")))
    o, s = run_gpu(w, gpu, path=path)
    assert torch.isfinite(o.float()).all() and torch.isfinite(s.float()).all()
    compare(w, o, s, run_oracle(w), bf16_tol, f"extreme gates {path}")


@pytest.mark.parametrize("path", PATHS)
def test_no_decay(gpu, path):
    _banner(f"g_raw = -inf (alpha = 1, DeltaNet), {path}")
    w = workloads.make(_lens(path, [50, 70]), 2, seed=83, init_std=0.02)
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
    w = workloads.make(_lens(path, [30, 45]), 3, seed=85)
    o1, s1 = run_gpu(w, gpu, path=path)  # workload has no initial state: NULL
    o2, s2 = run_gpu(w, gpu, path=path, initial_state=torch.zeros(w.N, 3, 128, 128))
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    compare(w, o1, s1, run_oracle(w), bf16_tol, f"null state {path}")


def _correlated_keys(w, spread, seed):
    """Keys of every token of a head share one random direction: k_t = u_h + spread n_t
    with u_h, n_t ~ N(0, 1) per channel, so distinct keys have cosine about
    1 / (1 + spread^2). The unit-lower-triangular matrix of a chunk then has
    entries near beta in its whole lower triangle."""
    gen = torch.Generator().manual_seed(seed)
    u = torch.randn(1, w.H, 128, generator=gen)
    n = torch.randn(w.T_tot, w.H, 128, generator=gen)
    return (u + spread * n).to(w.k.dtype)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("case", ["beta1_nodecay", "beta_n11_lb0"])
def test_correlated_keys_without_decay(gpu, path, case):
    """Keys with cosine ~0.96 and no decay (g_raw = -inf, or lower_bound 0), with
    beta = 1 (beta_raw = +inf) or beta_raw ~ N(1, 1): the inverse of I + R has entries
    bounded by one while the powers of R grow to the hundreds, so an inverse formed
    from those powers in low precision loses everything to cancellation."""
    _banner(f"correlated keys, {case}, {path}")
    lb = 0.0 if case == "beta_n11_lb0" else -5.0
    w = workloads.make(_lens(path, [64, 45]), 2, seed=86, init_std=0.02, beta_mean=1.0, lower_bound=lb)
    kw = dict(k=_correlated_keys(w, 0.2, 87))
    if case == "beta1_nodecay":
        kw.update(g_raw=torch.full_like(w.g_raw, float("-inf")), beta_raw=torch.full_like(w.beta_raw, float("inf")))
    w = _with(w, **kw)
    o, s = run_gpu(w, gpu, path=path)
    assert torch.isfinite(o.float()).all() and torch.isfinite(s.float()).all()
    compare(w, o, s, run_oracle(w), bf16_tol, f"correlated keys {case} {path}")


@pytest.mark.parametrize("path", PATHS)
def test_correlated_keys_over_long_sequences(gpu, path):
    """Keys with cosine ~0.96 over 512-token sequences, beta = 1 and no decay
    (lower_bound 0): the state-update key operand K_end is rounded every chunk into
    state directions that later keys never overwrite, which a one-bf16 K_end turned
    into twice the bound on the final state; every path keeps it as a hi/lo pair."""
    _banner(f"correlated keys over 512-token sequences, no decay, {path}")
    w = workloads.make([512, 512, 300], 2, seed=88, init_std=0.02, beta_mean=1.0, lower_bound=0.0)
    w = _with(w, k=_correlated_keys(w, 0.2, 89), beta_raw=torch.full_like(w.beta_raw, float("inf")))
    o, s = run_gpu(w, gpu, path=path)
    compare(w, o, s, run_oracle(w), bf16_tol, f"correlated keys 512 tokens {path}")
