"""kda_fwd_noalloc: the forward without a workspace argument, its scratch in the
library's static device buffer, checked through the C ABI against kda_fwd on the
same path (bitwise: the same kernels run) and against the fp64 oracle, on calls
in a row whose second and third are smaller than the first, so stale scratch
from an earlier call must not matter.
"""
import pytest
import torch

import kimi_delta_attention_k1_amd as kda
from kimi_delta_attention_k1_amd import workloads
from tests.gpu_helpers import bf16_tol, compare, run_oracle

pytestmark = pytest.mark.gpu


def _banner(name):
    print(f"\n[case] no-alloc: {name}", flush=True)


def _both(w, dev, path):
    """(kda_fwd on `path`, kda_fwd_noalloc unforced) on w, outputs preallocated."""
    q, k, v, g, b = (t.to(dev) for t in (w.q, w.k, w.v, w.g_raw, w.beta_raw))
    cu = w.cu_seqlens().to(dev)
    s0 = None if w.initial_state is None else w.initial_state.to(dev)
    ref = kda.fwd(q, k, v, g, b, lower_bound=w.lower_bound, initial_state=s0, cu_seqlens=cu, path=path)
    out = torch.empty_like(v)
    fin = torch.empty(w.N, w.H, 128, 128, device=dev)
    got = kda.fwd_noalloc(q, k, v, g, b, lower_bound=w.lower_bound, initial_state=s0, cu_seqlens=cu, out=out,
                          final_state=fin)
    torch.cuda.synchronize(dev)
    assert got[0].data_ptr() == out.data_ptr() and got[1].data_ptr() == fin.data_ptr()
    return ref, got


def test_noalloc_matches_kda_fwd_on_calls_in_a_row(gpu):
    cases = [
        ("40 ragged sequences x H=4 (single pass)", workloads.make(None, 4, seed=301, init_std=0.02,
                                                                   lens_drawn=(1, 300, 40)), "fused"),
        ("7 ragged sequences x H=2, smaller (single pass)", workloads.make(None, 2, seed=302, init_std=0.02,
                                                                          lens_drawn=(1, 90, 7)), "fused"),
        ("decode: 16 sequences x 1 token, H=4 (token by token)", workloads.make([1] * 16, 4, seed=303,
                                                                                 init_std=0.02), "recurrent"),
    ]
    for name, w, path in cases:
        _banner(name)
        (ro, rs), (go, gs) = _both(w, gpu, path)
        assert torch.equal(ro, go) and torch.equal(rs, gs), f"{name}: kda_fwd_noalloc differs from kda_fwd"
        compare(w, go, gs, run_oracle(w), bf16_tol, f"no-alloc {name}")


def test_noalloc_rejects_paths_with_a_large_workspace(gpu):
    _banner("split / segmented paths are refused")
    w = workloads.make([64], 1, seed=304)
    q, k, v, g, b = (t.to(gpu) for t in (w.q, w.k, w.v, w.g_raw, w.beta_raw))
    for path in ("split", "segmented"):
        with pytest.raises(kda.KdaError) as err:
            kda.fwd_noalloc(q, k, v, g, b, cu_seqlens=w.cu_seqlens().to(gpu), path=path)
        assert err.value.status == 5  # KDA_ERR_BAD_ARG
