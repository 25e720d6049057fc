"""A call whose tensors pass 2^31 bytes: one sequence of 131072 tokens with H = 72
(q, k, v and g_raw 2.4 GB each in bf16, the two-kernel path's workspace 11 GB), on
the automatic (segmented), single-pass and two-kernel paths. Every byte offset past
2^31 must be formed in 64 bits; the first and last heads, whose data sit at the
lowest and highest addresses, are compared with the oracle.

Inputs: a seeded [131072][8] workload drawn on the CPU, widened on the GPU by torch
to 72 heads (head h is base head h mod 8 scaled by 1 + h/128, rounded to bf16), so
every head differs; the oracle reads the sampled heads' inputs back from those tensors.
"""
import pytest
import torch

from kimi_delta_attention_k1_amd import workloads
import kimi_delta_attention_k1_amd as kda
from tests.gpu_helpers import bf16_tol, compare, run_oracle

pytestmark = pytest.mark.gpu

T, H, BASE_H = 131072, 72, 8


def _widen(x, dev):
    idx = torch.arange(H, device=dev) % BASE_H
    xh = x.to(dev)[:, idx]
    scale = (1 + torch.arange(H, dtype=torch.float32, device=dev) / 128).view(1, H, *([1] * (x.dim() - 2)))
    return (xh.float() * scale).to(torch.bfloat16).contiguous()


@pytest.mark.timeout(600)
def test_tensors_past_two_gigabytes(gpu):
    print(f"\n[case] large tensors: T={T}, H={H}", flush=True)
    base = workloads.make([T], BASE_H, seed=77, packed=False)
    q, k, v, g = (_widen(t, gpu) for t in (base.q, base.k, base.v, base.g_raw))
    b = _widen(base.beta_raw, gpu)
    assert q.numel() * q.element_size() > 2 ** 31
    torch.cuda.synchronize(gpu)
    # the sampled heads' inputs, as the calls see them
    heads = [0, H - 1]
    sampled = workloads.Workload("large", *(t[:, heads].cpu() for t in (q, k, v, g, b)), [T], False, None, -5.0)
    ref = run_oracle(sampled, threads=2)
    shp = (1, T, H, 128)
    for path in ("auto", "fused", "split"):
        print(f"[case] large tensors, path {path}", flush=True)
        o, s = kda.fwd(q.view(shp), k.view(shp), v.view(shp), g.view(shp), b.view(1, T, H), lower_bound=-5.0,
                       path=path)
        torch.cuda.synchronize(gpu)
        o_s = o.view(T, H, 128)[:, heads].contiguous()
        s_s = s[:, heads].contiguous()
        compare(sampled, o_s, s_s, ref, bf16_tol, f"large T={T} H={H} {path}")
        del o, s
        torch.cuda.empty_cache()
