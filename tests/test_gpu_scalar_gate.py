"""GPU parity of the scalar per-head gate (KDA_FLAG_SCALAR_GATE, Gated DeltaNet):
g_raw is [T, H] and its one value per token and head applies to every key
channel. Every path (split bf16, single pass, token by token, fp32 reference)
is compared with the fp64 oracle fed the gate broadcast over the 128 channels,
which is the definition of the scalar-gate case (Doubleword page, section 3),
and with the same kernels run on that broadcast [T, H, 128] gate: identical
inputs on every channel must give bitwise identical results.
"""
import pytest
import torch

from kimi_delta_attention_k1_amd import workloads
from tests.gpu_helpers import bf16_tol, compare, f32_tol, run_gpu, run_oracle

pytestmark = pytest.mark.gpu


def _banner(name):
    print(f"\n[case] scalar gate: {name}", flush=True)


def _broadcast(w):
    """The same workload with g_raw materialised as [T, H, 128]."""
    w2 = workloads.Workload(w.name + "-bcast", w.q, w.k, w.v, w.g_raw[..., None].expand(*w.g_raw.shape, 128).contiguous(),
                            w.beta_raw, w.seq_lens, w.packed, w.initial_state, w.lower_bound)
    return w2


@pytest.mark.parametrize("path,fp32", [("split", False), ("fused", False), ("recurrent", False), ("split", True)])
def test_paths_against_oracle_and_broadcast_gate(gpu, path, fp32):
    _banner(f"{path}{' fp32-compute' if fp32 else ''}: lengths 1,15,16,17,0,33,100, H=3")
    w = workloads.make([1, 15, 16, 17, 0, 33, 100], 3, seed=61, init_std=0.02, scalar_gate=True)
    assert w.g_raw.shape == (w.T_tot, 3)
    ref = run_oracle(w)
    o, s = run_gpu(w, gpu, path=path, fp32_compute=fp32)
    compare(w, o, s, ref, bf16_tol, f"scalar gate {path}")
    o2, s2 = run_gpu(_broadcast(w), gpu, path=path, fp32_compute=fp32)
    assert torch.equal(o, o2) and torch.equal(s, s2)


@pytest.mark.parametrize("path", ["split", "recurrent"])
def test_fp32_io_meets_fp32_bound(gpu, path):
    _banner(f"fp32 I/O on the {path} path")
    w = workloads.make([3, 40, 16], 2, seed=62, dtype=torch.float32, init_std=0.02, scalar_gate=True)
    compare(w, *run_gpu(w, gpu, path=path), run_oracle(w), f32_tol, f"scalar gate fp32 {path}")


@pytest.mark.parametrize("H", [1, 5])
def test_fused_odd_gate_address(gpu, H):
    """g_raw at a base address 2 mod 4: the single pass fetches the dword that
    holds each element and picks its half."""
    _banner(f"fused, H={H}, g_raw at an odd element offset")
    w = workloads.make([50, 31, 7], H, seed=63 + H, init_std=0.02, scalar_gate=True)
    ref = run_oracle(w)
    raw = torch.empty(w.g_raw.numel() + 1, dtype=torch.bfloat16, device=gpu)
    gs = raw[1:].view(w.g_raw.shape)
    gs.copy_(w.g_raw.to(gpu))
    assert gs.data_ptr() % 4 == 2
    w_dev = workloads.Workload(w.name, w.q, w.k, w.v, gs, w.beta_raw, w.seq_lens, w.packed, w.initial_state,
                               w.lower_bound)
    o, s = run_gpu(w_dev, gpu, path="fused")
    compare(w, o, s, ref, bf16_tol, f"scalar gate fused odd address H={H}")


def test_full_head_count_sampled(gpu):
    """8 x 2048 tokens, H=32 (256 pairs: the automatic rule picks the single
    pass); the split path on the same inputs, both on sampled pairs."""
    _banner("8 x 2048 tokens, H=32, sampled pairs, fused and split")
    w = workloads.make([2048] * 8, 32, seed=64, init_std=0.02, g_mean=-1.0, scalar_gate=True)
    ref = run_oracle(w, pairs=[(0, 0), (3, 17), (7, 31)])
    for path in ("auto", "split"):
        o, s = run_gpu(w, gpu, path=path)
        assert torch.isfinite(o).all() and torch.isfinite(s).all()
        compare(w, o, s, ref, bf16_tol, f"scalar gate 8x2048 {path}")


def test_batch_mode_bf16_state(gpu):
    _banner("batch rows, bf16 states, every path")
    w = workloads.make([40, 40], 2, seed=65, packed=False, init_std=0.05, scalar_gate=True)
    w.initial_state = w.initial_state.to(torch.bfloat16).to(torch.float32)  # exact in bf16
    ref = run_oracle(w)
    for path in ("split", "fused", "recurrent"):
        compare(w, *run_gpu(w, gpu, path=path, state_dtype=torch.bfloat16), ref, bf16_tol,
                f"scalar gate batch bf16 state {path}")
