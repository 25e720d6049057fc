"""GPU parity of the single-pass kernel (path="fused") against the fp64 oracle,
and its agreement with the two-kernel path, through the C ABI.

Same tolerances as test_gpu_parity.py (bf16 I/O: max|x_gpu - x_ref| <=
1e-2 max|x_ref| + 1e-3 for o and the final state). Each case forces the path
with the KDA_FLAG_FUSED flag, whatever the automatic rule would pick.
"""
import numpy as np
import pytest
import torch

import kimi_delta_attention_k1_amd as kda
from kimi_delta_attention_k1_amd import workloads
from tests.gpu_helpers import bf16_tol, compare, run_gpu, run_oracle

pytestmark = pytest.mark.gpu


def _banner(name):
    print(f"\n[case] fused: {name}", flush=True)


def test_c3_full_size_sampled_and_against_split(gpu):
    _banner("c3 packed 8 x 8192, H=32 (sampled pairs), fused vs split")
    w = workloads.c3()
    pairs = [(0, 0), (3, 17), (7, 31), (5, 8)]
    ref = run_oracle(w, pairs=pairs)
    of, sf = run_gpu(w, gpu, path="fused")
    assert torch.isfinite(of).all() and torch.isfinite(sf).all()
    compare(w, of, sf, ref, bf16_tol, "c3 fused sampled")
    os_, ss = run_gpu(w, gpu, path="split")
    # the two paths round differently; both sit inside the oracle bound, and they
    # agree with each other everywhere to the same bound
    for a, b, what in ((of, os_, "o"), (sf, ss, "state")):
        a32, b32 = a.float(), b.float()
        err = (a32 - b32).abs().max().item()
        tol = 1e-2 * b32.abs().max().item() + 1e-3
        print(f"c3 fused vs split {what}: max diff {err:.3e} (bound {tol:.3e})", flush=True)
        assert err <= tol


def test_c5_full_size_sampled(gpu):
    _banner("c5 ragged 64 sequences, H=32 (sampled pairs incl. shortest/longest)")
    w = workloads.c5()
    lens = w.seq_lens
    nmin, nmax = int(np.argmin(lens)), int(np.argmax(lens))
    odd = next(i for i, L in enumerate(lens) if L % 16 != 0)
    pairs = [(nmin, 3), (nmax, 30), (odd, 11), (62, 5)]
    ref = run_oracle(w, pairs=pairs)
    o, s = run_gpu(w, gpu, path="fused")
    assert torch.isfinite(o).all() and torch.isfinite(s).all()
    compare(w, o, s, ref, bf16_tol, "c5 fused sampled")


def test_c4_long_context_sampled(gpu):
    _banner("c4 long context T=131072, H=32 (sampled heads)")
    w = workloads.c4()
    ref = run_oracle(w, pairs=[(0, 2), (0, 29)])
    o, s = run_gpu(w, gpu, path="fused")
    assert torch.isfinite(o).all() and torch.isfinite(s).all()
    compare(w, o, s, ref, bf16_tol, "c4 fused sampled")


def test_ragged_tails_and_empty_sequences(gpu):
    _banner("lengths 1,15,16,17,0,33,100,64,65 with initial state")
    w = workloads.make([1, 15, 16, 17, 0, 33, 100, 64, 65], 4, seed=7, init_std=0.02, beta_mean=0.5)
    ref = run_oracle(w)
    o, s = run_gpu(w, gpu, path="fused")
    compare(w, o, s, ref, bf16_tol, "fused ragged")
    assert torch.equal(s[4].cpu(), w.initial_state[4])  # empty sequence: final = initial


@pytest.mark.parametrize("H", [1, 3, 5])
def test_head_counts_and_odd_beta_address(gpu, H):
    """beta_raw at a base address that is 2 mod 4: each token's element sits in
    the high or low half of the dword the kernel loads, alternating with the
    token when H is odd."""
    _banner(f"H={H}, beta_raw at an odd element offset")
    w = workloads.make([50, 31, 7], H, seed=200 + H, init_std=0.02)
    ref = run_oracle(w)
    compare(w, *run_gpu(w, gpu, path="fused"), ref, bf16_tol, f"fused H={H}")
    raw = torch.empty(w.beta_raw.numel() + 1, dtype=torch.bfloat16, device=gpu)
    shifted = raw[1:].view(w.beta_raw.shape)
    shifted.copy_(w.beta_raw.to(gpu))
    assert shifted.data_ptr() % 4 == 2
    compare(w, *run_gpu(w, gpu, path="fused", beta=shifted), ref, bf16_tol, f"fused H={H} odd beta")


@pytest.mark.parametrize("lb", [0.0, -1.0, -10.0])
def test_lower_bound_range(gpu, lb):
    _banner(f"lower_bound {lb}")
    w = workloads.make([64, 45, 130], 2, seed=23, init_std=0.02, lower_bound=lb)
    compare(w, *run_gpu(w, gpu, path="fused"), run_oracle(w), bf16_tol, f"fused lb={lb}")


def test_batch_mode_bf16_state_no_final(gpu):
    _banner("batch rows, bf16 states, final state not requested")
    w = workloads.make([90, 90], 2, seed=19, packed=False, init_std=0.05)
    w.initial_state = w.initial_state.to(torch.bfloat16).to(torch.float32)  # exact in bf16
    ref = run_oracle(w)
    o, s = run_gpu(w, gpu, state_dtype=torch.bfloat16, path="fused")
    assert s.dtype == torch.bfloat16
    compare(w, o, s, ref, bf16_tol, "fused bf16 state")
    o2, s2 = run_gpu(w, gpu, final=False, path="fused")
    assert s2 is None
    compare(w, o2, None, ref, bf16_tol, "fused no final state")


def test_streaming_inplace_and_determinism(gpu):
    _banner("streamed halves, final_state aliasing initial_state, bitwise determinism")
    T, T1, H = 200, 71, 2
    w = workloads.make([T], H, seed=13, init_std=0.02)
    ref = run_oracle(w)
    o1, s1 = run_gpu(w, gpu, path="fused")
    o2, s2 = run_gpu(w, gpu, path="fused")
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    compare(w, o1, s1, ref, bf16_tol, "fused one call")
    buf = w.initial_state.to(gpu).contiguous()
    dev = lambda t: t.to(gpu)  # noqa: E731
    oa, sa = kda.fwd(dev(w.q[:T1]), dev(w.k[:T1]), dev(w.v[:T1]), dev(w.g_raw[:T1]), dev(w.beta_raw[:T1]),
                     initial_state=buf, final_state=buf, cu_seqlens=torch.tensor([0, T1], dtype=torch.int32,
                                                                                 device=gpu), path="fused")
    ob, sb = kda.fwd(dev(w.q[T1:]), dev(w.k[T1:]), dev(w.v[T1:]), dev(w.g_raw[T1:]), dev(w.beta_raw[T1:]),
                     initial_state=buf, final_state=buf,
                     cu_seqlens=torch.tensor([0, T - T1], dtype=torch.int32, device=gpu), path="fused")
    torch.cuda.synchronize()
    assert sb.data_ptr() == buf.data_ptr()
    compare(w, torch.cat([oa, ob]), sb, ref, bf16_tol, "fused streamed in place")


def test_empty_batch_copies_state(gpu):
    _banner("T = 0 batch mode: final = initial")
    s0 = torch.randn(2, 3, 128, 128, device=gpu)
    z = torch.empty(2, 0, 3, 128, dtype=torch.bfloat16, device=gpu)
    o, s = kda.fwd(z, z, z, z, torch.empty(2, 0, 3, dtype=torch.bfloat16, device=gpu), initial_state=s0,
                   path="fused")
    torch.cuda.synchronize()
    assert o.shape == z.shape and torch.equal(s, s0)


def test_guard_bytes_and_small_workspace(gpu):
    _banner("canary bytes around out, final_state and the chunk-map-only workspace")
    w = workloads.make([37, 64, 16], 4, seed=31, init_std=0.02)
    G = 4096
    T, H = w.T_tot, w.H
    n_out = T * H * 128
    need = kda.workspace_size(1, T, w.N, H, path="fused")
    assert need < kda.workspace_size(1, T, w.N, H, path="split")
    out_buf = torch.full((n_out + 2 * G,), 12345.0, dtype=torch.bfloat16, device=gpu)
    st_buf = torch.full((w.N * H * 128 * 128 + 2 * G,), -777.0, device=gpu)
    ws_buf = torch.full((need + 2 * G,), 0xA5, dtype=torch.uint8, device=gpu)
    out = out_buf[G:G + n_out].view(T, H, 128)
    fin = st_buf[G:G + w.N * H * 128 * 128].view(w.N, H, 128, 128)
    o, s = run_gpu(w, gpu, out=out, final_state=fin, workspace=ws_buf[G:G + need], path="fused")
    for buf, val in ((out_buf, 12345.0), (st_buf, -777.0)):
        assert torch.all(buf[:G] == val) and torch.all(buf[-G:] == val)
    assert torch.all(ws_buf[:G] == 0xA5) and torch.all(ws_buf[-G:] == 0xA5)
    compare(w, o, s, run_oracle(w), bf16_tol, "fused canary run")


def test_automatic_rule_picks_fused_from_256_pairs(gpu):
    """Without a path flag, 256 pairs run the single pass: bitwise equal to the
    forced fused call and, with a workspace sized for it, accepted."""
    _banner("automatic path rule at 256 pairs")
    w = workloads.make([20] * 64, 4, seed=43, init_std=0.02)
    oa, sa = run_gpu(w, gpu)
    of, sf = run_gpu(w, gpu, path="fused")
    assert torch.equal(oa, of) and torch.equal(sa, sf)
    os_, ss = run_gpu(w, gpu, path="split")
    assert not torch.equal(oa, os_)  # the two paths round differently
    compare(w, oa, sa, run_oracle(w, pairs=[(0, 0), (63, 3), (31, 2)]), bf16_tol, "auto at 256 pairs")


def test_more_sequences_than_the_longest_first_ranking(gpu):
    """Beyond 1024 sequences the chunk map keeps the input order for the single pass."""
    _banner("1100 packed sequences of 5..40 tokens, H=1 (input order), and 1000 (ranked)")
    import random
    rng = random.Random(44)
    for count in (1100, 1000):
        lens = [rng.randint(5, 40) for _ in range(count)]
        w = workloads.make(lens, 1, seed=44 + count, init_std=0.02)
        o, s = run_gpu(w, gpu, path="fused")
        compare(w, o, s, run_oracle(w), bf16_tol, f"fused, {count} sequences")
