"""GPU parity of the segmented single pass (path="segmented", KDA_FLAG_SEGMENTED)
against the fp64 oracle, through the C ABI.

The segmented pass cuts each sequence into time segments, runs every segment
from a zero state and from the identity (the segment's key-space transfer),
then scans the segments and corrects the outputs; the result must meet the
same bounds as every bf16 path (max|x_gpu - x_ref| <= 1e-2 max|x_ref| + 1e-3
for o and the final state). Segments are 8 chunks long or more, so the small
cases below already span several segments and ragged segment ends.
"""
import numpy as np
import pytest
import torch

import kimi_delta_attention_k1_amd as kda
from kimi_delta_attention_k1_amd import workloads
from tests.gpu_helpers import bf16_tol, compare, run_gpu, run_oracle

pytestmark = pytest.mark.gpu


def _banner(name):
    print(f"\n[case] segmented: {name}", flush=True)


def test_c2_full_auto_picks_segmented(gpu):
    _banner("c2 B=1 T=4096 H=16, automatic rule, all pairs")
    w = workloads.c2()
    ref = run_oracle(w)
    o, s = run_gpu(w, gpu)  # 16 pairs of 256 chunks: the rule picks the segmented pass
    assert torch.isfinite(o).all() and torch.isfinite(s).all()
    compare(w, o, s, ref, bf16_tol, "c2 segmented (auto)")
    o2, s2 = run_gpu(w, gpu, path="segmented")
    assert torch.equal(o, o2) and torch.equal(s, s2)  # the rule did pick it; runs are deterministic


def test_c4_long_context_sampled_and_against_split(gpu):
    _banner("c4 long context T=131072, H=32 (sampled heads), segmented vs split")
    w = workloads.c4()
    ref = run_oracle(w, pairs=[(0, 0), (0, 13), (0, 31)])
    o, s = run_gpu(w, gpu, path="segmented")
    assert torch.isfinite(o).all() and torch.isfinite(s).all()
    compare(w, o, s, ref, bf16_tol, "c4 segmented sampled")
    o2, s2 = run_gpu(w, gpu, path="split")
    for a, b, what in ((o, o2, "o"), (s, s2, "state")):
        a32, b32 = a.float(), b.float()
        err = (a32 - b32).abs().max().item()
        tol = 1e-2 * b32.abs().max().item() + 1e-3
        print(f"c4 segmented vs split {what}: max diff {err:.3e} (bound {tol:.3e})", flush=True)
        assert err <= tol


@pytest.mark.parametrize("lb", [-10.0, -5.0, -1.0, 0.0])
def test_ragged_segments_and_empty_sequences(gpu, lb):
    _banner(f"ragged lengths around the 256-token segment, empty sequences, lb={lb}")
    lens = [0, 1, 255, 256, 257, 700, 1000, 33, 0, 513]
    w = workloads.make(lens, 3, seed=11, init_std=0.02, beta_mean=0.5, lower_bound=lb)
    ref = run_oracle(w)
    o, s = run_gpu(w, gpu, path="segmented")
    compare(w, o, s, ref, bf16_tol, f"segmented ragged lb={lb}")
    for n in (0, 8):  # empty sequences: final = initial
        assert torch.equal(s[n].cpu(), w.initial_state[n])


def test_segment_counts_five_six_seven(gpu):
    # 3 sequences x 2 heads: segments of L = 8 chunks after a first one of 12, so
    # 44, 52 and 60 chunks make 5, 6 and 7 segments. The scan walks segments 1..G-1
    # two at a time and then the one left over: 4, 5 and 6 steps cover two pairs,
    # two pairs and a tail of one, and three pairs.
    _banner("segment counts 5, 6 and 7 (scan pairs and tails), H=2, initial state")
    w = workloads.make([704, 832, 960], 2, seed=13, init_std=0.02, beta_mean=0.5)
    ref = run_oracle(w)
    o, s = run_gpu(w, gpu, path="segmented")
    compare(w, o, s, ref, bf16_tol, "segmented, 5/6/7 segments")


def test_one_pair_many_segments(gpu):
    # one pair of 4096 chunks: G = 256 segments wanted, L = 16 chunks after a first one
    # of 24, so 256 segments: a long scan and 255 corrected segments
    _banner("one sequence of 65536 tokens, H=1: 256 segments")
    w = workloads.make([65536], 1, seed=14, init_std=0.02, beta_mean=0.5)
    ref = run_oracle(w)
    o, s = run_gpu(w, gpu, path="segmented")
    compare(w, o, s, ref, bf16_tol, "segmented, 256 segments")


def test_batch_mode_no_initial_state_no_final(gpu):
    _banner("batch mode B=2 T=1000 H=4, no initial state, no final state")
    w = workloads.make([1000, 1000], 4, seed=12, packed=False)
    ref = run_oracle(w)
    o, s = run_gpu(w, gpu, path="segmented", final=False)
    assert s is None
    compare(w, o, None, ref, bf16_tol, "segmented batch mode")


def test_bf16_state_streaming_in_place(gpu):
    _banner("bf16 states, in-place streaming over two calls of 1200 + 900 tokens, H=2")
    w = workloads.make([2100], 2, seed=13, init_std=0.02)
    ref = run_oracle(w)
    dev = gpu
    st = w.initial_state.to(dev, torch.bfloat16).contiguous()
    cut = 1200
    outs = []
    for a, e in ((0, cut), (cut, 2100)):
        sl = lambda t: t[a:e].contiguous().to(dev)  # noqa: E731
        o, _ = kda.fwd(sl(w.q)[None], sl(w.k)[None], sl(w.v)[None], sl(w.g_raw)[None], sl(w.beta_raw)[None],
                       lower_bound=w.lower_bound, initial_state=st, final_state=st, path="segmented")
        outs.append(o[0])
    torch.cuda.synchronize(dev)
    o = torch.cat(outs)
    compare(w, o, st.float(), ref, bf16_tol, "segmented bf16 streaming in place")


def test_scalar_gate(gpu):
    _banner("scalar per-head gate, lengths 600 and 300, H=3")
    w = workloads.make([600, 300], 3, seed=14, init_std=0.02, scalar_gate=True)
    ref = run_oracle(w)
    o, s = run_gpu(w, gpu, path="segmented")
    compare(w, o, s, ref, bf16_tol, "segmented scalar gate")
    # bitwise the same as the same gate broadcast over the 128 channels
    wb = workloads.make([600, 300], 3, seed=14, init_std=0.02, scalar_gate=True)
    wb.g_raw = wb.g_raw[..., None].expand(*wb.g_raw.shape, 128).contiguous()
    ob, sb = run_gpu(wb, gpu, path="segmented")
    assert torch.equal(o, ob) and torch.equal(s, sb)


def test_guard_bytes_around_outputs_and_workspace(gpu):
    _banner("guard bytes after out, final state and the workspace")
    w = workloads.make([300, 45], 2, seed=15, init_std=0.02)
    dev = gpu
    T, H = w.T_tot, w.H
    cu = w.cu_seqlens().to(dev)
    ws_bytes = kda.workspace_size(1, T, w.N, H, path="segmented")
    guard = 4096
    ws = torch.full((ws_bytes + guard,), 0x5A, dtype=torch.uint8, device=dev)
    ob = torch.full((T * H * 128 + guard // 2,), 7.0, dtype=torch.bfloat16, device=dev)
    sb = torch.full((w.N * H * 128 * 128 + guard // 4,), 3.0, dtype=torch.float32, device=dev)
    out = ob[:T * H * 128].view(T, H, 128)
    fs = sb[:w.N * H * 128 * 128].view(w.N, H, 128, 128)
    o, s = kda.fwd(w.q.to(dev), w.k.to(dev), w.v.to(dev), w.g_raw.to(dev), w.beta_raw.to(dev),
                   lower_bound=w.lower_bound, initial_state=w.initial_state.to(dev), cu_seqlens=cu, out=out,
                   final_state=fs, workspace=ws[:ws_bytes], path="segmented")
    torch.cuda.synchronize(dev)
    assert (ws[ws_bytes:] == 0x5A).all()
    assert (ob[T * H * 128:] == 7.0).all()
    assert (sb[w.N * H * 128 * 128:] == 3.0).all()
    compare(w, o, s, run_oracle(w), bf16_tol, "segmented with guards")


def test_stage_entry_points_compose_to_kda_fwd(gpu):
    _banner("kda_fwd_seg_pass + kda_fwd_seg_finish == kda_fwd (bitwise), lengths 700 and 260, H=2")
    w = workloads.make([700, 260], 2, seed=16, init_std=0.02)
    dev = gpu
    args = [t.to(dev) for t in (w.q, w.k, w.v, w.g_raw, w.beta_raw)]
    cu = w.cu_seqlens().to(dev)
    s0 = w.initial_state.to(dev)
    whole = kda.prepare_call(*args, lower_bound=w.lower_bound, initial_state=s0, cu_seqlens=cu, path="segmented")
    whole.run()
    staged = kda.prepare_call(*args, lower_bound=w.lower_bound, initial_state=s0, cu_seqlens=cu, path="segmented")
    staged.seg_pass()
    staged.seg_finish()
    torch.cuda.synchronize(dev)
    assert torch.equal(whole.out, staged.out) and torch.equal(whole.final_state, staged.final_state)
    compare(w, staged.out, staged.final_state, run_oracle(w), bf16_tol, "segmented staged")


@pytest.mark.parametrize("N,H,T,expect", [
    (64, 2, 896, "segmented"),   # 128 pairs, 56 chunks per sequence
    (64, 2, 880, "fused"),       # 128 pairs, 55 chunks: too short to segment
    (43, 3, 2048, "fused"),      # 129 pairs: two segments per pair no longer fit one round
    (27, 3, 896, "segmented"),   # 81 pairs of 56 chunks
    (27, 3, 640, "fused"),       # 81 pairs of 40 chunks: above 80 pairs the threshold is 56
    (20, 4, 640, "segmented"),   # 80 pairs of 40 chunks: up to 80 pairs it is 40
    (20, 4, 624, "fused"),       # 80 pairs of 39 chunks: the single pass from 64 pairs on
    (21, 3, 624, "split"),       # 63 pairs of 39 chunks
    (21, 3, 640, "segmented"),   # 63 pairs of 40 chunks
    (8, 4, 128, "fused"),        # 32 pairs of 8 chunks: short sequences take the single pass
    (8, 4, 144, "split"),        # 9 chunks per sequence
])
def test_automatic_rule_boundaries(gpu, N, H, T, expect):
    """Without a path flag, kda_fwd runs exactly the path the rule names (bitwise
    equal to the forced call) on either side of each threshold, and meets the oracle
    on the first, a middle and the last (sequence, head) pair."""
    _banner(f"automatic rule: {N} x {T} tokens, H={H} ({N * H} pairs) -> {expect}")
    w = workloads.make([T] * N, H, seed=17, packed=False)
    oa, sa = run_gpu(w, gpu)
    oe, se = run_gpu(w, gpu, path=expect)
    assert torch.equal(oa, oe) and torch.equal(sa, se)
    ref = run_oracle(w, pairs=[(0, 0), (N // 2, H // 2), (N - 1, H - 1)])
    compare(w, oa, sa, ref, bf16_tol, f"automatic rule {N * H} pairs ({expect})")
