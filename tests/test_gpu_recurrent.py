"""GPU parity of the token-by-token path (path="recurrent", the decode and
short-sequence kernel) against the fp64 oracle, through the C ABI.

The kernel evaluates the recurrence in fp32, so beside the bf16 bound it is
held to the fp32 path's bound (max|x_gpu - x_ref| <= 1e-5 max|x_ref|) on fp32
I/O. Decode is checked as the pages use it: one token per call, the state
passed from call to call in place.
"""
import numpy as np
import pytest
import torch

import kimi_delta_attention_k1_amd as kda
from kimi_delta_attention_k1_amd import workloads
from tests.gpu_helpers import bf16_tol, compare, f32_tol, run_gpu, run_oracle

pytestmark = pytest.mark.gpu


def _banner(name):
    print(f"\n[case] recurrent: {name}", flush=True)


def test_d1_decode_step_all_pairs(gpu):
    _banner("d1 decode step, 256 sequences x 1 token, H=32 (auto path)")
    w = workloads.d1()
    ref = run_oracle(w, threads=8)
    o, s = run_gpu(w, gpu)
    compare(w, o, s, ref, bf16_tol, "d1 decode (auto)")
    o2, s2 = run_gpu(w, gpu, path="recurrent")
    assert torch.equal(o, o2) and torch.equal(s, s2)  # the rule picked this kernel


@pytest.mark.parametrize("state_dtype", [torch.float32, torch.bfloat16])
def test_short_ragged_sequences(gpu, state_dtype):
    _banner(f"lengths 0..5 and 17, 33, H=3, {state_dtype} state")
    w = workloads.make([1, 0, 2, 3, 5, 4, 1, 17, 33], 3, seed=51, init_std=0.05)
    if state_dtype == torch.bfloat16:
        w.initial_state = w.initial_state.to(torch.bfloat16).to(torch.float32)  # exact in bf16
    ref = run_oracle(w)
    o, s = run_gpu(w, gpu, state_dtype=state_dtype, path="recurrent")
    assert s.dtype == state_dtype
    compare(w, o, s, ref, bf16_tol, f"short ragged {state_dtype}")
    assert torch.equal(s[1].cpu().float(), w.initial_state[1])  # empty sequence: final = initial


def test_fp32_io_meets_fp32_bound(gpu):
    _banner("fp32 I/O, lengths 1, 16, 64, 7: fp32 tolerance")
    w = workloads.make([1, 16, 64, 7], 2, seed=52, dtype=torch.float32, init_std=0.02)
    compare(w, *run_gpu(w, gpu, path="recurrent"), run_oracle(w), f32_tol, "recurrent fp32 I/O")


@pytest.mark.parametrize("lb", [0.0, -1.0, -10.0])
def test_longer_sequences_and_lower_bounds(gpu, lb):
    """Several 16-token activation blocks and a ragged last block."""
    _banner(f"lengths 300, 45, lower_bound {lb}")
    w = workloads.make([300, 45], 2, seed=53, init_std=0.02, lower_bound=lb)
    compare(w, *run_gpu(w, gpu, path="recurrent"), run_oracle(w), bf16_tol, f"recurrent lb={lb}")


def test_token_at_a_time_decode_in_place(gpu):
    """Feeding a 40-token sequence one token per call, with final_state aliasing
    initial_state, equals the oracle on the whole sequence."""
    _banner("40 decode calls, state in place")
    T, H = 40, 4
    w = workloads.make([T], H, seed=54, init_std=0.02)
    ref = run_oracle(w)
    state = w.initial_state.to(gpu).contiguous()
    cu = torch.tensor([0, 1], dtype=torch.int32, device=gpu)
    outs = []
    for t in range(T):
        sl = lambda x: x[t:t + 1].to(gpu).contiguous()  # noqa: E731
        o, s = kda.fwd(sl(w.q), sl(w.k), sl(w.v), sl(w.g_raw), sl(w.beta_raw), lower_bound=w.lower_bound,
                       initial_state=state, final_state=state, cu_seqlens=cu)
        assert s.data_ptr() == state.data_ptr()
        outs.append(o)
    torch.cuda.synchronize()
    compare(w, torch.cat(outs), state, ref, bf16_tol, "decode x40 in place")


def test_batch_mode_equals_packed_and_determinism(gpu):
    _banner("batch rows of 3 tokens == packed; bitwise repeatable")
    w = workloads.make([3] * 5, 2, seed=55, packed=False, init_std=0.02)
    ob, sb = run_gpu(w, gpu, path="recurrent")
    ob2, sb2 = run_gpu(w, gpu)  # auto: 3 tokens per sequence
    assert torch.equal(ob, ob2) and torch.equal(sb, sb2)
    w.packed = True
    op, sp = run_gpu(w, gpu, path="recurrent")
    assert torch.equal(ob, op) and torch.equal(sb, sp)
    compare(w, op, sp, run_oracle(w), bf16_tol, "recurrent batch/packed")


def test_guard_bytes(gpu):
    _banner("canary bytes around out, final_state and the chunk-map-only workspace")
    w = workloads.make([2, 5, 1], 4, seed=56, init_std=0.02)
    G = 4096
    T, H = w.T_tot, w.H
    n_out = T * H * 128
    need = kda.workspace_size(1, T, w.N, H, path="recurrent")
    out_buf = torch.full((n_out + 2 * G,), 12345.0, dtype=torch.bfloat16, device=gpu)
    st_buf = torch.full((w.N * H * 128 * 128 + 2 * G,), -777.0, device=gpu)
    ws_buf = torch.full((need + 2 * G,), 0xA5, dtype=torch.uint8, device=gpu)
    out = out_buf[G:G + n_out].view(T, H, 128)
    fin = st_buf[G:G + w.N * H * 128 * 128].view(w.N, H, 128, 128)
    o, s = run_gpu(w, gpu, out=out, final_state=fin, workspace=ws_buf[G:G + need], path="recurrent")
    for buf, val in ((out_buf, 12345.0), (st_buf, -777.0)):
        assert torch.all(buf[:G] == val) and torch.all(buf[-G:] == val)
    assert torch.all(ws_buf[:G] == 0xA5) and torch.all(ws_buf[-G:] == 0xA5)
    compare(w, o, s, run_oracle(w), bf16_tol, "recurrent canary run")


def test_agrees_with_chunked_paths(gpu):
    """On 64-token sequences the token-by-token result matches both chunked
    paths to the bf16 bound (each is checked against the oracle elsewhere)."""
    _banner("recurrent vs split vs fused on 64-token sequences")
    w = workloads.make([64, 64, 64], 2, seed=57, init_std=0.02)
    res = {p: run_gpu(w, gpu, path=p) for p in ("recurrent", "split", "fused")}
    for p in ("split", "fused"):
        for i, what in ((0, "o"), (1, "state")):
            a, b = res["recurrent"][i].float(), res[p][i].float()
            err = (a - b).abs().max().item()
            tol = 1e-2 * a.abs().max().item() + 1e-3
            print(f"recurrent vs {p} {what}: {err:.3e} (bound {tol:.3e})", flush=True)
            assert err <= tol
