"""GPU parity: the HIP library through its C ABI against the fp64 oracle.

The cases here run the two-kernel path (and its fp32 form) unless they name another
path; the full-size workloads run the automatic rule. The automatic rule sends short
sequences to the single pass, whose edge cases tests/test_gpu_fused.py covers.

Tolerances (global max over the compared tensor):
  bf16 I/O : max|x_gpu - x_ref| <= 1e-2 max|x_ref| + 1e-3, for o and the final state
  fp32 path: max|x_gpu - x_ref| <= 1e-5 max|x_ref|
Every case, the full-size workloads on the automatic path included, is
compared with the oracle on every (sequence, head) pair.
"""
import numpy as np
import pytest
import torch

import kimi_delta_attention_k1_amd as kda
from kimi_delta_attention_k1_amd import workloads
from oracle import chunked
from tests.gpu_helpers import bf16_tol, compare, f32_tol, np64, run_oracle
from tests.gpu_helpers import run_gpu as _run_gpu

pytestmark = pytest.mark.gpu


def _banner(name):
    print(f"\n[case] {name}", flush=True)


def run_gpu(w, dev, **kw):
    kw.setdefault("path", "split")
    return _run_gpu(w, dev, **kw)


# ------------------------------------------------------------------ named workloads
def test_c1_fp32_path(gpu):
    _banner("c1 fp32 I/O, NULL and explicit-zero initial state")
    w = workloads.c1()
    ref = run_oracle(w)
    o, s = run_gpu(w, gpu)
    compare(w, o, s, ref, f32_tol, "c1 fp32 (NULL init)")
    o2, s2 = run_gpu(w, gpu, initial_state=torch.zeros(1, 1, 128, 128))
    compare(w, o2, s2, ref, f32_tol, "c1 fp32 (zero init)")


def test_c2_bf16_all_pairs(gpu):
    _banner("c2 bf16 matrix-core path, all 16 heads")
    w = workloads.c2()
    ref = run_oracle(w)
    o, s = run_gpu(w, gpu)
    compare(w, o, s, ref, bf16_tol, "c2 bf16")


def test_c2_fp32_compute_flag(gpu):
    _banner("c2 bf16 I/O through the fp32 reference kernels")
    w = workloads.c2()
    ref = run_oracle(w, pairs=[(0, h) for h in range(0, 16, 3)])
    o, s = run_gpu(w, gpu, fp32_compute=True)
    compare(w, o, s, ref, bf16_tol, "c2 fp32-compute")
    # the state stays fp32 end to end: much tighter than the bf16 bound
    worst = max(np.max(np.abs(np64(s[0, h]) - ref[(0, h)][1])) for (_, h) in ref) / \
        max(np.max(np.abs(r[1])) for r in ref.values())
    print(f"c2 fp32-compute state rel err {worst:.2e}", flush=True)
    assert worst < 1e-4


def _all_pairs(w):
    return [(n, h) for n in range(w.N) for h in range(w.H)]


def test_c3_all_pairs(gpu):
    _banner("c3 packed 8 x 8192, H=32, automatic path (single pass), all 256 pairs")
    w = workloads.c3()
    o, s = run_gpu(w, gpu, path="auto")
    assert torch.isfinite(o).all() and torch.isfinite(s).all()
    compare(w, o, s, run_oracle(w, pairs=_all_pairs(w)), bf16_tol, "c3 bf16 all pairs")


def test_c4_all_heads(gpu):
    _banner("c4 long context T=131072, H=32, automatic path (segmented), all 32 heads")
    w = workloads.c4()
    o, s = run_gpu(w, gpu, path="auto")
    assert torch.isfinite(o).all() and torch.isfinite(s).all()
    compare(w, o, s, run_oracle(w, pairs=_all_pairs(w)), bf16_tol, "c4 bf16 all heads")


def test_c5_all_pairs(gpu):
    _banner("c5 ragged 64 sequences, H=32, automatic path (single pass), all 2048 pairs")
    w = workloads.c5()
    o, s = run_gpu(w, gpu, path="auto")
    assert torch.isfinite(o).all() and torch.isfinite(s).all()
    compare(w, o, s, run_oracle(w, pairs=_all_pairs(w)), bf16_tol, "c5 bf16 all pairs")


# ------------------------------------------------------------------ edge cases (all pairs)
def test_ragged_tails_and_empty_sequences(gpu):
    _banner("ragged: lengths 1,15,16,17,0,33,100 with initial state")
    w = workloads.make([1, 15, 16, 17, 0, 33, 100], 4, seed=7, init_std=0.02, beta_mean=0.5)
    ref = run_oracle(w)
    o, s = run_gpu(w, gpu)
    compare(w, o, s, ref, bf16_tol, "ragged bf16")
    assert torch.equal(s[4].cpu(), w.initial_state[4])  # empty sequence: final = initial
    o, s = run_gpu(w, gpu, fp32_compute=True)
    compare(w, o, s, ref, bf16_tol, "ragged fp32-compute")


@pytest.mark.parametrize("H", [1, 3, 6])
def test_head_counts(gpu, H):
    _banner(f"heads H={H}")
    w = workloads.make([50, 31], H, seed=100 + H, init_std=0.02)
    compare(w, *run_gpu(w, gpu), run_oracle(w), bf16_tol, f"H={H}")


def test_fp32_io_ragged(gpu):
    _banner("fp32 I/O ragged")
    w = workloads.make([3, 40, 16], 2, seed=9, dtype=torch.float32, init_std=0.02)
    compare(w, *run_gpu(w, gpu), run_oracle(w), f32_tol, "fp32 ragged")


def test_batch_mode_equals_packed(gpu):
    _banner("batch rows == packed equal-length sequences (bitwise)")
    w = workloads.make([40, 40, 40], 2, seed=11, packed=False, init_std=0.02)
    ob, sb = run_gpu(w, gpu)
    w.packed = True
    op, sp = run_gpu(w, gpu)
    assert torch.equal(ob, op) and torch.equal(sb, sp)
    compare(w, op, sp, run_oracle(w), bf16_tol, "batch/packed")


def test_streaming_state_passing(gpu):
    _banner("streaming: run(T) vs run(T1) then run(T-T1)")
    T, T1, H = 200, 71, 2
    w = workloads.make([T], H, seed=13, init_std=0.02)
    ref = run_oracle(w)
    o, s = run_gpu(w, gpu)
    w1 = workloads.make([T], H, seed=13, init_std=0.02)
    a = workloads.Workload("a", w1.q[:T1], w1.k[:T1], w1.v[:T1], w1.g_raw[:T1], w1.beta_raw[:T1], [T1], True,
                           w1.initial_state)
    oa, sa = run_gpu(a, gpu)
    b = workloads.Workload("b", w1.q[T1:], w1.k[T1:], w1.v[T1:], w1.g_raw[T1:], w1.beta_raw[T1:], [T - T1], True,
                           sa.cpu())
    ob, sb = run_gpu(b, gpu)
    o2 = torch.cat([oa, ob])
    compare(w, o2, sb, ref, bf16_tol, "streamed")
    compare(w, o, s, ref, bf16_tol, "one call")


def test_inplace_state_and_determinism(gpu):
    _banner("final_state aliasing initial_state; bitwise determinism")
    w = workloads.make([300, 77], 4, seed=17, init_std=0.02)
    o1, s1 = run_gpu(w, gpu)
    o2, s2 = run_gpu(w, gpu)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    buf = w.initial_state.to(gpu).contiguous()
    q, k, v, g, b = (t.to(gpu) for t in (w.q, w.k, w.v, w.g_raw, w.beta_raw))
    o3, s3 = kda.fwd(q, k, v, g, b, initial_state=buf, final_state=buf, cu_seqlens=w.cu_seqlens().to(gpu),
                     path="split")
    torch.cuda.synchronize()
    assert s3.data_ptr() == buf.data_ptr()
    assert torch.equal(o3, o1) and torch.equal(s3, s1)


def test_bf16_state_and_no_final_state(gpu):
    _banner("bf16 states; final state not requested")
    w = workloads.make([90, 33], 2, seed=19, init_std=0.05)
    w.initial_state = w.initial_state.to(torch.bfloat16).to(torch.float32)  # exact in bf16
    ref = run_oracle(w)
    o, s = run_gpu(w, gpu, state_dtype=torch.bfloat16)
    assert s.dtype == torch.bfloat16
    compare(w, o, s, ref, bf16_tol, "bf16 state")
    o2, s2 = run_gpu(w, gpu, final=False)
    assert s2 is None
    compare(w, o2, None, ref, bf16_tol, "no final state")


def test_empty_batch_copies_state(gpu):
    _banner("T = 0 batch mode: final = initial")
    s0 = torch.randn(2, 3, 128, 128, device=gpu)
    z = torch.empty(2, 0, 3, 128, dtype=torch.bfloat16, device=gpu)
    o, s = kda.fwd(z, z, z, z, torch.empty(2, 0, 3, dtype=torch.bfloat16, device=gpu), initial_state=s0)
    torch.cuda.synchronize()
    assert o.shape == z.shape and torch.equal(s, s0)


@pytest.mark.parametrize("lb", [0.0, -1.0, -10.0])
def test_lower_bound_range(gpu, lb):
    _banner(f"lower_bound {lb}")
    w = workloads.make([64, 45], 2, seed=23, init_std=0.02, lower_bound=lb)
    ref = run_oracle(w)
    compare(w, *run_gpu(w, gpu), ref, bf16_tol, f"lb={lb}")
    compare(w, *run_gpu(w, gpu, fp32_compute=True), ref, bf16_tol, f"lb={lb} fp32-compute")


def test_malformed_cu_seqlens_are_clamped(gpu):
    _banner("malformed cu_seqlens: clamped on the device, flag cleared")
    w = workloads.make([100], 2, seed=29)
    q, k, v, g, b = (t.to(gpu) for t in (w.q, w.k, w.v, w.g_raw, w.beta_raw))
    ws = torch.empty(kda.workspace_size(1, 100, 3, 2), dtype=torch.uint8, device=gpu)
    good = torch.tensor([0, 50, 50, 100], dtype=torch.int32, device=gpu)
    bad = torch.tensor([0, 50, 30, 200], dtype=torch.int32, device=gpu)  # clamps to [0, 50, 50, 100]
    o1, s1 = kda.fwd(q, k, v, g, b, cu_seqlens=good, workspace=ws)
    assert kda.seqlens_flag(ws) == 1
    o2, s2 = kda.fwd(q, k, v, g, b, cu_seqlens=bad, workspace=ws)
    assert kda.seqlens_flag(ws) == 0
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_guard_bytes_untouched(gpu):
    _banner("canary bytes around out, final_state and workspace")
    w = workloads.make([37, 64], 4, seed=31, init_std=0.02)
    G = 4096
    T, H = w.T_tot, w.H
    n_out = T * H * 128
    out_buf = torch.full((n_out + 2 * G,), 12345.0, dtype=torch.bfloat16, device=gpu)
    st_buf = torch.full((w.N * H * 128 * 128 + 2 * G,), -777.0, device=gpu)
    need = kda.workspace_size(1, T, w.N, H)
    ws_buf = torch.full((need + 2 * G,), 0xA5, dtype=torch.uint8, device=gpu)
    out = out_buf[G:G + n_out].view(T, H, 128)
    fin = st_buf[G:G + w.N * H * 128 * 128].view(w.N, H, 128, 128)
    o, s = run_gpu(w, gpu, out=out, final_state=fin, workspace=ws_buf[G:G + need])
    for buf, val in ((out_buf, 12345.0), (st_buf, -777.0)):
        assert torch.all(buf[:G] == val) and torch.all(buf[-G:] == val)
    assert torch.all(ws_buf[:G] == 0xA5) and torch.all(ws_buf[-G:] == 0xA5)
    compare(w, o, s, run_oracle(w), bf16_tol, "canary run")


# ------------------------------------------------------------------ K1 intermediates
def _decode_unit(raw: torch.Tensor):
    """Unpack one bf16-path workspace unit (18944 bytes) into row-major tiles.
    The fragment order is the recurrence kernel's matrix-core operand order; K_end
    is a bf16 hi/lo pair (2 KB per tile pair; per lane: tile 2p hi, lo, tile 2p+1 hi,
    lo, four tokens each)."""
    u = raw.cpu()
    bf = lambda a, b: u[a:b].view(torch.bfloat16).float().view(4, 64, 8)  # noqa: E731
    KB, QB = bf(0, 4096), bf(4096, 8192)
    KE = u[8192:16384].view(torch.bfloat16).float().view(4, 64, 2, 2, 4)  # pair, lane, tile, hi/lo, token
    kb = torch.zeros(16, 128)
    qb = torch.zeros(16, 128)
    ke = torch.zeros(16, 128)
    for p in range(4):
        for lane in range(64):
            t, g = lane % 16, lane // 16
            for e in range(8):
                ch = 32 * p + (4 * g + e if e < 4 else 16 + 4 * g + e - 4)
                kb[t, ch] = KB[p, lane, e]
                qb[t, ch] = QB[p, lane, e]
            for tt in range(2):
                for e in range(4):
                    ke[4 * g + e, 32 * p + 16 * tt + t] = KE[p, lane, tt, 0, e] + KE[p, lane, tt, 1, e]
    hl = lambda a, b: u[a:b].view(torch.bfloat16).float().view(64, 2, 4).sum(1)  # noqa: E731  hi + lo
    ab = hl(16384, 17408)
    aq = hl(17408, 18432)
    AB = torch.zeros(16, 16)
    AQ = torch.zeros(16, 16)
    for lane in range(64):
        for r in range(4):
            AB[lane % 16, 4 * (lane // 16) + r] = ab[lane, r]
            AQ[lane % 16, 4 * (lane // 16) + r] = aq[lane, r]
    gm = u[18432:18944].view(torch.float32).clone()
    return dict(Kb=kb, Qb=qb, Kend=ke, Ab=AB, Aqk=AQ, gamma=gm)


def test_k1_intermediates_against_chunked_oracle(gpu):
    _banner("chunk-parallel kernel outputs vs the chunkwise oracle's intermediates")
    w = workloads.make([40, 16], 2, seed=37)
    T, H = w.T_tot, w.H
    ws = torch.zeros(kda.workspace_size(1, T, w.N, H), dtype=torch.uint8, device=gpu)
    run_gpu(w, gpu, workspace=ws, path="split")  # the chunk kernel writes the units
    f = lambda t: t.float().numpy()  # noqa: E731
    _, _, inter = chunked.forward(f(w.q), f(w.k), f(w.v), f(w.g_raw), f(w.beta_raw), w.offsets(),
                                  lower_bound=w.lower_bound, keep=True)
    N = w.N
    units = 128 + 2 * ((4 * (N + 1) + 127) // 128 * 128)  # header, tok_off, chunk_off
    n_c_max = (T + 15 * N) // 16
    s = 128 ** -0.5
    chunk = 0
    for n in range(N):
        for j, _ in enumerate(inter[(n, 0)]):
            for h in range(H):
                it = inter[(n, h)][j]
                L = it["Kb"].shape[0]
                base = units + (h * n_c_max + chunk) * 18944
                d = _decode_unit(ws[base:base + 18944])
                # K_b and Q_b are one bf16 (2^-9 relative); K_end is a hi/lo pair, so it meets
                # 2^-13, which one bf16 cannot
                for key, ref, rel in (("Kb", it["Kb"], 2 ** -8), ("Qb", s * it["Qbnd"], 2 ** -8),
                                      ("Kend", it["Kend"], 2 ** -13)):
                    got = d[key][:L].numpy()
                    assert np.all(np.abs(got - ref) <= rel * np.abs(ref) + 1e-30), key
                    assert torch.all(d[key][L:] == 0), key + " padded rows"
                ab_ref = it["Akk"] * it["beta"][None, :]
                assert np.max(np.abs(d["Ab"][:L, :L].numpy() - ab_ref)) <= 1e-4 * np.max(np.abs(ab_ref))
                assert np.max(np.abs(d["Aqk"][:L, :L].numpy() - it["Aqk"])) <= 1e-4 * np.max(np.abs(it["Aqk"]))
                assert np.allclose(d["gamma"].numpy(), it["gamma"], rtol=5e-5, atol=0)
            chunk += 1


@pytest.mark.parametrize("nseq,H", [(10, 4), (12, 6), (30, 4), (50, 4)])
def test_pair_counts_select_each_recurrence_shape(gpu, nseq, H):
    """On the two-kernel path, (sequence, head) pair counts 40, 72, 120 and 200 run the
    recurrence with 1, 2, 4 and 8 consumer waves per workgroup (8, 4, 2 and 1
    workgroups per pair; four producer waves for the first two, two for the others)."""
    _banner(f"split path: {nseq} sequences x {H} heads = {nseq * H} pairs")
    w = workloads.make(None, H, seed=41 + nseq, init_std=0.02, lens_drawn=(1, 70, nseq))
    compare(w, *run_gpu(w, gpu, path="split"), run_oracle(w), bf16_tol, f"{nseq * H} pairs")


@pytest.mark.parametrize("nseq,H,dtype", [(2, 2, torch.bfloat16), (25, 4, torch.bfloat16), (3, 2, torch.float32)])
def test_stage_entry_points_compose_to_kda_fwd(gpu, nseq, H, dtype):
    """kda_fwd_prepare followed by kda_fwd_recur gives kda_fwd's results bitwise on the
    two-kernel path: the look-ahead recurrence (4 pairs), the consumer-wave one (100)
    and the fp32 kernels (fp32 I/O)."""
    _banner(f"split path staged vs whole: {nseq} x {H}, {dtype}")
    w = workloads.make(None, H, seed=90 + nseq, dtype=dtype, init_std=0.02, lens_drawn=(1, 300, nseq))
    args = [t.to(gpu) for t in (w.q, w.k, w.v, w.g_raw, w.beta_raw)]
    cu = w.cu_seqlens().to(gpu)
    s0 = w.initial_state.to(gpu)
    whole = kda.prepare_call(*args, lower_bound=w.lower_bound, initial_state=s0, cu_seqlens=cu, path="split")
    whole.run()
    staged = kda.prepare_call(*args, lower_bound=w.lower_bound, initial_state=s0, cu_seqlens=cu, path="split")
    staged.prepare()
    staged.recur()
    torch.cuda.synchronize(gpu)
    assert torch.equal(whole.out, staged.out) and torch.equal(whole.final_state, staged.final_state)
    tol = f32_tol if dtype == torch.float32 else bf16_tol
    compare(w, staged.out, staged.final_state, run_oracle(w), tol, f"split staged {nseq}x{H}")
