"""The chunk map that every forward call builds first (the workspace's header flag,
token offsets, chunk offsets, segment offsets and the longest-first order), read
back from the workspace and compared with its definition, computed here: cu_seqlens
clamped into [0, T_tot] and made non-decreasing (a running maximum, first entry 0,
last T_tot), chunks of 16 tokens per sequence, exclusive scans, the segments of
each sequence (the first 3/2 as long as the others) and the sequences ranked by
chunk count, longest first, ties by index (beyond 1024 sequences the order is
the input order). One wave builds it for up to 63 sequences (one entry per lane)
and up to 127 (two), one workgroup beyond; the cases cover each.
"""
import numpy as np
import pytest
import torch

import kimi_delta_attention_k1_amd as kda
from kimi_delta_attention_k1_amd import workloads

pytestmark = pytest.mark.gpu

HEADER = 128  # bytes before the token offsets


def _align(x):
    return (x + 127) // 128 * 128


def _expected(cu, T_tot, seg_len=None, seg_first=None):
    cu = np.asarray(cu, dtype=np.int64)
    N = len(cu) - 1
    c = np.clip(cu, 0, T_tot)
    c[0], c[N] = 0, T_tot
    ok = bool(np.all(c == cu) and np.all(np.diff(cu) >= 0))
    tok = np.maximum.accumulate(c)
    cnt = (np.diff(tok) + 15) // 16
    chk = np.concatenate([[0], np.cumsum(cnt)])
    order = sorted(range(N), key=lambda n: (-cnt[n], n)) if N <= 1024 else list(range(N))
    seg = None
    if seg_len is not None:
        segs = [0 if x <= 0 else 1 if x <= seg_first else 1 + (x - seg_first + seg_len - 1) // seg_len for x in cnt]
        seg = np.concatenate([[0], np.cumsum(segs)])
    return ok, tok, chk, order, seg


def _seg_len(N, H, n_c):
    G = max(2, 256 // (N * H))
    A = -(-n_c // N)
    return max(8, (2 * A + 2 * G) // (2 * G + 1))


def _cu(N, rng, malformed):
    lens = rng.integers(0, 70, size=N)
    lens[rng.integers(0, N)] += 40  # at least one sequence longer than a chunk
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T_tot = int(cu[-1])
    if malformed:
        bad = cu.copy()
        for i in rng.choice(N + 1, size=max(1, (N + 1) // 4), replace=False):
            bad[i] = rng.choice([-5, T_tot + 9, int(rng.integers(0, T_tot + 1))])
        cu = bad
    return cu, T_tot


@pytest.mark.parametrize("path", ["fused", "segmented", "recurrent"])
@pytest.mark.parametrize("N", [1, 7, 63, 64, 127, 150, 300, 1100])
@pytest.mark.parametrize("malformed", [False, True])
def test_chunk_map_against_its_definition(gpu, path, N, malformed):
    print(f"\n[case] chunk map: {path}, N={N}, malformed={malformed}", flush=True)
    rng = np.random.default_rng(1000 * N + 2 * malformed + ["fused", "segmented", "recurrent"].index(path))
    cu, T_tot = _cu(N, rng, malformed)
    H = 1
    w = workloads.make([T_tot], H, seed=N)
    q, k, v, g, b = (t.to(gpu) for t in (w.q, w.k, w.v, w.g_raw, w.beta_raw))
    need = kda.workspace_size(1, T_tot, N, H, path=path)
    ws = torch.zeros(need, dtype=torch.uint8, device=gpu)
    cu_d = torch.tensor(cu, dtype=torch.int32, device=gpu)
    kda.fwd(q, k, v, g, b, cu_seqlens=cu_d, workspace=ws, path=path)
    torch.cuda.synchronize(gpu)
    raw = ws.cpu().numpy().view(np.int32)
    n_c = (T_tot + 15 * N) // 16
    L = _seg_len(N, H, n_c) if path == "segmented" else None
    ok, tok, chk, order, seg = _expected(cu, T_tot, L, None if L is None else L + (L + 1) // 2)
    at = lambda byte, n: raw[byte // 4: byte // 4 + n]  # noqa: E731
    t_off = HEADER
    c_off = _align(t_off + 4 * (N + 1))
    u_off = _align(c_off + 4 * (N + 1))
    assert int(raw[0]) == int(ok)
    assert np.array_equal(at(t_off, N + 1), tok)
    assert np.array_equal(at(c_off, N + 1), chk)
    if path == "fused":
        assert list(at(u_off, N)) == order
    elif path == "segmented":
        assert np.array_equal(at(u_off, N + 1), seg)
