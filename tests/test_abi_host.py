"""Host-side checks of the C ABI (CPU only, no kernel is ever launched).

Every kda_fwd call here carries an argument that validation rejects, so the
library returns before touching the GPU; the fake addresses are never used.
"""
import ctypes
import os
import re

import pytest

import kimi_delta_attention_k1_amd as kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

OK, NULL_ARG, BAD_SHAPE, BAD_DTYPE, BAD_SEQLENS, BAD_ARG, WORKSPACE, MISALIGNED, HIP, TOO_LARGE = range(10)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kda.library_path()):
        import __graft_entry__
        __graft_entry__.build()
    return kda.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_\w+)\s*\(", text)))


def test_header_symbols_are_exported(lib):
    names = declared_functions()
    assert {"kda_fwd", "kda_fwd_workspace_size", "kda_status_str", "kda_version"} <= set(names)
    for name in names:
        assert hasattr(lib, name), f"{name} declared in include/kda.h but not exported"


def test_version_and_status_strings(lib):
    assert lib.kda_version() >= 200
    for code in range(10):
        assert kda.status_str(code) and kda.status_str(code) != "unknown status"
    assert kda.status_str(99) == "unknown status"


def test_desc_struct_matches_header():
    # kda_desc_t: 3 x int64, 4 x int32, float, uint32 -> 48 bytes, no padding surprises
    assert ctypes.sizeof(kda.KdaDesc) == 48


def _layout(N, H, n_c, unit, look=False):
    """Header, token and chunk offsets, one unit per (chunk, head); with fewer than 96
    bf16 (sequence, head) pairs the look-ahead recurrence also keeps 4096 B per
    (chunk, head) of K_end in K_b order after the units."""
    tok = 128
    chk = (tok + 4 * (N + 1) + 127) // 128 * 128
    units = (chk + 4 * (N + 1) + 127) // 128 * 128
    end = units + unit * H * n_c
    return (end + 127) // 128 * 128 + 4096 * H * n_c if look else end


def test_workspace_size_arithmetic(lib):
    # batch mode, one sequence of 64 tokens -> 4 chunks
    assert kda.workspace_size(1, 64, 1, 1, kda.DTYPE_FP32) == _layout(1, 1, 4, 27136)
    assert kda.workspace_size(1, 64, 1, 1, kda.DTYPE_BF16) == _layout(1, 1, 4, 18944, look=True)
    # batch of 2 rows of 17 tokens -> 2 x 2 chunks
    assert kda.workspace_size(2, 17, 2, 3) == _layout(2, 3, 4, 18944, look=True)
    # 95 pairs still take the look-ahead recurrence, 96 do not
    assert kda.workspace_size(1, 160, 5, 19) == _layout(5, 19, (160 + 15 * 5) // 16, 18944, look=True)
    assert kda.workspace_size(1, 160, 6, 16) == _layout(6, 16, (160 + 15 * 6) // 16, 18944)
    # the bf16-resident-state variant keeps the plain recurrence
    assert kda.workspace_size(1, 64, 1, 1, kda.DTYPE_BF16, bf16_resident_state=True) == _layout(1, 1, 4, 18944)
    # packed: 8 x 8192 tokens (bound (T + 15 N) / 16)
    assert kda.workspace_size(1, 65536, 8, 32) == _layout(8, 32, (65536 + 15 * 8) // 16, 18944)
    # fp32 compute flag selects the fp32 unit size
    assert kda.workspace_size(1, 64, 1, 1, kda.DTYPE_BF16, fp32_compute=True) == _layout(1, 1, 4, 27136)
    # invalid descriptions report 0
    assert kda.workspace_size(1, 64, 1, 0) == 0
    d = kda.make_desc(1, 64, 1, 1, 0, 1, 0.1, head_dim=64)
    assert lib.kda_fwd_workspace_size(ctypes.byref(d)) == 0
    assert lib.kda_fwd_workspace_size(None) == 0


class Fake:
    """Disjoint, 256-B aligned fake addresses (never dereferenced)."""
    BASE = 0x7F0000000000

    def __init__(self, sizes):
        self.addr = {}
        a = self.BASE
        for name, size in sizes.items():
            self.addr[name] = a
            a += (size + (1 << 20)) // 256 * 256 + 256


def _call(lib, desc, *, cu=False, drop=(), shift=None, lb=-5.0, ws_bytes=None, overrides=None):
    d = desc if desc is not None else _desc()
    T_tot = d.seqlen if cu else d.batch * d.seqlen
    H, N = max(d.num_heads, 1), max(d.num_seqs, 1)
    esz = 2 if d.io_dtype == 0 else 4
    sizes = dict(q=T_tot * H * 128 * esz, k=T_tot * H * 128 * esz, v=T_tot * H * 128 * esz,
                 g=T_tot * H * 128 * esz, b=T_tot * H * esz, cu=4 * (N + 1), s0=N * H * 128 * 128 * 4,
                 out=T_tot * H * 128 * esz, s1=N * H * 128 * 128 * 4, ws=1 << 34)
    f = Fake(sizes)
    p = {k_: ctypes.c_void_p(v_) for k_, v_ in f.addr.items()}
    if not cu:
        p["cu"] = None
    for name in drop:
        p[name] = None
    if shift:
        for name, off in shift.items():
            p[name] = ctypes.c_void_p(f.addr[name] + off)
    if overrides:
        for name, other in overrides.items():
            p[name] = ctypes.c_void_p(f.addr[other[0]] + other[1])
    wsb = (1 << 34) if ws_bytes is None else ws_bytes
    return lib.kda_fwd(p["q"], p["k"], p["v"], p["g"], p["b"], p["cu"], p["s0"], p["out"], p["s1"],
                       ctypes.c_float(lb), ctypes.byref(desc) if desc is not None else None, p["ws"],
                       ctypes.c_size_t(wsb), None)


def _desc(**kw):
    base = dict(batch=1, seqlen=64, num_seqs=1, num_heads=2, io_dtype=0, state_dtype=1, scale=128 ** -0.5)
    base.update(kw)
    return kda.make_desc(base["batch"], base["seqlen"], base["num_seqs"], base["num_heads"], base["io_dtype"],
                         base["state_dtype"], base["scale"], base.get("flags", 0), base.get("head_dim", 128))


@pytest.mark.parametrize("case,expect", [
    (dict(desc=dict(head_dim=64)), BAD_SHAPE),
    (dict(desc=dict(num_heads=0)), BAD_SHAPE),
    (dict(desc=dict(batch=0)), BAD_SHAPE),
    (dict(desc=dict(seqlen=-1)), BAD_SHAPE),
    (dict(desc=dict(batch=2, num_seqs=3)), BAD_SHAPE),
    (dict(desc=dict(io_dtype=7)), BAD_DTYPE),
    (dict(desc=dict(state_dtype=-1)), BAD_DTYPE),
    (dict(desc=dict(batch=2, num_seqs=2), cu=True), BAD_SEQLENS),
    (dict(lb=-10.5), BAD_ARG),
    (dict(lb=0.5), BAD_ARG),
    (dict(lb=float("nan")), BAD_ARG),
    (dict(desc=dict(scale=0.0)), BAD_ARG),
    (dict(desc=dict(scale=float("inf"))), BAD_ARG),
    (dict(desc=dict(flags=128)), BAD_ARG),                   # unknown flag bit
    (dict(desc=dict(flags=kda.FLAG_SEGMENTED | kda.FLAG_FUSED)), BAD_ARG),
    (dict(desc=dict(flags=kda.FLAG_SEGMENTED | kda.FLAG_SPLIT)), BAD_ARG),
    (dict(desc=dict(flags=kda.FLAG_SEGMENTED | kda.FLAG_FP32_COMPUTE)), BAD_ARG),
    (dict(desc=dict(flags=kda.FLAG_SEGMENTED | kda.FLAG_BF16_RESIDENT_STATE)), BAD_ARG),
    (dict(desc=dict(io_dtype=1, flags=kda.FLAG_SEGMENTED)), BAD_ARG),  # fp32 I/O has no segmented pass
    (dict(desc=dict(flags=kda.FLAG_BF16_RESIDENT_STATE | kda.FLAG_FUSED)), BAD_ARG),
    (dict(desc=dict(flags=kda.FLAG_BF16_RESIDENT_STATE | kda.FLAG_RECURRENT)), BAD_ARG),
    (dict(desc=dict(flags=kda.FLAG_BF16_RESIDENT_STATE | kda.FLAG_FP32_COMPUTE)), BAD_ARG),
    (dict(desc=dict(io_dtype=1, flags=kda.FLAG_BF16_RESIDENT_STATE)), BAD_ARG),
    (dict(desc=dict(flags=kda.FLAG_RECURRENT | kda.FLAG_FUSED)), BAD_ARG),
    (dict(desc=dict(flags=kda.FLAG_RECURRENT | kda.FLAG_SPLIT)), BAD_ARG),
    (dict(desc=dict(flags=kda.FLAG_SPLIT | kda.FLAG_FUSED)), BAD_ARG),
    (dict(desc=dict(flags=kda.FLAG_FP32_COMPUTE | kda.FLAG_FUSED)), BAD_ARG),
    (dict(desc=dict(io_dtype=1, flags=kda.FLAG_FUSED)), BAD_ARG),  # fp32 I/O has no single pass
    (dict(desc=dict(num_heads=65536)), BAD_SHAPE),
    (dict(desc=dict(flags=kda.FLAG_SPLIT), ws_bytes=1024), WORKSPACE),
    (dict(drop=("q",)), NULL_ARG),
    (dict(drop=("out",)), NULL_ARG),
    (dict(drop=("ws",)), WORKSPACE),
    (dict(ws_bytes=256), WORKSPACE),  # below every path's chunk map
    (dict(shift=dict(ws=64)), WORKSPACE),
    (dict(shift=dict(q=2)), MISALIGNED),
    (dict(shift=dict(g=2)), MISALIGNED),                     # [T][H][128] g_raw needs 16 bytes
    (dict(desc=dict(flags=kda.FLAG_SCALAR_GATE), shift=dict(g=1)), MISALIGNED),  # scalar g_raw: 2 bytes
    (dict(shift=dict(s1=8)), MISALIGNED),
    (dict(overrides=dict(out=("q", 0))), BAD_ARG),          # out aliases q
    (dict(overrides=dict(s1=("s0", 256))), BAD_ARG),        # partial state overlap
    (dict(overrides=dict(ws=("v", 0))), BAD_ARG),           # workspace over an input
])
def test_validation_rejects_before_launch(lib, case, expect):
    desc = _desc(**case.get("desc", {}))
    rc = _call(lib, desc, cu=case.get("cu", False), drop=case.get("drop", ()), shift=case.get("shift"),
               lb=case.get("lb", -5.0), ws_bytes=case.get("ws_bytes"), overrides=case.get("overrides"))
    assert rc == expect, kda.status_str(rc)


def test_null_desc(lib):
    assert _call(lib, None) == NULL_ARG


def test_path_flags_and_workspace(lib):
    # the single pass needs only the chunk map; without its flag the size covers the split path
    # ... plus the longest-first order of the sequences, [N] int32
    fused = (_layout(8, 32, 0, 18944) + 4 * 8 + 127) // 128 * 128
    assert kda.workspace_size(1, 65536, 8, 32, path="fused") == fused
    assert kda.workspace_size(1, 65536, 8, 32, path="split") == kda.workspace_size(1, 65536, 8, 32)
    assert kda.workspace_size(1, 65536, 8, 32, path="auto") == _layout(8, 32, (65536 + 15 * 8) // 16, 18944)
    assert kda.workspace_size(1, 64, 1, 1, kda.DTYPE_FP32, path="fused") == 0  # invalid: fp32 I/O
    # the token-by-token path also needs only the chunk map, for any dtype
    assert kda.workspace_size(1, 65536, 8, 32, path="recurrent") == _layout(8, 32, 0, 18944)
    assert kda.workspace_size(1, 64, 1, 1, kda.DTYPE_FP32, path="recurrent") == _layout(1, 1, 0, 27136)
    with pytest.raises(ValueError):
        kda.workspace_size(1, 64, 1, 1, path="both")


def _seg_layout(N, H, T_tot, n_c):
    """Chunk map, segment offsets, three fp32 [128][128] matrices per (segment, head)
    and a bf16 [n_c][H][16][128] buffer. G = max(2, 256 // (N H)) segments per average
    sequence of A = ceil(n_c / N) chunks, the first 3/2 as long as the others:
    L = max(8, (2 A + 2 G) // (2 G + 1)), at most n_c // L + N segments."""
    G = max(2, 256 // (N * H))
    A = -(-n_c // N)
    L = max(8, (2 * A + 2 * G) // (2 * G + 1))
    smax = n_c // L + N
    seg = _layout(N, H, 0, 0)
    sfin = (seg + 4 * (N + 1) + 127) // 128 * 128
    return sfin + 3 * smax * H * 128 * 128 * 4 + n_c * H * 16 * 128 * 2


def test_segmented_path_workspace(lib):
    # C4: one sequence of 131072 tokens, H=32 -> 8192 chunks: segments of 1446 chunks, then 964
    assert kda.workspace_size(1, 131072, 1, 32, path="segmented") == _seg_layout(1, 32, 131072, 8192)
    # the automatic rule picks the segmented pass there; the size covers it and the split path
    split = _layout(1, 32, 8192, 18944, look=True)
    assert kda.workspace_size(1, 131072, 1, 32) == max(split, _seg_layout(1, 32, 131072, 8192))
    # packed few-pair batch: n_c bound (T + 15 N) / 16
    n_c = (5000 + 15 * 3) // 16
    assert kda.workspace_size(1, 5000, 3, 2, path="segmented") == _seg_layout(3, 2, 5000, n_c)
    # 256 pairs: no segments needed, the size is the split path's
    assert kda.workspace_size(1, 65536, 8, 32) == _layout(8, 32, (65536 + 15 * 8) // 16, 18944)
    # 32 pairs of 39 chunks: below the 40-chunk average (up to 80 pairs) the rule
    # keeps the split path; at 40 chunks it picks the segmented pass and the size covers both
    assert kda.workspace_size(2, 624, 2, 16) == _layout(2, 16, 78, 18944, look=True)
    assert kda.workspace_size(2, 640, 2, 16) == max(_layout(2, 16, 80, 18944, look=True),
                                                     _seg_layout(2, 16, 1280, 80))
    assert kda.workspace_size(1, 64, 1, 1, kda.DTYPE_FP32, path="segmented") == 0  # invalid: fp32 I/O


@pytest.mark.parametrize("flag", [kda.FLAG_FUSED, kda.FLAG_RECURRENT, kda.FLAG_SEGMENTED])
def test_stage_entry_points_reject_single_call_paths(lib, flag):
    desc = _desc(flags=flag)
    f = Fake(dict(x=1 << 20))
    a = ctypes.c_void_p(f.addr["x"])
    for fn in (lib.kda_fwd_prepare, lib.kda_fwd_recur):
        rc = fn(a, a, a, a, a, None, None, a, None, ctypes.c_float(-5.0), ctypes.byref(desc), a,
                ctypes.c_size_t(1 << 30), None)
        assert rc == BAD_ARG, kda.status_str(rc)


@pytest.mark.parametrize("desc_kw", [dict(flags=kda.FLAG_FUSED), dict(flags=kda.FLAG_RECURRENT),
                                     dict(flags=kda.FLAG_SPLIT), dict(flags=kda.FLAG_BF16_RESIDENT_STATE),
                                     dict(flags=kda.FLAG_FP32_COMPUTE), dict(io_dtype=1)])
def test_segmented_stage_entry_points_reject_other_paths(lib, desc_kw):
    desc = _desc(**desc_kw)
    f = Fake(dict(x=1 << 20))
    a = ctypes.c_void_p(f.addr["x"])
    for fn in (lib.kda_fwd_seg_pass, lib.kda_fwd_seg_finish):
        rc = fn(a, a, a, a, a, None, None, a, None, ctypes.c_float(-5.0), ctypes.byref(desc), a,
                ctypes.c_size_t(1 << 30), None)
        assert rc == BAD_ARG, kda.status_str(rc)


def test_bf16_resident_state_needs_a_decaying_gate(lib):
    """The bf16-resident recurrence accumulates its roundings when the state barely
    decays: lower_bound above -0.2 is rejected; at -0.2 validation goes on (here to the
    missing workspace)."""
    desc = _desc(flags=kda.FLAG_BF16_RESIDENT_STATE)
    assert _call(lib, desc, lb=0.0) == BAD_ARG
    assert _call(lib, desc, lb=-0.19) == BAD_ARG
    assert _call(lib, desc, lb=-0.2, drop=("ws",)) == WORKSPACE
    assert _call(lib, _desc(flags=kda.FLAG_SPLIT), lb=0.0, drop=("ws",)) == WORKSPACE  # fp32 state: any bound


@pytest.mark.parametrize("flags,N,H", [
    (kda.FLAG_RECURRENT, 65536, 64),  # 2^22 pairs x 8 workgroups of 128 threads = 2^32 work-items
    (kda.FLAG_FUSED, 95327, 64),      # 6,100,928 pairs x 704 threads >= 2^32
])
def test_grid_limits_rejected_before_launch(lib, flags, N, H):
    """A launch whose work-items along x reach 2^32 is refused with BAD_SHAPE before
    anything is enqueued (batch mode, one token or one chunk per sequence)."""
    T = 1 if flags == kda.FLAG_RECURRENT else 16
    desc = _desc(batch=N, seqlen=T, num_seqs=N, num_heads=H, flags=flags)
    assert _call(lib, desc) == BAD_SHAPE


def _noalloc(lib, desc, N, H, T_tot):
    f = Fake(dict(q=T_tot * H * 256, k=T_tot * H * 256, v=T_tot * H * 256, g=T_tot * H * 256, b=T_tot * H * 2,
                  cu=4 * (N + 1), out=T_tot * H * 256, s1=N * H * 65536))
    a = {k_: ctypes.c_void_p(v_) for k_, v_ in f.addr.items()}
    return lib.kda_fwd_noalloc(a["q"], a["k"], a["v"], a["g"], a["b"], a["cu"], None, a["out"], a["s1"],
                               ctypes.c_float(-5.0), ctypes.byref(desc), None)


def test_noalloc_rejects_before_any_gpu_call(lib):
    """Too many sequences for the static scratch, and the paths with a large workspace,
    are refused before the library looks up its scratch or enqueues anything."""
    N = 65537
    assert _noalloc(lib, _desc(seqlen=16 * N, num_seqs=N), N, 2, 16 * N) == TOO_LARGE
    for flags in (kda.FLAG_SPLIT, kda.FLAG_SEGMENTED, kda.FLAG_BF16_RESIDENT_STATE):
        assert _noalloc(lib, _desc(seqlen=64, num_seqs=2, flags=flags), 2, 2, 64) == BAD_ARG
    assert lib.kda_fwd_noalloc(None, None, None, None, None, None, None, None, None, ctypes.c_float(-5.0), None,
                               None) == NULL_ARG
