"""Kimi Delta Attention forward on MI355X (gfx950): Python binding.

This module only marshals arguments into the C ABI of libkda.so (declared in
include/kda.h). Every step of the computation runs in the library's HIP
kernels; PyTorch provides device memory and the current stream. There is no
CPU or PyTorch fallback: if the library is missing the calls raise.

    out, final_state = fwd(q, k, v, g_raw, beta_raw, lower_bound=-5.0,
                           initial_state=None, output_final_state=True,
                           cu_seqlens=None, path="auto")

`path` picks the kernels: "split" (chunk-parallel kernel, then recurrence
kernel), "fused" (one single-pass kernel, bf16 compute only), "segmented" (the
single pass over time segments of each sequence, then a scan over segments and
an output correction; bf16 compute only), "recurrent" (the recurrence token by
token, for decode and short sequences) or "auto" (the library's rule: recurrent
up to RECURRENT_MAX_AVG_TOKENS tokens per sequence on average, else segmented
up to SEGMENTED_MAX_PAIRS (sequence, head) pairs when the sequences average at
least SEGMENTED_MIN_AVG_CHUNKS chunks (SEGMENTED_MIN_AVG_CHUNKS_FEW_PAIRS up to
SEGMENTED_FEW_PAIRS pairs), else fused from FUSED_MIN_PAIRS pairs on
or when the sequences average at most FUSED_MAX_AVG_CHUNKS chunks, else split).

Layouts follow the FlashKDA API (DocSearch FlashKDA digest, "flash_kda.fwd API
reference"): q, k, v, g_raw are [B, T, H, 128] (or packed [T_tot, H, 128]),
beta_raw is [B, T, H] (or [T_tot, H]); states are [N, H, 128 (V), 128 (K)];
with cu_seqlens (int32, N+1 offsets) B must be 1. A g_raw shaped like beta_raw
is a scalar per-head gate (Gated DeltaNet): one value per token and head for
every key channel (KDA_FLAG_SCALAR_GATE).
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["fwd", "fwd_noalloc", "prepare_call", "Call", "workspace_size", "KdaError", "load_library", "library_path", "seqlens_flag",
           "HEAD_DIM", "CHUNK", "FLAG_FP32_COMPUTE", "FLAG_SPLIT", "FLAG_FUSED", "FLAG_RECURRENT", "FLAG_SCALAR_GATE",
           "FLAG_BF16_RESIDENT_STATE", "FLAG_SEGMENTED",
           "FUSED_MIN_PAIRS", "FUSED_MAX_AVG_CHUNKS", "SEGMENTED_MAX_PAIRS", "SEGMENTED_MIN_AVG_CHUNKS",
           "SEGMENTED_FEW_PAIRS", "SEGMENTED_MIN_AVG_CHUNKS_FEW_PAIRS", "RECURRENT_MAX_AVG_TOKENS"]

HEAD_DIM = 128
CHUNK = 16
FLAG_FP32_COMPUTE = 1
FLAG_SPLIT = 2
FLAG_FUSED = 4
FLAG_RECURRENT = 8
FLAG_SCALAR_GATE = 16
FLAG_BF16_RESIDENT_STATE = 32
FLAG_SEGMENTED = 64
FUSED_MIN_PAIRS = 64
FUSED_MAX_AVG_CHUNKS = 8
SEGMENTED_MAX_PAIRS = 128
SEGMENTED_MIN_AVG_CHUNKS = 56
SEGMENTED_FEW_PAIRS = 80
SEGMENTED_MIN_AVG_CHUNKS_FEW_PAIRS = 40
RECURRENT_MAX_AVG_TOKENS = 4
_PATH_FLAGS = {"auto": 0, "split": FLAG_SPLIT, "fused": FLAG_FUSED, "recurrent": FLAG_RECURRENT,
               "segmented": FLAG_SEGMENTED}
DTYPE_BF16 = 0
DTYPE_FP32 = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libkda.so")
_lib = None


class KdaDesc(ctypes.Structure):
    """Mirror of kda_desc_t."""
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("num_seqs", ctypes.c_int64),
                ("num_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("io_dtype", ctypes.c_int32),
                ("state_dtype", ctypes.c_int32), ("scale", ctypes.c_float), ("flags", ctypes.c_uint32)]


class KdaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"kda_fwd failed with status {status}: {message}")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libkda.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it first (python -m kimi_delta_attention_k1_amd.build "
                           "or __graft_entry__.build()); there is no fallback implementation")
    lib = ctypes.CDLL(_LIB_PATH)
    vp = ctypes.c_void_p
    lib.kda_fwd_workspace_size.restype = ctypes.c_size_t
    lib.kda_fwd_workspace_size.argtypes = [ctypes.POINTER(KdaDesc)]
    for name in ("kda_fwd", "kda_fwd_prepare", "kda_fwd_recur", "kda_fwd_seg_pass", "kda_fwd_seg_finish"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, ctypes.POINTER(KdaDesc),
                       vp, ctypes.c_size_t, vp]
    lib.kda_fwd_noalloc.restype = ctypes.c_int
    lib.kda_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, ctypes.POINTER(KdaDesc), vp]
    lib.kda_status_str.restype = ctypes.c_char_p
    lib.kda_status_str.argtypes = [ctypes.c_int]
    lib.kda_version.restype = ctypes.c_int
    lib.kda_version.argtypes = []
    _lib = lib
    return lib


def make_desc(batch, seqlen, num_seqs, num_heads, io_dtype, state_dtype, scale, flags=0,
              head_dim=HEAD_DIM) -> KdaDesc:
    return KdaDesc(int(batch), int(seqlen), int(num_seqs), int(num_heads), int(head_dim), int(io_dtype),
                   int(state_dtype), float(scale), int(flags))


def status_str(status: int) -> str:
    return load_library().kda_status_str(int(status)).decode()


def _flags(fp32_compute, path):
    if path not in _PATH_FLAGS:
        raise ValueError(f"path must be one of {sorted(_PATH_FLAGS)}, not {path!r}")
    return (FLAG_FP32_COMPUTE if fp32_compute else 0) | _PATH_FLAGS[path]


def workspace_size(batch, seqlen, num_seqs, num_heads, io_dtype=DTYPE_BF16, state_dtype=DTYPE_FP32,
                   fp32_compute=False, path="auto", bf16_resident_state=False) -> int:
    flags = _flags(fp32_compute, path) | (FLAG_BF16_RESIDENT_STATE if bf16_resident_state else 0)
    d = make_desc(batch, seqlen, num_seqs, num_heads, io_dtype, state_dtype, HEAD_DIM ** -0.5, flags)
    return int(load_library().kda_fwd_workspace_size(ctypes.byref(d)))


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype == torch.float32:
        return DTYPE_FP32
    raise TypeError(f"unsupported dtype {t.dtype}: bf16 or fp32 expected")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


class Call:
    """A marshalled kda_fwd argument list; run() / prepare() / recur() / seg_pass() /
    seg_finish() enqueue it.

    Holds references to every tensor it points at, so the buffers stay alive
    while the object does.
    """

    def __init__(self, lib, args, keep, out, final_state):
        self._lib, self._args, self._keep = lib, args, keep
        self.out, self.final_state = out, final_state

    def _go(self, fn):
        st = fn(*self._args)
        if st != 0:
            raise KdaError(st, self._lib.kda_status_str(st).decode())

    def run(self):
        self._go(self._lib.kda_fwd)

    def prepare(self):
        self._go(self._lib.kda_fwd_prepare)

    def recur(self):
        self._go(self._lib.kda_fwd_recur)

    def seg_pass(self):
        self._go(self._lib.kda_fwd_seg_pass)

    def seg_finish(self):
        self._go(self._lib.kda_fwd_seg_finish)

    def run_noalloc(self):
        """The same call through kda_fwd_noalloc (the library's static scratch
        instead of the workspace)."""
        st = self._lib.kda_fwd_noalloc(*self._args[:11], self._args[13])
        if st != 0:
            raise KdaError(st, self._lib.kda_status_str(st).decode())


def fwd(q, k, v, g_raw, beta_raw, *, lower_bound: float = -5.0, scale: float | None = None,
        initial_state=None, output_final_state: bool = True, cu_seqlens=None, out=None, final_state=None,
        workspace=None, fp32_compute: bool = False, path: str = "auto", bf16_resident_state: bool = False,
        stream=None):
    """KDA forward through kda_fwd. Returns (out, final_state or None).

    All tensors must be contiguous and on the same GPU. `stream` is a
    torch.cuda.Stream (default: the current stream). `workspace` may be a
    preallocated uint8 tensor of at least workspace_size(...) bytes.
    bf16_resident_state runs the two-kernel path with the recurrence's state
    rounded to bf16 between chunk updates (KDA_FLAG_BF16_RESIDENT_STATE).
    """
    c = prepare_call(q, k, v, g_raw, beta_raw, lower_bound=lower_bound, scale=scale, initial_state=initial_state,
                     output_final_state=output_final_state, cu_seqlens=cu_seqlens, out=out,
                     final_state=final_state, workspace=workspace, fp32_compute=fp32_compute, path=path,
                     bf16_resident_state=bf16_resident_state, stream=stream)
    c.run()
    return c.out, c.final_state


def fwd_noalloc(q, k, v, g_raw, beta_raw, *, lower_bound: float = -5.0, scale: float | None = None,
                initial_state=None, output_final_state: bool = True, cu_seqlens=None, out=None, final_state=None,
                fp32_compute: bool = False, path: str = "auto", stream=None):
    """KDA forward through kda_fwd_noalloc: no workspace; the library's static
    scratch on the device serves as one. `path` is "auto", "fused" or
    "recurrent" (the paths with a small workspace). out and final_state are
    allocated here when not given; pass them to keep the call free of
    allocations."""
    c = prepare_call(q, k, v, g_raw, beta_raw, lower_bound=lower_bound, scale=scale, initial_state=initial_state,
                     output_final_state=output_final_state, cu_seqlens=cu_seqlens, out=out,
                     final_state=final_state, fp32_compute=fp32_compute, path=path, stream=stream,
                     no_workspace=True)
    c.run_noalloc()
    return c.out, c.final_state


def prepare_call(q, k, v, g_raw, beta_raw, *, lower_bound: float = -5.0, scale: float | None = None,
                 initial_state=None, output_final_state: bool = True, cu_seqlens=None, out=None,
                 final_state=None, workspace=None, fp32_compute: bool = False, path: str = "auto",
                 bf16_resident_state: bool = False, stream=None, no_workspace: bool = False) -> Call:
    """Check and marshal fwd's arguments once (allocating out, final_state and
    the workspace when not given) without launching anything. no_workspace: for
    kda_fwd_noalloc, which takes none (the call then passes NULL and 0)."""
    import torch
    lib = load_library()
    tensors = (q, k, v, g_raw, beta_raw)
    for t in tensors:
        if not t.is_contiguous():
            raise ValueError("kda.fwd needs contiguous inputs")
    if q.dim() == 4:
        B, T, H, D = q.shape
    elif q.dim() == 3:
        B, (T, H, D) = 1, q.shape
    else:
        raise ValueError("q must be [B,T,H,128] or [T_tot,H,128]")
    for t in (k, v):
        if t.shape != q.shape:
            raise ValueError("q, k and v must have the same shape")
    if tuple(beta_raw.shape) != tuple(q.shape[:-1]):
        raise ValueError("beta_raw must have the shape of q without the last dimension")
    if tuple(g_raw.shape) == tuple(q.shape):
        scalar_gate = False
    elif tuple(g_raw.shape) == tuple(q.shape[:-1]):
        scalar_gate = True  # one gate per token and head
    else:
        raise ValueError("g_raw must have the shape of q, or of beta_raw for a scalar per-head gate")
    io = _dtype_code(q)
    if any(_dtype_code(t) != io for t in tensors):
        raise TypeError("q, k, v, g_raw and beta_raw must share one dtype")
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or not cu_seqlens.is_contiguous():
            raise ValueError("cu_seqlens must be a contiguous 1-D int32 tensor")
        N = cu_seqlens.shape[0] - 1
        seqlen = B * T
    else:
        N = B
        seqlen = T
    if initial_state is not None and final_state is not None and initial_state.dtype != final_state.dtype:
        raise TypeError("initial_state and final_state must have the same dtype")
    st_t = initial_state if initial_state is not None else final_state
    st_code = _dtype_code(st_t) if st_t is not None else DTYPE_FP32
    for s in (initial_state, final_state):
        if s is not None and (tuple(s.shape) != (N, H, D, D) or not s.is_contiguous()):
            raise ValueError(f"states must be contiguous [{N}, {H}, {D}, {D}]")
    if out is None:
        out = torch.empty_like(v)
    if final_state is None and output_final_state:
        final_state = torch.empty((N, H, D, D), dtype=st_t.dtype if st_t is not None else torch.float32,
                                  device=q.device)
    if scale is None:
        scale = D ** -0.5
    flags = _flags(fp32_compute, path) | (FLAG_SCALAR_GATE if scalar_gate else 0) | \
        (FLAG_BF16_RESIDENT_STATE if bf16_resident_state else 0)
    desc = make_desc(B, seqlen, N, H, io, st_code, scale, flags, head_dim=D)
    need = 0 if no_workspace else int(lib.kda_fwd_workspace_size(ctypes.byref(desc)))
    if no_workspace:
        if workspace is not None:
            raise ValueError("no_workspace excludes a workspace")
    elif workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    elif workspace.numel() < need:
        raise ValueError(f"workspace too small: {workspace.numel()} < {need} bytes")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(g_raw), _ptr(beta_raw), _ptr(cu_seqlens), _ptr(initial_state),
            _ptr(out), _ptr(final_state), ctypes.c_float(lower_bound), ctypes.byref(desc), _ptr(workspace),
            ctypes.c_size_t(0 if workspace is None else workspace.numel()), ctypes.c_void_p(stream.cuda_stream))
    keep = (q, k, v, g_raw, beta_raw, cu_seqlens, initial_state, out, final_state, workspace, desc, stream)
    return Call(lib, args, keep, out, final_state)


def seqlens_flag(workspace) -> int:
    """1 if the cu_seqlens of the last call on this workspace were well formed
    (reads the workspace's first int32; synchronises on it)."""
    return int(workspace[:4].view(dtype=__import__("torch").int32).item())
