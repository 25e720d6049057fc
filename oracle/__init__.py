"""fp64 CPU oracle for the KDA forward pass -- TEST INFRASTRUCTURE.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package. The GPU library never imports, links or calls it.

Two independent implementations live here:
  * kda_oracle.c (loaded through ctypes): the token-by-token recurrence of the
    Doubleword page "You Could Have Come Up with Kimi Delta Attention",
    section 4 (boxed KDA equations), with the FlashKDA activations in front.
  * chunked.py: the chunkwise derivation of the same page, section 6.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import chunked  # noqa: F401  (re-exported)

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libkda_oracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from .build import build
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.kda_oracle_sigmoid.restype = ctypes.c_double
    lib.kda_oracle_sigmoid.argtypes = [ctypes.c_double]
    lib.kda_oracle_core.restype = ctypes.c_int
    lib.kda_oracle_core.argtypes = [ctypes.c_int64] * 3 + [_dp] * 5 + [ctypes.c_double, _dp, _dp]
    lib.kda_oracle_fwd.restype = ctypes.c_int
    lib.kda_oracle_fwd.argtypes = ([ctypes.c_int64, _i64p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64]
                                   + [_dp] * 6 + [ctypes.c_double] * 3 + [_dp, _dp, ctypes.c_int])
    lib.kda_oracle_max_threads.restype = ctypes.c_int
    lib.kda_oracle_max_threads.argtypes = []
    _lib = lib
    return lib


def _f64(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_dp)


def sigmoid(x: float) -> float:
    """The C oracle's sigmoid at one point."""
    return float(_load().kda_oracle_sigmoid(float(x)))


def core(q, k, v, alpha, beta, S0, scale):
    """Token recurrence for one (sequence, head) on pre-activated inputs.

    q, k, alpha: [T,K]; v: [T,V]; beta: [T]; S0: [V,K]. Keys are used as given.
    Returns (o [T,V], S_T [V,K]).
    """
    q, k, v, alpha, beta = map(_f64, (q, k, v, alpha, beta))
    T, K = k.shape
    V = v.shape[1]
    S = _f64(S0).copy()
    o = np.zeros((T, V))
    rc = _load().kda_oracle_core(T, K, V, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                 float(scale), _ptr(S), _ptr(o))
    if rc != 0:
        raise ValueError("kda_oracle_core rejected its arguments")
    return o, S


def token_forward(q, k, v, g_raw, beta_raw, seq_offsets, initial_state=None,
                  lower_bound=-5.0, scale=None, eps=1e-6, threads=0, want_state=True):
    """Token-by-token fp64 forward on the packed layout.

    q, k, g_raw: [T_tot,H,K]; v: [T_tot,H,V]; beta_raw: [T_tot,H];
    seq_offsets: N+1 token offsets; initial_state: [N,H,V,K] or None.
    Returns (o [T_tot,H,V] fp64, final_state [N,H,V,K] fp64 or None).
    """
    q, k, v, g_raw, beta_raw = map(_f64, (q, k, v, g_raw, beta_raw))
    T_tot, H, K = k.shape
    V = v.shape[2]
    offs = np.ascontiguousarray(np.asarray(seq_offsets, dtype=np.int64))
    N = offs.shape[0] - 1
    if scale is None:
        scale = K ** -0.5
    S0 = None if initial_state is None else _f64(initial_state)
    out = np.zeros((T_tot, H, V))
    fin = np.zeros((N, H, V, K)) if want_state else None
    rc = _load().kda_oracle_fwd(N, offs.ctypes.data_as(_i64p), H, K, V,
                                _ptr(q), _ptr(k), _ptr(v), _ptr(g_raw), _ptr(beta_raw), _ptr(S0),
                                float(lower_bound), float(scale), float(eps),
                                _ptr(out), _ptr(fin), int(threads))
    if rc != 0:
        raise ValueError("kda_oracle_fwd rejected its arguments")
    return out, fin


def max_threads() -> int:
    return int(_load().kda_oracle_max_threads())
