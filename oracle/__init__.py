"""fp64 CPU oracle for Kimi Delta Attention -- TEST INFRASTRUCTURE.

Only the test-suite, the package smoke check and the benchmark's CPU-baseline
leg may import this package. The GPU library never does, and this package
imports nothing from it. What the oracle computes, and the passages it
follows, are stated at the top of ``kda_oracle.c``.

Inputs are numpy float32 arrays holding the exact values the GPU receives
(bf16 values are exact in float32); outputs are float64.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile kda_oracle.c with gcc (fp64, OpenMP, strict IEEE)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared",
                               "-std=c99", "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _bind(path):
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i32, f64 = ctypes.c_int32, ctypes.c_double
    lib.kda_oracle_prefill.argtypes = [P, P, P, P, P, P, i32, i32, i32,
                                       i32, f64, P, P, P, i32]
    lib.kda_oracle_prefill.restype = ctypes.c_int
    lib.kda_oracle_decode.argtypes = [P, P, P, P, P, P, P, i32, i32, i32,
                                      i32, i32, f64, P, i32]
    lib.kda_oracle_decode.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = _bind(_LIB)
    return _lib


def load_variant(path: str):
    """The same Python interface over another build of the oracle source
    (used by the mutation test, which compiles deliberately broken copies)."""
    import functools
    import types
    lib = _bind(path)
    return types.SimpleNamespace(prefill=functools.partial(prefill, _lib=lib),
                                 decode=functools.partial(decode, _lib=lib))


def _f32(x):
    return np.ascontiguousarray(x, dtype=np.float32)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def prefill(q, k, v, log_alpha, beta, cu_seqlens, scale: float = 1.0,
            initial_state=None, nthreads: int = 0, _lib=None
            ) -> Tuple[np.ndarray, np.ndarray]:
    """Token-by-token fp64 KDA over packed sequences.

    q, k, log_alpha: [T, H, K]; v: [T, H, V]; beta: [T, H];
    cu_seqlens: [N+1]; initial_state: [N, H, K, V] or None.
    Returns (o [T, H, V], final_state [N, H, K, V]) in float64.
    """
    q, k, v, g, b = (_f32(x) for x in (q, k, v, log_alpha, beta))
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    T, H, K = q.shape
    V = v.shape[2]
    N = cu.shape[0] - 1
    if int(cu[-1]) != T or k.shape != q.shape or g.shape != q.shape \
            or v.shape[:2] != (T, H) or b.shape != (T, H):
        raise ValueError("inconsistent shapes")
    s0 = None if initial_state is None else _f32(initial_state)
    if s0 is not None and s0.shape != (N, H, K, V):
        raise ValueError("initial_state shape")
    o = np.zeros((T, H, V), dtype=np.float64)
    sf = np.zeros((N, H, K, V), dtype=np.float64)
    rc = (_lib or _load()).kda_oracle_prefill(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(b), _ptr(cu), N, H, K, V,
        float(scale), _ptr(s0), _ptr(o), _ptr(sf), int(nthreads))
    if rc != 0:
        raise ValueError("kda_oracle_prefill rejected its arguments")
    return o, sf


def decode(q, k, v, log_alpha, beta, state: np.ndarray,
           slot_idx: Optional[np.ndarray] = None, scale: float = 1.0,
           nthreads: int = 0, _lib=None) -> np.ndarray:
    """One fp64 decode step; `state` [slots, H, K, V] float64 is updated in place.

    q, k, log_alpha: [B, H, K]; v: [B, H, V]; beta: [B, H]. Returns o [B, H, V].
    """
    q, k, v, g, b = (_f32(x) for x in (q, k, v, log_alpha, beta))
    if state.dtype != np.float64 or not state.flags.c_contiguous:
        raise ValueError("state must be a C-contiguous float64 array")
    B, H, K = q.shape
    V = v.shape[2]
    slots = state.shape[0]
    if state.shape != (slots, H, K, V):
        raise ValueError("state shape")
    si = None if slot_idx is None else np.ascontiguousarray(slot_idx, dtype=np.int32)
    o = np.zeros((B, H, V), dtype=np.float64)
    rc = (_lib or _load()).kda_oracle_decode(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(b), _ptr(state), _ptr(si),
        B, H, K, V, slots, float(scale), _ptr(o), int(nthreads))
    if rc != 0:
        raise ValueError("kda_oracle_decode rejected its arguments")
    return o
