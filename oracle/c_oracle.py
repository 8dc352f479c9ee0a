"""ctypes wrapper of the fp64 C oracle (TEST INFRASTRUCTURE ONLY).

Same recurrence and layouts as ``oracle.reference.recurrent`` (and, for the
gradient, as ``oracle.backward``); the C code
(``gdn2_oracle.c``) follows the burn-gdn2 README's per-token formula
("Architecture" section) step by step in double precision and splits the work
over (batch, head, value-column block) with OpenMP.  Inputs are widened to
float32 (exact for bf16 and fp32 inputs) before the call.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SRC_PATH = os.path.join(_HERE, "gdn2_oracle.c")

_lib = None


def build(force: bool = True) -> str:
    """Compile ``gdn2_oracle.c`` into ``liboracle.so`` (gcc, -O2 -fopenmp)."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared",
                               "-o", tmp, SRC_PATH, "-lm"])
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build(force=True)
        lib = ctypes.CDLL(LIB_PATH)
        f = lib.gdn2_oracle_f64
        f.restype = ctypes.c_int
        i64, vp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        f.argtypes = [i64] * 5 + [vp] * 9 + [ci, i64, ci]
        lib.gdn2_oracle_max_threads.restype = ctypes.c_int
        fb = lib.gdn2_oracle_bwd_f64
        fb.restype = ctypes.c_int
        fb.argtypes = [i64] * 5 + [vp] * 16 + [ci, ci]
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().gdn2_oracle_max_threads())


def _f32(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def recurrent(q, k, v, alpha, b, w, S0=None, nthreads: int = 0, col_block: int = 16, flags: int = 0):
    """fp64 recurrence; returns (o, S_T) as float64 arrays.  ``flags``: the prologue options
    (1 gate logits -> sigmoid, 2 with 1: b = 2 sigmoid(b), 4 q/k L2 norm), as in
    ``oracle.reference.prologue``."""
    q, k, v, alpha, b, w = map(_f32, (q, k, v, alpha, b, w))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    for x, last in ((k, dk), (alpha, dk), (b, dk), (v, dv), (w, dv)):
        if x.shape != (B, T, H, last):
            raise ValueError("oracle: inconsistent input shapes")
    S0a = None if S0 is None else _f32(S0)
    if S0a is not None and S0a.shape != (B, H, dk, dv):
        raise ValueError("oracle: S0 shape")
    o = np.zeros((B, T, H, dv), dtype=np.float64)
    S = np.zeros((B, H, dk, dv), dtype=np.float64)
    p = lambda a: None if a is None else a.ctypes.data
    rc = _load().gdn2_oracle_f64(B, T, H, dk, dv, p(q), p(k), p(v), p(alpha), p(b), p(w),
                                 p(S0a), p(o), p(S), int(nthreads), int(col_block), int(flags))
    if rc != 0:
        raise RuntimeError("oracle: bad sizes")
    return o, S


def recurrent_bwd(q, k, v, alpha, b, w, S0, dO, dS_T=None, flags: int = 0, nthreads: int = 0):
    """fp64 gradient of sum(dO * o) + sum(dS_T * S_T) with respect to q, k, v, alpha, b, w
    and S0 (the C routine ``gdn2_oracle_bwd_f64``; the same quantity as
    ``oracle.backward.recurrent_bwd`` / ``full_bwd`` for one value head per query/key head).
    Returns a dict dq, dk, dv, dalpha, db, dw, dS0 of float64 arrays."""
    q, k, v, alpha, b, w, dO = map(_f32, (q, k, v, alpha, b, w, dO))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    for x, last in ((k, dk), (alpha, dk), (b, dk), (v, dv), (w, dv), (dO, dv)):
        if x.shape != (B, T, H, last):
            raise ValueError("oracle: inconsistent input shapes")
    S0a = None if S0 is None else _f32(S0)
    dSa = None if dS_T is None else _f32(dS_T)
    for x in (S0a, dSa):
        if x is not None and x.shape != (B, H, dk, dv):
            raise ValueError("oracle: state shape")
    out = {n: np.zeros(x.shape, dtype=np.float64) for n, x in
           (("dq", q), ("dk", k), ("dv", v), ("dalpha", alpha), ("db", b), ("dw", w))}
    out["dS0"] = np.zeros((B, H, dk, dv), dtype=np.float64)
    p = lambda a: None if a is None else a.ctypes.data
    rc = _load().gdn2_oracle_bwd_f64(B, T, H, dk, dv, p(q), p(k), p(v), p(alpha), p(b), p(w), p(S0a), p(dO),
                                     p(dSa), p(out["dq"]), p(out["dk"]), p(out["dv"]), p(out["dalpha"]),
                                     p(out["db"]), p(out["dw"]), p(out["dS0"]), int(nthreads), int(flags))
    if rc != 0:
        raise RuntimeError("oracle: bad sizes or out of memory")
    return out
