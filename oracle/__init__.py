"""CPU oracle for the Comba mixer. TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import, call or link anything in this package. The device
library (``bilinear_rnn_amd``) never imports it, and this package never
imports the device library.

Two implementations of the same definition are provided:
- :mod:`oracle.reference` — numpy fp64, token by token, plus the fp64
  chunk-wise form used to check intermediates;
- ``comba_oracle.c`` — plain C fp64 with OpenMP over (sequence, head, value
  rows), for large cases and CPU timing, loaded here through ctypes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

from .reference import (comba_backward, comba_forward, comba_forward_chunked, expand_shared_qk,  # noqa: F401
                        fused_inputs, rel_l2, row_rel_err)

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "comba_oracle.c")
# COMBA_ORACLE_LIBRARY names another build of comba_oracle.c (the sanitizer build of
# the CPU checks); by default the one build_c() writes here.
_DEFAULT_LIB = os.path.join(_HERE, "libcomba_oracle.so")
_LIB = os.environ.get("COMBA_ORACLE_LIBRARY") or _DEFAULT_LIB
_lib = None


def build_c(force: bool = True) -> str:
    """Compile the C oracle with gcc (-O2, OpenMP)."""
    if force or not os.path.exists(_DEFAULT_LIB):
        tmp = _DEFAULT_LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11",
                               "-Wall", "-Wextra", "-o", tmp, _SRC])
        os.replace(tmp, _DEFAULT_LIB)
    return _DEFAULT_LIB


def build_c_sanitized(path: str) -> str:
    """The same source under gcc's address and undefined-behaviour sanitizers
    (any undefined behaviour aborts), for the CPU checks. Load it through
    COMBA_ORACLE_LIBRARY with gcc's libasan and libubsan preloaded."""
    subprocess.check_call(["gcc", "-O1", "-g", "-fopenmp", "-shared", "-fPIC", "-std=c11", "-Wall", "-Wextra",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                           "-fno-omit-frame-pointer", "-o", path, _SRC])
    return path


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build_c(force=True)
        lib = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        i32p = ctypes.POINTER(ctypes.c_int32)
        lib.comba_oracle_forward.argtypes = [dp, dp, dp, dp, dp, dp, dp, i32p, ctypes.c_int32,
                                             ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                             ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                             dp, dp, ctypes.c_int32]
        lib.comba_oracle_forward.restype = ctypes.c_int
        lib.comba_oracle_backward.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp, dp, i32p, ctypes.c_int32,
                                              ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                              ctypes.c_int32, ctypes.c_int32,
                                              dp, dp, dp, dp, dp, dp, dp, ctypes.c_int32]
        lib.comba_oracle_backward.restype = ctypes.c_int
        lib.comba_oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().comba_oracle_max_threads())


def comba_forward_c(q, k, v, alpha, beta, d, s0=None, cu_seqlens=None,
                    nthreads: int = 0, rows_per_task: int = 16):
    """Same definition as :func:`oracle.reference.comba_forward`, in C fp64."""
    lib = _load()

    def f64(x):
        return np.ascontiguousarray(x, dtype=np.float64)

    q, k, v, alpha, beta, d = map(f64, (q, k, v, alpha, beta, d))
    B, T, H, K = q.shape
    V = v.shape[-1]
    cu = None if cu_seqlens is None else np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    N = B if cu is None else len(cu) - 1
    s0a = None if s0 is None else f64(s0)
    o = np.zeros((B, T, H, V), dtype=np.float64)
    sf = np.zeros((N, H, V, K), dtype=np.float64)
    dp = ctypes.POINTER(ctypes.c_double)

    def ptr(a):
        return None if a is None else a.ctypes.data_as(dp)

    rc = lib.comba_oracle_forward(ptr(q), ptr(k), ptr(v), ptr(alpha), ptr(beta), ptr(d), ptr(s0a),
                                  None if cu is None else cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                  N, B, T, H, K, V, rows_per_task, ptr(o), ptr(sf), nthreads)
    if rc != 0:
        raise ValueError("comba_oracle_forward rejected its arguments")
    return o, sf


def comba_backward_c(q, k, v, alpha, beta, d, do, s0=None, dsf=None, cu_seqlens=None, nthreads: int = 0):
    """Same definition as :func:`oracle.reference.comba_backward`, in C fp64
    (one OpenMP task per sequence and head). Returns the same dict of float64
    arrays: dq, dk, dv, dalpha, dbeta, dd (summed over the sequences in order)
    and ds0."""
    lib = _load()

    def f64(x):
        return np.ascontiguousarray(x, dtype=np.float64)

    q, k, v, alpha, beta, d, do = map(f64, (q, k, v, alpha, beta, d, do))
    B, T, H, K = q.shape
    V = v.shape[-1]
    cu = None if cu_seqlens is None else np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    N = B if cu is None else len(cu) - 1
    s0a = None if s0 is None else f64(s0)
    dsfa = None if dsf is None else f64(dsf)
    g = {"dq": np.zeros((B, T, H, K)), "dk": np.zeros((B, T, H, K)), "dv": np.zeros((B, T, H, V)),
         "dalpha": np.zeros((B, T, H)), "dbeta": np.zeros((B, T, H)), "ds0": np.zeros((N, H, V, K))}
    dd_part = np.zeros((N, H))
    dp = ctypes.POINTER(ctypes.c_double)

    def ptr(a):
        return None if a is None else a.ctypes.data_as(dp)

    rc = lib.comba_oracle_backward(ptr(q), ptr(k), ptr(v), ptr(alpha), ptr(beta), ptr(d), ptr(do), ptr(s0a),
                                   ptr(dsfa),
                                   None if cu is None else cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                   N, B, T, H, K, V, ptr(g["dq"]), ptr(g["dk"]), ptr(g["dv"]), ptr(g["dalpha"]),
                                   ptr(g["dbeta"]), ptr(dd_part), ptr(g["ds0"]), nthreads)
    if rc != 0:
        raise ValueError("comba_oracle_backward rejected its arguments")
    g["dd"] = np.zeros((H,))
    for n in range(N):
        g["dd"] += dd_part[n]
    return g
