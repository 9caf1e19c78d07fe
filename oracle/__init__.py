"""CPU fp64 oracle for the deterministic attention backward.

TEST INFRASTRUCTURE ONLY.  Only the tests, `__graft_entry__.smoke()` and the
benchmark's `cpu_baseline` leg may import this package; the product library
(`tile_scheduling_attn_amd`) never does, and shares no code with it.

* `oracle.c`  - attention forward and backward in double precision, written
  out from the definition (see the header of that file for the formulas and
  the passage of the DASH paper they follow).  Built with gcc into
  `liboracle.so` by `build()`.
* `dag.py`    - the schedules and the DAG critical-path model in plain Python.

Parity status: every function here is pinned by CPU tests against finite
differences, closed forms, identities and brute force (tests/test_oracle*.py).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (-O3 -march=native -fopenmp) into
    liboracle.so next to it.  `-ffp-contract=off` keeps every product and sum
    as written (no fused multiply-add rounding changes)."""
    if not force and os.path.exists(_LIB_PATH) and \
            os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    tmp = _LIB_PATH + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O3", "-march=native", "-ffp-contract=off", "-fopenmp", "-fPIC",
           "-shared", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        i, d = ctypes.c_int, ctypes.c_double
        lib.oracle_attn_fwd.argtypes = [i, i, i, d, i, dp, dp, dp, dp, dp]
        lib.oracle_attn_bwd.argtypes = [i, i, i, d, i, dp, dp, dp, dp, dp, dp, dp, dp, dp, dp]
        lib.oracle_attn_delta.argtypes = [i, i, i, dp, dp, dp]
        lib.oracle_num_threads.restype = i
        _lib = lib
    return _lib


def _as_f64(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _heads(x):
    """View [..., s, d] as [H, s, d]."""
    x = _as_f64(x)
    return x.reshape((-1,) + x.shape[-2:])


def attn_fwd(q, k, v, causal: bool, scale: float | None = None):
    """Forward pass in fp64: returns (O, lse) with shapes [..., s, d], [..., s]."""
    lib = _load()
    shape = np.shape(q)
    qh, kh, vh = _heads(q), _heads(k), _heads(v)
    H, s, d = qh.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    o = np.empty_like(qh)
    lse = np.empty((H, s), dtype=np.float64)
    lib.oracle_attn_fwd(H, s, d, float(scale), int(bool(causal)), _ptr(qh), _ptr(kh), _ptr(vh),
                        _ptr(o), _ptr(lse))
    return o.reshape(shape), lse.reshape(shape[:-1])


def attn_bwd(q, k, v, o, do, lse, causal: bool, scale: float | None = None):
    """Backward pass in fp64 from the given O and lse ("given" mode).
    Returns (dq, dk, dv, D) with D = rowsum(dO * O)."""
    lib = _load()
    shape = np.shape(q)
    qh, kh, vh, oh, doh = (_heads(t) for t in (q, k, v, o, do))
    H, s, d = qh.shape
    lseh = _as_f64(lse).reshape(H, s)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    dq, dk, dv = (np.empty_like(qh) for _ in range(3))
    D = np.empty((H, s), dtype=np.float64)
    lib.oracle_attn_bwd(H, s, d, float(scale), int(bool(causal)), _ptr(qh), _ptr(kh), _ptr(vh),
                        _ptr(oh), _ptr(doh), _ptr(lseh), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(D))
    return dq.reshape(shape), dk.reshape(shape), dv.reshape(shape), D.reshape(shape[:-1])


def attn_fwd_bwd(q, k, v, do, causal: bool, scale: float | None = None):
    """"Truth" mode: fp64 forward from Q, K, V, then the fp64 backward.
    Returns dict with o, lse, dq, dk, dv, D."""
    o, lse = attn_fwd(q, k, v, causal, scale)
    dq, dk, dv, D = attn_bwd(q, k, v, o, do, lse, causal, scale)
    return {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv, "D": D}


def delta(o, do):
    """D = rowsum(dO * O) in fp64, shape [..., s]."""
    lib = _load()
    shape = np.shape(o)
    oh, doh = _heads(o), _heads(do)
    H, s, d = oh.shape
    D = np.empty((H, s), dtype=np.float64)
    lib.oracle_attn_delta(H, s, d, _ptr(oh), _ptr(doh), _ptr(D))
    return D.reshape(shape[:-1])


def num_threads() -> int:
    return _load().oracle_num_threads()
