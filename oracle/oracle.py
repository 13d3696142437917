"""Python front end of the CPU oracle (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module.  It compiles ``gdn_oracle.c`` with gcc
(no HIP, no code shared with the GPU library) and wraps it with ctypes.

Every function takes float64-convertible numpy arrays in the layouts listed in
``gdn_oracle.c`` and returns float64 results.  See that file for what is
computed and which passage of the SpecLA review pages it follows.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gdn_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

_lock = threading.Lock()
_lib = None


class OracleError(RuntimeError):
    pass


def build(force: bool = True) -> str:
    """Compile the oracle into ``oracle/liboracle.so`` with gcc and OpenMP."""
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build(force=False)
            lib = ctypes.CDLL(LIB)
            P = ctypes.c_void_p
            I = ctypes.c_int
            lib.gdno_set_threads.argtypes = [I]
            lib.gdno_set_threads.restype = I
            lib.gdno_masks.argtypes = [I, I, P, P, P]
            lib.gdno_masks.restype = I
            lib.gdno_tree_verify.argtypes = [I, I, I, I, I, P, P, P, P, P, P, P,
                                             ctypes.c_double, P, P, P]
            lib.gdno_tree_verify.restype = I
            lib.gdno_commit.argtypes = [I, I, I, I, I, P, P, P, P, P, P, P, P, P, P]
            lib.gdno_commit.restype = I
            lib.gdno_sequential_decode.argtypes = [I, I, I, I, I, P, P, P, P, P, P,
                                                   ctypes.c_double, P, P]
            lib.gdno_sequential_decode.restype = I
            _lib = lib
    return _lib


def _f64(x):
    return np.ascontiguousarray(x, dtype=np.float64)


def _i32(x):
    return np.ascontiguousarray(x, dtype=np.int32)


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, what):
    if rc != 0:
        raise OracleError(f"{what} returned {rc}")


def set_threads(n: int) -> int:
    """Set the OpenMP thread count (n <= 0 keeps it); returns the count in use."""
    return int(_load().gdno_set_threads(int(n)))


def masks(parents):
    """Ancestor-or-self bitmasks (uint64 [B][N]) and depths (int32 [B][N])."""
    par = _i32(parents)
    B, N = par.shape
    m = np.zeros((B, N), dtype=np.uint64)
    d = np.zeros((B, N), dtype=np.int32)
    _check(_load().gdno_masks(B, N, _ptr(par), _ptr(m), _ptr(d)), "gdno_masks")
    return m, d


def tree_verify(S0, parents, q, k, v, beta, g, scale=1.0):
    """Outputs [B][N][H][dv], u' [B][H][N][dv] and G [B][H][N] by per-path replay."""
    S0, q, k, v, beta, g = map(_f64, (S0, q, k, v, beta, g))
    par = _i32(parents)
    B, H, dv, dk = S0.shape
    N = par.shape[1]
    assert q.shape == (B, N, H, dk) and k.shape == (B, N, H, dk) and v.shape == (B, N, H, dv)
    assert beta.shape == (B, N, H) and g.shape == (B, N, H)
    out = np.zeros((B, N, H, dv))
    up = np.zeros((B, H, N, dv))
    G = np.zeros((B, H, N))
    rc = _load().gdno_tree_verify(B, N, H, dk, dv, _ptr(S0), _ptr(par), _ptr(q), _ptr(k),
                                  _ptr(v), _ptr(beta), _ptr(g), float(scale), _ptr(out),
                                  _ptr(up), _ptr(G))
    _check(rc, "gdno_tree_verify")
    return out, up, G


def commit(S0, parents, k, v, beta, g, last_accepted):
    """State after the accepted path, root-first path lists and their lengths."""
    S0, k, v, beta, g = map(_f64, (S0, k, v, beta, g))
    par = _i32(parents)
    last = _i32(last_accepted)
    B, H, dv, dk = S0.shape
    N = par.shape[1]
    Snew = np.zeros_like(S0)
    path = np.zeros((B, N), dtype=np.int32)
    plen = np.zeros(B, dtype=np.int32)
    rc = _load().gdno_commit(B, N, H, dk, dv, _ptr(S0), _ptr(par), _ptr(k), _ptr(v),
                             _ptr(beta), _ptr(g), _ptr(last), _ptr(Snew), _ptr(path),
                             _ptr(plen))
    _check(rc, "gdno_commit")
    return Snew, path, plen


def sequential_decode(S0, q, k, v, beta, g, scale=1.0):
    """Token-by-token decode of a linear sequence: outputs and final state."""
    S0, q, k, v, beta, g = map(_f64, (S0, q, k, v, beta, g))
    B, H, dv, dk = S0.shape
    N = q.shape[1]
    out = np.zeros((B, N, H, dv))
    Sf = np.zeros_like(S0)
    rc = _load().gdno_sequential_decode(B, N, H, dk, dv, _ptr(S0), _ptr(q), _ptr(k), _ptr(v),
                                        _ptr(beta), _ptr(g), float(scale), _ptr(out), _ptr(Sf))
    _check(rc, "gdno_sequential_decode")
    return out, Sf


def draft_verify(d):
    """tree_verify on a workloads.Draft (bf16 inputs widened exactly)."""
    return tree_verify(d.S0, d.parents, d.q64(), d.k64(), d.v64(), d.beta, d.g, d.scale)


def draft_commit(d, last_accepted=None):
    """commit on a workloads.Draft; ``last_accepted`` overrides the draft's own."""
    last = d.last_accepted if last_accepted is None else last_accepted
    return commit(d.S0, d.parents, d.k64(), d.v64(), d.beta, d.g, last)
