"""Build and call the C fp64 twin of the oracle (gdn_oracle.c).

TEST INFRASTRUCTURE: used by the test suite, the smoke check and the benchmark's
CPU baseline only. Inputs are widened to float64 exactly before the call.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from .recurrence import _f64

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gdn_oracle.c")
LIB = os.path.join(HERE, "libgdn_oracle.so")

_lib = None


def build(verbose: bool = False) -> str:
    """Compile gdn_oracle.c with gcc (-O3, OpenMP, no fast-math) into libgdn_oracle.so."""
    cmd = ["gcc", "-O3", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-Wall", "-Wextra",
           SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        lib = ctypes.CDLL(LIB)
        P = ctypes.c_void_p
        lib.gdn_oracle_forward.argtypes = [P] * 9 + [ctypes.c_int] * 4 + [P, ctypes.c_int]
        lib.gdn_oracle_forward.restype = ctypes.c_int
        lib.gdn_oracle_decode.argtypes = [P] * 7 + [ctypes.c_long, ctypes.c_int, ctypes.c_int]
        lib.gdn_oracle_decode.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def prepare_forward(q, k, v, g, beta, h0=None, cu_seqlens=None):
    """Widen inputs to contiguous float64 arrays once (kept out of any timing)."""
    q, k, v, g, beta, h0 = (_f64(x) for x in (q, k, v, g, beta, h0))
    B, T, H, dk = q.shape
    if cu_seqlens is None:
        seg = np.arange(B + 1, dtype=np.int64) * T
    else:
        if B != 1:
            raise ValueError("packed sequences need B == 1")
        seg = np.asarray(_f64(cu_seqlens)).astype(np.int64)
    arrs = [np.ascontiguousarray(x) for x in (q, k, v, g, beta)]
    return dict(q=arrs[0], k=arrs[1], v=arrs[2], g=arrs[3], beta=arrs[4],
                h0=None if h0 is None else np.ascontiguousarray(h0), seg=seg,
                B=B, T=T, H=H, dk=dk, dv=v.shape[-1])


def forward_prepared(p, heads=None):
    """Run the C twin on prepared inputs. Returns (o, hT, threads_used)."""
    lib = load()
    N = len(p["seg"]) - 1
    H, dk, dv = p["H"], p["dk"], p["dv"]
    o = np.full((p["B"] * p["T"], H, dv), np.nan)
    hT = np.full((N, H, dv, dk), np.nan)
    hs = None if heads is None else np.ascontiguousarray(np.asarray(heads, dtype=np.int32))
    used = lib.gdn_oracle_forward(_ptr(p["q"]), _ptr(p["k"]), _ptr(p["v"]), _ptr(p["g"]),
                                  _ptr(p["beta"]), _ptr(p["h0"]), _ptr(o), _ptr(hT),
                                  _ptr(p["seg"]), N, H, dk, dv, _ptr(hs),
                                  0 if hs is None else len(hs))
    return o.reshape(p["B"], p["T"], H, dv), hT, used


def forward(q, k, v, g, beta, h0=None, cu_seqlens=None, heads=None):
    """Same interface as recurrence.forward; returns (o, hT) in float64."""
    o, hT, _ = forward_prepared(prepare_forward(q, k, v, g, beta, h0, cu_seqlens), heads)
    return o, hT


def decode(state, q, k, v, g, beta):
    """Same interface as recurrence.decode; returns (new_state, o) in float64."""
    lib = load()
    state, q, k, v, g, beta = (np.ascontiguousarray(_f64(x)) for x in (state, q, k, v, g, beta))
    N, H, dv, dk = state.shape
    S = state.copy()
    o = np.zeros((N, H, dv))
    lib.gdn_oracle_decode(_ptr(S), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(o),
                          N * H, dk, dv)
    return S, o
