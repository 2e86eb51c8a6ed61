"""CPU oracle for the ragged BF16 grouped GEMM -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never imports,
links or calls it; the two share no code.

The arithmetic lives in ``oracle.c`` (plain C99, binary64 accumulation in
increasing reduction index, one rounding at the end).  This module only
marshals numpy arrays into it:

* ``fwd / dgrad / wgrad`` return ``(value, q)`` as float64 arrays: the
  unrounded result and ``q = sqrt(sum of squared products)`` per element.
  With ``idx`` (flat row-major output indices) only those elements are
  computed, which is how parity is checked at sizes too large for a full CPU
  product.
* ``round_f32 / round_bf16`` round a float64 array once (ties to even);
  ``round_bf16`` returns the BF16 bit patterns as uint16.
* ``router_exact / router_bf16x3``: the FP32 router GEMM, exactly and as the
  BF16x3 emulation.

Every function here is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_pins.py`` (integer-exact library matmuls, closed forms,
finite differences, rounding special cases).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with the host C compiler."""
    from . import build_oracle

    return build_oracle.build(force=force)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        build(force=False)
    lib = ctypes.CDLL(LIB_PATH)
    i64, i32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
    for name in ("oracle_fwd", "oracle_dgrad", "oracle_wgrad"):
        f = getattr(lib, name)
        f.argtypes = [vp, vp, vp, i32, i64, i64, i64, vp, i64, vp, vp]
        f.restype = ctypes.c_int
    for name in ("oracle_router_exact", "oracle_router_bf16x3"):
        f = getattr(lib, name)
        f.argtypes = [vp, vp, i64, i64, i64, vp, i64, vp]
        f.restype = ctypes.c_int
    lib.oracle_round_f32.argtypes = [vp, vp, i64]
    lib.oracle_round_f32.restype = None
    lib.oracle_round_bf16.argtypes = [vp, vp, i64]
    lib.oracle_round_bf16.restype = None
    lib.oracle_threads.argtypes = []
    lib.oracle_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def threads() -> int:
    """OpenMP threads the oracle runs with."""
    return int(_load().oracle_threads())


def _u16(a):
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("BF16 operands are passed as uint16 bit patterns")
    return a


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _offsets(offs, M):
    o = np.ascontiguousarray(offs, dtype=np.int32)
    if o.ndim != 1 or o.size < 2:
        raise ValueError("offsets must be int32 [E+1]")
    return o


def _run3(fname, A, B, offs, E, M, N, K, size, idx):
    lib = _load()
    if idx is None:
        count = size
        idx_arr = None
    else:
        idx_arr = np.ascontiguousarray(idx, dtype=np.int64).ravel()
        count = idx_arr.size
    out = np.empty(count, dtype=np.float64)
    q = np.empty(count, dtype=np.float64)
    rc = getattr(lib, fname)(_ptr(A), _ptr(B), _ptr(offs), E, M, N, K,
                             _ptr(idx_arr), count, _ptr(out), _ptr(q))
    if rc != 0:
        raise ValueError(f"{fname} failed with code {rc}")
    return out, q


def fwd(X, W, offs, idx=None):
    """y[t,n] = sum_k x[t,k] w[e(t),n,k].  X [M,K], W [E,N,K] (uint16 BF16)."""
    X, W = _u16(X), _u16(W)
    o = _offsets(offs, X.shape[0])
    E, N, K = W.shape
    M = X.shape[0]
    if X.shape[1] != K or o.size != E + 1:
        raise ValueError("shape mismatch")
    v, q = _run3("oracle_fwd", X, W, o, E, M, N, K, M * N, idx)
    return (v.reshape(M, N), q.reshape(M, N)) if idx is None else (v, q)


def dgrad(G, W, offs, idx=None):
    """dx[t,k] = sum_n g[t,n] w[e(t),n,k].  G [M,N], W [E,N,K]."""
    G, W = _u16(G), _u16(W)
    o = _offsets(offs, G.shape[0])
    E, N, K = W.shape
    M = G.shape[0]
    if G.shape[1] != N or o.size != E + 1:
        raise ValueError("shape mismatch")
    v, q = _run3("oracle_dgrad", G, W, o, E, M, N, K, M * K, idx)
    return (v.reshape(M, K), q.reshape(M, K)) if idx is None else (v, q)


def wgrad(X, G, offs, idx=None):
    """dw[e,n,k] = sum over tokens t of expert e of g[t,n] x[t,k].
    X [M,K], G [M,N]; result [E,N,K]."""
    X, G = _u16(X), _u16(G)
    o = _offsets(offs, X.shape[0])
    E = o.size - 1
    M, K = X.shape
    N = G.shape[1]
    if G.shape[0] != M:
        raise ValueError("shape mismatch")
    v, q = _run3("oracle_wgrad", X, G, o, E, M, N, K, E * N * K, idx)
    return (v.reshape(E, N, K), q.reshape(E, N, K)) if idx is None else (v, q)


def round_f32(v):
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.float32)
    _load().oracle_round_f32(_ptr(v), _ptr(out), v.size)
    return out


def round_bf16(v):
    """Round float64 values once to BF16; returns uint16 bit patterns."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    _load().oracle_round_bf16(_ptr(v), _ptr(out), v.size)
    return out


def _router(fname, X, Wr, idx):
    X = np.ascontiguousarray(X, dtype=np.float32)
    Wr = np.ascontiguousarray(Wr, dtype=np.float32)
    M, K = X.shape
    N = Wr.shape[0]
    if Wr.shape[1] != K:
        raise ValueError("shape mismatch")
    if idx is None:
        idx_arr, count = None, M * N
    else:
        idx_arr = np.ascontiguousarray(idx, dtype=np.int64).ravel()
        count = idx_arr.size
    out = np.empty(count, dtype=np.float64)
    rc = getattr(_load(), fname)(_ptr(X), _ptr(Wr), M, N, K, _ptr(idx_arr), count, _ptr(out))
    if rc != 0:
        raise ValueError(f"{fname} failed with code {rc}")
    return out.reshape(M, N) if idx is None else out


def router_exact(X, Wr, idx=None):
    """out[m,n] = sum_k x[m,k] wr[n,k] of FP32 inputs, summed in binary64."""
    return _router("oracle_router_exact", X, Wr, idx)


def router_bf16x3(X, Wr, idx=None):
    """The BF16x3 emulation: hi*hi + hi*lo + lo*hi per product, in binary64."""
    return _router("oracle_router_bf16x3", X, Wr, idx)
