"""CPU oracle for the Interleaved Head Attention forward pass (ctypes wrapper).

TEST INFRASTRUCTURE ONLY.  The oracle is a plain double-precision C++
implementation of Algorithm 1 of the "Interleaved Head Attention" page, with
the textbook's Algorithm 5.1 ("Attention mechanism" chapter, section 5.3) as
its per-row attention core.  Only the test-suite, the smoke check and the
benchmark's CPU-baseline leg may import this package; the product path never
does.  It shares no code with the HIP library.

Functions and the passages they follow:
  attention(...)    textbook section 5.3, eq. 5.11 and Algorithm 5.1
  forward(...)      IHA page section 4, Algorithm 1 (mixing, stacking, attention,
                    collapse, concatenation)
  nexus_inner(...)  "Higher-order attention mechanisms" page, section 2: the inner
                    attention softmax(Q Q^T / sqrt(d_k)) Q, per head, each row by
                    Algorithm 5.1 with the queries as keys and values
  param_count()     IHA page, Theorem 2: Q + 4 H^2 P
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "iha_oracle.cpp")
_LIB = os.path.join(_HERE, "libiha_oracle.so")

OK, ERR_ARG, ERR_EMPTY_ROW, ERR_NONFINITE = 0, 1, 2, 3
MASK_NONE, MASK_CAUSAL, MASK_WINDOW = 0, 1, 2


class OracleError(RuntimeError):
    def __init__(self, code: int):
        names = {ERR_ARG: "invalid argument", ERR_EMPTY_ROW: "empty allowed set",
                 ERR_NONFINITE: "non-finite value"}
        super().__init__(f"oracle error {code}: {names.get(code, '?')}")
        self.code = code


def build(verbose: bool = False) -> str:
    """Compile the oracle with g++ (OpenMP, -O3; no target-specific flags)."""
    cmd = ["g++", "-std=c++17", "-O3", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           _SRC, "-o", _LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        d = ctypes.POINTER(ctypes.c_double)
        i64 = ctypes.c_int64
        lib.iho_attention.argtypes = [i64, i64, i64, i64, d, d, d, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_int, i64, ctypes.c_double,
                                      d, ctypes.c_void_p, ctypes.c_void_p]
        lib.iho_attention.restype = ctypes.c_int
        lib.iho_forward.argtypes = [i64, i64, i64, i64, i64, ctypes.c_int, i64] + [d] * 8 + [
            ctypes.c_void_p, i64, d, ctypes.c_void_p, ctypes.c_int]
        lib.iho_forward.restype = ctypes.c_int
        lib.iho_threads.argtypes = [ctypes.c_int]
        lib.iho_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _d(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def threads(nthreads: int = 0) -> int:
    return _load().iho_threads(nthreads)


def attention(Q, K, V, mask: int = MASK_NONE, window: int = 0, qpos=None, kpos=None,
              scale: Optional[float] = None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Single-head strict-visibility attention (Algorithm 5.1).  Returns (O, A, rowsum)."""
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    T, dk = Q.shape
    S, dv = V.shape
    assert K.shape == (S, dk)
    O = np.zeros((T, dv))
    A = np.zeros((T, S))
    rs = np.zeros(T)
    qp = None if qpos is None else np.ascontiguousarray(qpos, dtype=np.int64)
    kp = None if kpos is None else np.ascontiguousarray(kpos, dtype=np.int64)
    sc = 1.0 / np.sqrt(dk) if scale is None else float(scale)
    rc = _load().iho_attention(T, S, dk, dv, _d(Q), _d(K), _d(V),
                               None if qp is None else qp.ctypes.data,
                               None if kp is None else kp.ctypes.data,
                               mask, window, sc, _d(O), A.ctypes.data, rs.ctypes.data)
    if rc != OK:
        raise OracleError(rc)
    return O, A, rs


def forward(X, WQ, WK, WV, aQ, aK, aV, R, H: int, P: int, mask: int, window: int = 0,
            tokens: Optional[Sequence[int]] = None, nthreads: int = 0,
            return_rowsum_dev: bool = False):
    """IHA forward (Algorithm 1) in double.

    X is [B, N, D].  With ``tokens`` (flat indices b*N + t) only those output rows
    are produced, as a [len(tokens), D] array; otherwise [B, N, D].
    """
    X = _f64(X)
    B, N, D = X.shape
    arrs = [X] + [_f64(a) for a in (WQ, WK, WV, aQ, aK, aV, R)]
    assert arrs[1].shape == (D, D) and arrs[4].shape == (H, H, P) and arrs[7].shape == (H, H * P)
    if tokens is None:
        out = np.zeros((B, N, D))
        tk, nt = None, 0
    else:
        tk = np.ascontiguousarray(tokens, dtype=np.int64)
        nt = tk.size
        out = np.zeros((nt, D))
    dev = np.zeros(1)
    rc = _load().iho_forward(B, N, D, H, P, mask, window, *[_d(a) for a in arrs],
                             None if tk is None else tk.ctypes.data, nt, _d(out),
                             dev.ctypes.data, nthreads)
    if rc != OK:
        raise OracleError(rc)
    return (out, float(dev[0])) if return_rowsum_dev else out


def nexus_inner(Q, mask: int = MASK_NONE, window: int = 0) -> np.ndarray:
    """Nexus inner attention ("Higher-order attention mechanisms" page, section 2):
    Attention_q(X) = softmax(Q Q^T / sqrt(d_k)) Q, for Q [B, L, H, d] per (b, h) - the
    attention of each row over the visible rows of the same Q, which serve as keys and
    values.  The page's formula has no mask (MASK_NONE); causal and window masks restrict
    the visible rows as for the IHA forward.  Returns [B, L, H, d] in double."""
    Q = _f64(Q)
    B, L, H, d = Q.shape
    out = np.zeros_like(Q)
    for b in range(B):
        for h in range(H):
            q = np.ascontiguousarray(Q[b, :, h])
            out[b, :, h], _, _ = attention(q, q, q, mask, window)
    return out


def param_count(D: int, H: int, P: int) -> int:
    """Q + 4 H^2 P (IHA page, Theorem 2): Q = 3 D^2 projection weights, 3 H^2 P mixing
    coefficients and H^2 P collapse entries."""
    return 3 * D * D + 4 * H * H * P
