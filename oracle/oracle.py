"""Python face of the f64 CPU oracle (test infrastructure only).

Only tests, the smoke check and the benchmark's CPU-baseline leg may import this
module.  It loads ``libfab_oracle.so`` (plain C, built by ``oracle/build.py``)
and adds the central-difference helper that the ggmlR test file
"tests/testthat/test-flash-attn-back.R" uses as its gradient check (`num_grad`:
central differences of sum(d * attn) with eps = 1e-3).

Arrays follow ggml ne order stored C-contiguous with the shape reversed:
q (B,H,N,DK), k (B,Hkv,M,DK), v (B,Hkv,M,DV), d and O (B,N,H,DV),
LSE and D (B,H,N), mask bits uint16 (N,M).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfab_oracle.so")

_lib = None


def use_library(path):
    """Point this module at another build of the oracle source (used by the tests
    that plant mistakes in a copy of the oracle); returns the previous handle."""
    global _lib
    prev = _lib
    _lib = _load(path)
    return prev


def restore_library(handle):
    global _lib
    _lib = handle


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _b  # noqa: F401  (package-relative when imported as oracle.oracle)
            _b.build()
        _lib = _load(LIB_PATH)
    return _lib


def _load(path):
    L = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    L.fab_oracle_half_to_double.restype = ctypes.c_double
    L.fab_oracle_half_to_double.argtypes = [ctypes.c_uint16]
    L.fab_oracle_forward.restype = ctypes.c_int
    L.fab_oracle_forward.argtypes = [P, P, P, P, P, ctypes.c_double, P, P, ctypes.c_int]
    L.fab_oracle_backward.restype = ctypes.c_int
    L.fab_oracle_backward.argtypes = [P, P, P, P, P, P, ctypes.c_double, P, P, P, P, P, P,
                                      ctypes.c_int]
    L.fab_oracle_backward_sampled.restype = ctypes.c_int
    L.fab_oracle_backward_sampled.argtypes = [P, P, P, P, P, P, ctypes.c_double, P, I64, P,
                                              P, I64, P, P, ctypes.c_int]
    L.fab_oracle_forward_alibi.restype = ctypes.c_int
    L.fab_oracle_forward_alibi.argtypes = [P, P, P, P, P, P, ctypes.c_double, P, P, ctypes.c_int]
    L.fab_oracle_backward_alibi.restype = ctypes.c_int
    L.fab_oracle_backward_alibi.argtypes = [P, P, P, P, P, P, P, ctypes.c_double, P, P, P, P, P, P,
                                            ctypes.c_int]
    L.fab_oracle_backward_sampled_alibi.restype = ctypes.c_int
    L.fab_oracle_backward_sampled_alibi.argtypes = [P, P, P, P, P, P, P, ctypes.c_double, P, I64, P,
                                                    P, I64, P, P, ctypes.c_int]
    L.fab_oracle_blob_layout.restype = ctypes.c_int
    L.fab_oracle_blob_layout.argtypes = [P, P]
    L.fab_oracle_pack.restype = ctypes.c_int
    L.fab_oracle_pack.argtypes = [P, P, P, P, P]
    return L


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _shape7(shape):
    return np.ascontiguousarray(np.array(shape.astuple(), dtype=np.int64))


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _mask(mask):
    if mask is None:
        return None
    return np.ascontiguousarray(mask, dtype=np.uint16)


def _alibi(shape, alibi):
    """Per-head ALiBi slopes as f64 [H], or None."""
    if alibi is None:
        return None
    a = np.ascontiguousarray(np.asarray(alibi, dtype=np.float64).reshape(-1))
    if a.size != shape.H:
        raise ValueError(f"alibi needs {shape.H} slopes, got {a.size}")
    return a


def half_to_double(bits: int) -> float:
    return lib().fab_oracle_half_to_double(int(bits))


def forward(shape, q, k, v, mask, scale, nthreads=None, alibi=None):
    """O (B,N,H,DV) and LSE (B,H,N) in f64.  alibi: per-head slopes [H] or None
    (score scale*q.k + alibi[h]*(m - n) + mask)."""
    s = shape
    O = np.zeros((s.B, s.N, s.H, s.DV))
    lse = np.zeros((s.B, s.H, s.N))
    q, k, v, m = _f64(q), _f64(k), _f64(v), _mask(mask)
    a = _alibi(s, alibi)
    sh = _shape7(s)
    rc = lib().fab_oracle_forward_alibi(_ptr(sh), _ptr(q), _ptr(k), _ptr(v), _ptr(m), _ptr(a), float(scale),
                                        _ptr(O), _ptr(lse), nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle forward rejected the shape ({rc})")
    return O, lse


def backward(shape, q, k, v, mask, d, scale, nthreads=None, alibi=None):
    """dict with dq, dk, dv (ne-shaped f64), O, lse, D.  alibi as for forward()."""
    s = shape
    out = dict(
        dq=np.zeros(s.q_shape), dk=np.zeros(s.k_shape), dv=np.zeros(s.v_shape),
        O=np.zeros(s.d_shape), lse=np.zeros((s.B, s.H, s.N)), D=np.zeros((s.B, s.H, s.N)))
    q, k, v, d, m = _f64(q), _f64(k), _f64(v), _f64(d), _mask(mask)
    a = _alibi(s, alibi)
    sh = _shape7(s)
    rc = lib().fab_oracle_backward_alibi(_ptr(sh), _ptr(q), _ptr(k), _ptr(v), _ptr(m), _ptr(a), _ptr(d),
                                         float(scale), _ptr(out["dq"]), _ptr(out["dk"]),
                                         _ptr(out["dv"]), _ptr(out["O"]), _ptr(out["lse"]),
                                         _ptr(out["D"]), nthreads or default_threads())
    if rc == -2:
        raise AssertionError("oracle self-check D = dO.O = sum P dP failed")
    if rc != 0:
        raise ValueError(f"oracle backward rejected the shape ({rc})")
    return out


def backward_sampled(shape, q, k, v, mask, d, scale, rows, keys, nthreads=None, alibi=None):
    """dQ rows for flat row ids (n + N*(h + H*b)) and dK/dV rows for flat key ids
    (m + M*(g + Hkv*b)).  Returns (dq [len(rows), DK], dk [len(keys), DK], dv [len(keys), DV])."""
    s = shape
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    keys = np.ascontiguousarray(np.asarray(keys, dtype=np.int64))
    dq = np.zeros((len(rows), s.DK))
    dk = np.zeros((len(keys), s.DK))
    dv = np.zeros((len(keys), s.DV))
    q, k, v, d, m = _f64(q), _f64(k), _f64(v), _f64(d), _mask(mask)
    a = _alibi(s, alibi)
    sh = _shape7(s)
    rc = lib().fab_oracle_backward_sampled_alibi(
        _ptr(sh), _ptr(q), _ptr(k), _ptr(v), _ptr(m), _ptr(a), _ptr(d), float(scale),
        _ptr(rows), len(rows), _ptr(dq), _ptr(keys), len(keys), _ptr(dk), _ptr(dv),
        nthreads or default_threads())
    if rc == -2:
        raise AssertionError("oracle self-check D = dO.O = sum P dP failed")
    if rc != 0:
        raise ValueError(f"oracle rejected the shape ({rc})")
    return dq, dk, dv


def blob_layout(shape):
    """(off_q, off_k, off_v, total) in floats."""
    off = np.zeros(4, dtype=np.int64)
    sh = _shape7(shape)
    lib().fab_oracle_blob_layout(_ptr(sh), _ptr(off))
    return tuple(int(x) for x in off)


def pack(shape, dq, dk, dv):
    """f64 blob [dQ | pad | dK | pad | dV | pad] with zero pads."""
    total = blob_layout(shape)[3]
    blob = np.zeros(max(total, 1))
    sh = _shape7(shape)
    dq, dk, dv = _f64(dq), _f64(dk), _f64(dv)
    lib().fab_oracle_pack(_ptr(sh), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(blob))
    return blob[:total]


def loss(shape, q, k, v, mask, d, scale, alibi=None):
    """sum(d * attn(q, k, v)) in f64: the scalar whose gradient the backward returns."""
    O, _ = forward(shape, q, k, v, mask, scale, nthreads=1, alibi=alibi)
    return float(np.sum(_f64(d) * O))


def num_grad(shape, q, k, v, mask, d, scale, which, eps=1e-3, alibi=None):
    """Central-difference gradient of sum(d * attn) w.r.t. q, k or v (f64 inputs)."""
    vals = {"q": _f64(q).copy(), "k": _f64(k).copy(), "v": _f64(v).copy()}
    x = vals[which]
    g = np.zeros(x.size)
    flat = x.reshape(-1)
    for i in range(x.size):
        orig = flat[i]
        flat[i] = orig + eps
        fh = loss(shape, vals["q"], vals["k"], vals["v"], mask, d, scale, alibi)
        flat[i] = orig - eps
        fl = loss(shape, vals["q"], vals["k"], vals["v"], mask, d, scale, alibi)
        flat[i] = orig
        g[i] = (fh - fl) / (2 * eps)
    return g.reshape(x.shape)
