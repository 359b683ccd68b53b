"""CPU oracle for the offline top-K distillation KL loss (ctypes binding).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg import this package.  The GPU library and its
Python binding never import, load or call it, and share no code with it.

The arithmetic lives in ``fckl_oracle.c`` (plain C, IEEE double, OpenMP over
tokens); this module only compiles it with gcc and marshals numpy arrays.  Every
floating-point input is converted to float64 before the call, so bf16 or fp32
values reach the oracle exactly.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fckl_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libfckl_oracle.so")
_lib: Optional[ctypes.CDLL] = None

ORACLE_OK, ORACLE_EARG, ORACLE_EIDX, ORACLE_EMEM = 0, -1, -2, -3


class OracleError(RuntimeError):
    pass


def build(force: bool = True) -> str:
    """Compile fckl_oracle.c into libfckl_oracle.so next to it (gcc, -O2, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-Wall", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        # FCKL_ORACLE_LIB names another build of the same source (the mutation tests
        # use it to load an oracle with a planted mistake); it is never rebuilt here.
        path = os.environ.get("FCKL_ORACLE_LIB")
        if not path:
            path = _LIB_PATH
            if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_SRC):
                build(force=True)
        lib = ctypes.CDLL(path)
        i64, f64, vp = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        lib.fckl_oracle_forward.argtypes = [i64, i64, i64, i64, f64, vp, vp, vp, vp, i64, vp, vp, vp]
        lib.fckl_oracle_forward.restype = ctypes.c_int
        lib.fckl_oracle_loss_mean.argtypes = [i64, i64, i64, i64, f64, vp, vp, vp, vp, vp]
        lib.fckl_oracle_loss_mean.restype = ctypes.c_int
        lib.fckl_oracle_backward.argtypes = [i64, i64, i64, i64, f64, vp, vp, vp, vp, f64, i64, i64, vp, vp, vp]
        lib.fckl_oracle_backward.restype = ctypes.c_int
        lib.fckl_oracle_weighted_mean.argtypes = [i64, i64, i64, i64, f64, vp, vp, vp, vp, vp, vp]
        lib.fckl_oracle_weighted_mean.restype = ctypes.c_int
        lib.fckl_oracle_weighted_backward.argtypes = [i64, i64, i64, i64, f64, vp, vp, vp, vp, vp, f64, i64, vp,
                                                      vp, vp]
        lib.fckl_oracle_weighted_backward.restype = ctypes.c_int
        lib.fckl_oracle_topk.argtypes = [i64, i64, i64, i64, vp, vp, vp, vp]
        lib.fckl_oracle_topk.restype = ctypes.c_int
        lib.fckl_oracle_full.argtypes = [i64, i64, i64, i64, f64, vp, vp, vp, vp, vp, f64, vp, vp, vp, vp, vp]
        lib.fckl_oracle_full.restype = ctypes.c_int
        lib.fckl_oracle_num_threads.argtypes = []
        lib.fckl_oracle_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _shapes(h, W, idx, tl):
    N, H = h.shape
    V, H2 = W.shape
    N2, K = idx.shape
    if H2 != H or N2 != N or tl.shape != idx.shape:
        raise ValueError("inconsistent shapes h%s W%s idx%s tl%s" % (h.shape, W.shape, idx.shape, tl.shape))
    return N, H, V, K


def _check(rc: int):
    if rc != ORACLE_OK:
        raise OracleError({ORACLE_EARG: "invalid argument", ORACLE_EIDX: "index out of range",
                           ORACLE_EMEM: "host allocation failed"}.get(rc, "error %d" % rc))


def forward(h, W, idx, tl, T: float, rows=None):
    """Per-token loss and lse = logsumexp(z/T) for the selected rows (all rows if None).

    Returns (loss[nrows], lse[nrows]) as float64 arrays.
    """
    h, W, idx, tl = _f64(h), _f64(W), _i32(idx), _f64(tl)
    N, H, V, K = _shapes(h, W, idx, tl)
    r = None if rows is None else np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    nrows = N if r is None else r.shape[0]
    loss = np.empty(nrows, np.float64)
    lse = np.empty(nrows, np.float64)
    _check(_load().fckl_oracle_forward(N, H, V, K, float(T), _ptr(h), _ptr(W), _ptr(idx), _ptr(tl),
                                       nrows, _ptr(r), _ptr(loss), _ptr(lse)))
    return loss, lse


def loss_mean(h, W, idx, tl, T: float) -> float:
    """Mean over all tokens of the per-token loss."""
    h, W, idx, tl = _f64(h), _f64(W), _i32(idx), _f64(tl)
    N, H, V, K = _shapes(h, W, idx, tl)
    out = np.zeros(1, np.float64)
    _check(_load().fckl_oracle_loss_mean(N, H, V, K, float(T), _ptr(h), _ptr(W), _ptr(idx), _ptr(tl), _ptr(out)))
    return float(out[0])


def backward(h, W, idx, tl, T: float, grad_scale: float = 1.0, n_norm: Optional[int] = None,
             rows=None, want_dH: bool = True, want_dW: bool = True):
    """Gradients of grad_scale * (1/n_norm) * sum_{selected rows} loss[i].

    n_norm defaults to N (the gradient of grad_scale * mean loss when rows is None).
    Returns (dH[nrows, H] or None, dW[V, H] or None), float64.
    """
    h, W, idx, tl = _f64(h), _f64(W), _i32(idx), _f64(tl)
    N, H, V, K = _shapes(h, W, idx, tl)
    r = None if rows is None else np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    nrows = N if r is None else r.shape[0]
    dH = np.empty((nrows, H), np.float64) if want_dH else None
    dW = np.empty((V, H), np.float64) if want_dW else None
    _check(_load().fckl_oracle_backward(N, H, V, K, float(T), _ptr(h), _ptr(W), _ptr(idx), _ptr(tl),
                                        float(grad_scale), int(N if n_norm is None else n_norm),
                                        nrows, _ptr(r), _ptr(dH), _ptr(dW)))
    return dH, dW


def weighted_mean(h, W, idx, tl, T: float, w) -> float:
    """sum_i w[i] loss[i] / sum_i w[i] over all tokens (0 when every weight is 0)."""
    h, W, idx, tl, w = _f64(h), _f64(W), _i32(idx), _f64(tl), _f64(w)
    N, H, V, K = _shapes(h, W, idx, tl)
    if w.shape != (N,):
        raise ValueError("weights must have shape (N,)")
    out = np.zeros(1, np.float64)
    _check(_load().fckl_oracle_weighted_mean(N, H, V, K, float(T), _ptr(h), _ptr(W), _ptr(idx), _ptr(tl), _ptr(w),
                                             _ptr(out)))
    return float(out[0])


def weighted_backward(h, W, idx, tl, T: float, w, grad_scale: float = 1.0, rows=None, want_dH: bool = True,
                      want_dW: bool = True):
    """Gradients of grad_scale * weighted mean loss; row i scaled by w[i] / sum_j w[j].

    Returns (dH[nrows, H] or None, dW[V, H] or None), float64; dW sums the selected rows.
    """
    h, W, idx, tl, w = _f64(h), _f64(W), _i32(idx), _f64(tl), _f64(w)
    N, H, V, K = _shapes(h, W, idx, tl)
    if w.shape != (N,):
        raise ValueError("weights must have shape (N,)")
    r = None if rows is None else np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    nrows = N if r is None else r.shape[0]
    dH = np.empty((nrows, H), np.float64) if want_dH else None
    dW = np.empty((V, H), np.float64) if want_dW else None
    _check(_load().fckl_oracle_weighted_backward(N, H, V, K, float(T), _ptr(h), _ptr(W), _ptr(idx), _ptr(tl),
                                                 _ptr(w), float(grad_scale), nrows, _ptr(r), _ptr(dH), _ptr(dW)))
    return dH, dW


def topk(h, W, K: int):
    """Per token, the K largest z = h W^T in descending order, equal values by smaller index.

    Returns (idx[N, K] int32, z[N, K] float64).
    """
    h, W = _f64(h), _f64(W)
    N, H = h.shape
    V, H2 = W.shape
    if H2 != H:
        raise ValueError("inconsistent shapes h%s W%s" % (h.shape, W.shape))
    idx = np.empty((N, K), np.int32)
    val = np.empty((N, K), np.float64)
    _check(_load().fckl_oracle_topk(N, H, V, int(K), _ptr(h), _ptr(W), _ptr(idx), _ptr(val)))
    return idx, val


def full(hs, Ws, ht, Wt, T: float, w=None, grad_scale: float = 1.0, want_grads: bool = True):
    """Online distillation against the full teacher distribution p = softmax(ht Wt^T / T).

    Returns (loss[N], lse[N] of the student, weighted mean, dH[N,Hs] or None, dW[V,Hs] or None).
    """
    hs, Ws, ht, Wt = _f64(hs), _f64(Ws), _f64(ht), _f64(Wt)
    N, Hs = hs.shape
    V, Hs2 = Ws.shape
    N2, Ht = ht.shape
    if Hs2 != Hs or N2 != N or Wt.shape != (V, Ht):
        raise ValueError("inconsistent shapes hs%s Ws%s ht%s Wt%s" % (hs.shape, Ws.shape, ht.shape, Wt.shape))
    wv = None if w is None else _f64(w)
    if wv is not None and wv.shape != (N,):
        raise ValueError("weights must have shape (N,)")
    loss = np.empty(N, np.float64)
    lse = np.empty(N, np.float64)
    mean = np.zeros(1, np.float64)
    dH = np.empty((N, Hs), np.float64) if want_grads else None
    dW = np.empty((V, Hs), np.float64) if want_grads else None
    _check(_load().fckl_oracle_full(N, Hs, Ht, V, float(T), _ptr(hs), _ptr(Ws), _ptr(ht), _ptr(Wt), _ptr(wv),
                                    float(grad_scale), _ptr(loss), _ptr(lse), _ptr(mean), _ptr(dH), _ptr(dW)))
    return loss, lse, float(mean[0]), dH, dW


def num_threads() -> int:
    """OpenMP threads the oracle's parallel regions use (OMP_NUM_THREADS or all cores)."""
    return int(_load().fckl_oracle_num_threads())
