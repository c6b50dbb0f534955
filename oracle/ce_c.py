"""ctypes front end of the loss and gradient oracle in ``ce.c`` -- TEST INFRASTRUCTURE ONLY.

The C file's header states the definition and the passages it follows
("sampled_softmax.py" module docstring; "Learning Triton one kernel at a time:
softmax"; "16_optimization_checks.py" lm_gradient). The functions mirror ``ce.py``
(float64 numpy, an independent implementation of the same definition that pins this
one) but take the LM head W [V, d] and the candidate classes C (None: the whole
vocabulary) instead of the gathered rows:

* ``lse_rows``: L[t] for the given rows;
* ``loss_from_lse``: (loss, row_loss, N) from every row's L;
* ``dx_rows`` / ``dwc_rows``: rows of dX / of dW_C (candidate positions);
* ``forward_backward``: all of it, dense: (loss, dX, dW [V, d], L, row_loss).

Inputs are float64 (exact widenings of the bf16 / fp32 inputs). OpenMP spreads token
blocks over the host's cores (OMP_NUM_THREADS); results do not depend on the count.
"""
import ctypes

import numpy as np

from . import build as _build

_lib = None


class OracleCeError(RuntimeError):
    pass


def _load():
    global _lib
    if _lib is None:
        if _build.stale():
            _build.build(force=True)
        lib = ctypes.CDLL(_build.LIB)
        p, i64 = ctypes.c_void_p, ctypes.c_int64
        lib.oracle_ce_lse.argtypes = [i64, i64, i64, p, p, p, p, i64, p]
        lib.oracle_ce_loss.argtypes = [i64, i64, i64, p, p, p, p, p, p, p, p]
        lib.oracle_ce_dx_rows.argtypes = [i64, i64, i64, p, p, p, p, p, p, i64, p, i64, p]
        lib.oracle_ce_dwc_rows.argtypes = [i64, i64, i64, p, p, p, p, p, p, i64, p, i64, p]
        lib.oracle_ce_threads.argtypes = []
        for f in (lib.oracle_ce_threads, lib.oracle_ce_lse, lib.oracle_ce_loss, lib.oracle_ce_dx_rows, lib.oracle_ce_dwc_rows):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, name):
    if rc != 0:
        raise OracleCeError(f"{name} failed with code {rc}")


def _prep(x, W, C):
    x = np.ascontiguousarray(x, dtype=np.float64)
    W = np.ascontiguousarray(W, dtype=np.float64)
    if x.ndim != 2 or W.ndim != 2 or x.shape[1] != W.shape[1]:
        raise ValueError("x [T, d] and W [V, d] share d")
    if C is None:
        return x, W, None, W.shape[0]
    C = np.ascontiguousarray(C, dtype=np.int32)
    if C.size and (C.min() < 0 or C.max() >= W.shape[0]):
        raise ValueError("candidate classes outside [0, V)")
    return x, W, C, C.shape[0]


def _labels(target_pos, prefix_pos):
    t = np.ascontiguousarray(target_pos, dtype=np.int32)
    p = None if prefix_pos is None else np.ascontiguousarray(prefix_pos, dtype=np.int32)
    return t, p


def _idx(rows):
    return None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)


def threads():
    """Host threads the oracle's parallel loops use (OpenMP)."""
    return int(_load().oracle_ce_threads())


def lse_rows(x, W, C, rows=None):
    """L[t] of the given rows (all rows when None)."""
    x, W, C, P = _prep(x, W, C)
    rows = _idx(rows)
    n = x.shape[0] if rows is None else rows.shape[0]
    L = np.empty(n)
    _check(_load().oracle_ce_lse(x.shape[0], x.shape[1], P, _p(x), _p(W), _p(C), _p(rows), n, _p(L)),
           "oracle_ce_lse")
    return L


def loss_from_lse(x, W, C, L, target_pos, prefix_pos=None):
    """(loss, row_loss, N) given every row's L."""
    x, W, C, P = _prep(x, W, C)
    t, p = _labels(target_pos, prefix_pos)
    L = np.ascontiguousarray(L, dtype=np.float64)
    row_loss = np.empty(x.shape[0])
    out = np.zeros(2)
    _check(_load().oracle_ce_loss(x.shape[0], x.shape[1], P, _p(x), _p(W), _p(C), _p(L), _p(t), _p(p),
                                  _p(row_loss), _p(out)), "oracle_ce_loss")
    return float(out[0]), row_loss, int(out[1])


def dx_rows(x, W, C, L, target_pos, prefix_pos, N, rows=None):
    """dX[t] of the given rows (all when None)."""
    x, W, C, P = _prep(x, W, C)
    t, p = _labels(target_pos, prefix_pos)
    L = np.ascontiguousarray(L, dtype=np.float64)
    rows = _idx(rows)
    n = x.shape[0] if rows is None else rows.shape[0]
    out = np.empty((n, x.shape[1]))
    _check(_load().oracle_ce_dx_rows(x.shape[0], x.shape[1], P, _p(x), _p(W), _p(C), _p(L), _p(t), _p(p),
                                     int(N), _p(rows), n, _p(out)), "oracle_ce_dx_rows")
    return out


def dwc_rows(x, W, C, L, target_pos, prefix_pos, N, cand_rows=None):
    """dW_C[j] of the given candidate positions (all P when None), summed over every token."""
    x, W, C, P = _prep(x, W, C)
    t, p = _labels(target_pos, prefix_pos)
    L = np.ascontiguousarray(L, dtype=np.float64)
    cols = _idx(cand_rows)
    n = P if cols is None else cols.shape[0]
    out = np.empty((n, x.shape[1]))
    _check(_load().oracle_ce_dwc_rows(x.shape[0], x.shape[1], P, _p(x), _p(W), _p(C), _p(L), _p(t),
                                      _p(p), int(N), _p(cols), n, _p(out)), "oracle_ce_dwc_rows")
    return out


def forward_backward(x, W, C, target_pos, prefix_pos=None):
    """Dense: (loss, dX [T, d], dW [V, d], L [T], row_loss [T]); dW holds dW_C in the
    rows of C and exact zeros elsewhere."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    W = np.ascontiguousarray(W, dtype=np.float64)
    T, d = x.shape
    V = W.shape[0]
    if T == 0:
        return 0.0, np.zeros((0, d)), np.zeros((V, d)), np.zeros(0), np.zeros(0)
    L = lse_rows(x, W, C)
    loss, row_loss, N = loss_from_lse(x, W, C, L, target_pos, prefix_pos)
    dX = dx_rows(x, W, C, L, target_pos, prefix_pos, N)
    dWC = dwc_rows(x, W, C, L, target_pos, prefix_pos, N)
    dW = np.zeros((V, d))
    if C is None:
        dW[:] = dWC
    else:
        dW[np.asarray(C, dtype=np.int64)] = dWC
    return loss, dX, dW, L, row_loss
