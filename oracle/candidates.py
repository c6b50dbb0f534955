"""ctypes front end of the candidate-build oracle in ``candidates.c``.

Test infrastructure only. Follows "sampled_softmax.py" (modded-nanogpt,
track_1_short), CandidateBuilder.build and CandidateBuilder._negatives; the C
file's header states each step.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_ERRORS = {1: "bad argument", 2: "more distinct targets than P", 3: "label out of range",
           4: "out of memory"}
_lib = None


class OracleError(RuntimeError):
    def __init__(self, code):
        super().__init__(f"oracle candidate build failed: {_ERRORS.get(code, code)}")
        self.code = code


def _load():
    global _lib
    if _lib is None:
        path = _build.LIB
        if _build.stale():
            _build.build(force=True)
        lib = ctypes.CDLL(path)
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        lib.oracle_build_candidates.argtypes = [i64, i64, i64, i64, i64, p, p, p, p, p, p, p]
        lib.oracle_build_candidates.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def build_candidates(V, P, stride, offset, targets, prefix_targets=None):
    """Run the candidate build for one microbatch.

    Returns a dict with ``C`` (int32 [P], ascending; [0, V) when P == 0),
    ``vocab_pos`` (int32 [V], -1 outside C), ``target_pos`` / ``prefix_pos``
    (int32 [T]; -1 for no label or a prefix target outside C; ``prefix_pos`` is
    all -1 when ``prefix_targets`` is None), and ``num_targets``, ``need``,
    ``draw``, ``next_offset``, ``fallback``, ``N``. Raises OracleError on the
    conditions the page asserts (too many distinct targets, gcd != 1) and on
    labels outside [-1, V).
    """
    lib = _load()
    targets = np.ascontiguousarray(targets, dtype=np.int64)
    T = targets.shape[0]
    pref = None if prefix_targets is None else np.ascontiguousarray(prefix_targets, dtype=np.int64)
    C = np.zeros(max(P, 1), dtype=np.int32)
    vocab_pos = np.zeros(V, dtype=np.int32)
    tpos = np.zeros(max(T, 1), dtype=np.int32)
    ppos = np.zeros(max(T, 1), dtype=np.int32)
    info = np.zeros(6, dtype=np.int64)
    rc = lib.oracle_build_candidates(V, P, stride, offset, T, _ptr(targets), _ptr(pref),
                                     _ptr(C), _ptr(vocab_pos), _ptr(tpos), _ptr(ppos), _ptr(info))
    if rc != 0:
        raise OracleError(rc)
    out = dict(C=np.arange(V, dtype=np.int32) if P == 0 else C[:P], vocab_pos=vocab_pos,
               target_pos=tpos[:T], prefix_pos=ppos[:T])
    out.update(num_targets=int(info[0]), need=int(info[1]), draw=int(info[2]),
               next_offset=int(info[3]), fallback=bool(info[4]), N=int(info[5]))
    return out
