"""Thin ctypes binding of libsampledce.so (C ABI in include/sampled_ce.h).

Argument marshalling only: tensors become device pointers, the current HIP
stream is passed through, outputs are allocated with torch. Every step of the
computation runs in the library's HIP kernels; there is no Python or CPU
fallback, and a missing library raises.
"""
import ctypes
import os

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libsampledce.so")

SCE_F32, SCE_BF16, SCE_E4M3, SCE_E4M3_BF16W = 0, 1, 2, 3
DEV_TOO_MANY_TARGETS, DEV_LABEL_RANGE, DEV_SCALE_RANGE = 1, 2, 4
# size limits (SCE_MAX_V_SAMPLED, SCE_MAX_V, SCE_MAX_D of include/sampled_ce.h)
MAX_V_SAMPLED, MAX_V, MAX_D = 131072, 1048576, 16384
STATUS = {0: "SCE_OK", 1: "SCE_EINVAL", 2: "SCE_EWORKSPACE", 3: "SCE_EHIP"}

EXPORTS = ("sce_workspace_size", "sce_build_candidates", "sce_build_candidates_noalloc",
           "sce_build_candidates_host",
           "sampled_ce_forward_backward", "sampled_ce_forward_backward_prebuilt",
           "sampled_ce_forward_backward_fp8", "sampled_ce_forward_backward_fp8_prebuilt",
           "sampled_ce_forward_backward_fp8_bf16w",
           "sce_refresh_e4m3_cache",
           "sce_ce_rows_workspace_size", "sce_ce_rows", "sce_gather_rows",
           "sce_profile_enable", "sce_profile_collect", "sce_status_string", "sce_abi_version")
STAGES = ("candidates", "logits", "ce", "dx", "dx_reduce", "dw", "scatter")

_lib = None


class SceError(RuntimeError):
    def __init__(self, fn, code):
        super().__init__(f"{fn} returned {STATUS.get(code, code)}")
        self.code = code


def load_library(path: str = LIB_PATH):
    """Load libsampledce.so (built by sampled_softmax_cross_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m sampled_softmax_cross_amd.build`; "
            "there is no fallback implementation")
    lib = ctypes.CDLL(path)
    p, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    lib.sce_workspace_size.argtypes = [i64, i64, i64, i64, i32, ctypes.POINTER(sz)]
    lib.sce_workspace_size.restype = i32
    lib.sce_build_candidates.argtypes = [p, p, i64, i64, i64, i64, i64, p, p, p, p, p, p, sz, p]
    lib.sce_build_candidates.restype = i32
    lib.sce_build_candidates_host.argtypes = [p, p, i64, i64, i64, i64, i64, p, p, p, p]
    lib.sce_build_candidates_host.restype = i32
    lib.sce_build_candidates_noalloc.argtypes = [p, p, i64, i64, i64, i64, i64, p, p, p, p, p, p]
    lib.sce_build_candidates_noalloc.restype = i32
    lib.sampled_ce_forward_backward.argtypes = [p, p, p, p, i64, i64, i64, i64, i64, i64, i32,
                                                p, p, p, p, p, p, p, p, p, p, sz, p]
    lib.sampled_ce_forward_backward.restype = i32
    lib.sampled_ce_forward_backward_prebuilt.argtypes = [p, p, p, p, p, p, i64, i64, i64, i64,
                                                         i32, p, p, p, p, p, p, p, sz, p]
    lib.sampled_ce_forward_backward_prebuilt.restype = i32
    lib.sampled_ce_forward_backward_fp8.argtypes = [p, p, ctypes.c_float, p, p, p, i64, i64, i64,
                                                    i64, i64, i64, p, p, p, p, p, p, p, p, p, p,
                                                    p, sz, p]
    lib.sampled_ce_forward_backward_fp8.restype = i32
    lib.sampled_ce_forward_backward_fp8_prebuilt.argtypes = [p, p, ctypes.c_float, p, p, p, p, p,
                                                             i64, i64, i64, i64, p, p, p, p, p,
                                                             p, p, p, sz, p]
    lib.sampled_ce_forward_backward_fp8_prebuilt.restype = i32
    lib.sampled_ce_forward_backward_fp8_bf16w.argtypes = [p, p, p, p, i64, i64, i64, i64, i64, i64,
                                                          p, p, p, p, p, p, p, p, p, p, p, sz, p]
    lib.sampled_ce_forward_backward_fp8_bf16w.restype = i32
    lib.sce_refresh_e4m3_cache.argtypes = [p, i64, i64, p, p, p, p, sz, p]
    lib.sce_refresh_e4m3_cache.restype = i32
    lib.sce_ce_rows_workspace_size.argtypes = [i64, ctypes.POINTER(sz)]
    lib.sce_ce_rows_workspace_size.restype = i32
    lib.sce_ce_rows.argtypes = [p, i64, i64, i64, i32, p, p, p, p, p, p, p, sz, p]
    lib.sce_ce_rows.restype = i32
    lib.sce_gather_rows.argtypes = [p, i64, i64, p, i64, i32, p, i64, p, p]
    lib.sce_gather_rows.restype = i32
    lib.sce_status_string.argtypes = [i32]
    lib.sce_status_string.restype = ctypes.c_char_p
    lib.sce_profile_enable.argtypes = [i32]
    lib.sce_profile_enable.restype = i32
    lib.sce_profile_collect.argtypes = [ctypes.POINTER(ctypes.c_double), i32, ctypes.POINTER(i32)]
    lib.sce_profile_collect.restype = i32
    lib.sce_abi_version.argtypes = []
    lib.sce_abi_version.restype = i32
    _lib = lib
    return lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return SCE_BF16
    if dt == torch.float32:
        return SCE_F32
    raise ValueError(f"unsupported dtype {dt}")


def workspace_size(T, d, V, P, dtype) -> int:
    lib = load_library()
    out = ctypes.c_size_t(0)
    rc = lib.sce_workspace_size(T, d, V, P, dtype_code(dtype) if isinstance(dtype, torch.dtype)
                                else int(dtype), ctypes.byref(out))
    if rc != 0:
        raise SceError("sce_workspace_size", rc)
    return out.value


_ws_cache = {}


def workspace(nbytes: int, device) -> torch.Tensor:
    """A reusable device workspace of at least nbytes (one per device and stream)."""
    key = (str(device), torch.cuda.current_stream(device).cuda_stream)
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < nbytes:
        _ws_cache.pop(key, None)
        ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        _ws_cache[key] = ws
    return ws


def build_candidates(targets, prefix_targets, V, P, stride, offset, *, want_vocab_pos=False,
                     ws=None, outputs=None):
    """Device candidate build; returns dict of tensors (C, target_pos, prefix_pos,
    vocab_pos or None, aux int64[4] = distinct, N, next_offset, device status).
    `outputs` may pass a previous result to write into (same T, V, P)."""
    lib = load_library()
    dev = targets.device
    T = targets.shape[0]
    o = outputs or {}
    C = o["C"] if "C" in o else torch.empty(P, dtype=torch.int32, device=dev)
    tpos = o["_tpos"] if "_tpos" in o else torch.empty(max(T, 1), dtype=torch.int32, device=dev)
    ppos = o["_ppos"] if "_ppos" in o else torch.empty(max(T, 1), dtype=torch.int32, device=dev)
    vpos = (o.get("vocab_pos") if o.get("vocab_pos") is not None
            else torch.empty(V, dtype=torch.int32, device=dev)) if want_vocab_pos else None
    aux = o["aux"] if "aux" in o else torch.empty(4, dtype=torch.int64, device=dev)
    nbytes = workspace_size(T, 8, V, P, SCE_F32)
    if ws is None:
        ws = workspace(nbytes, dev)
    rc = lib.sce_build_candidates(_ptr(targets), _ptr(prefix_targets), T, V, P, stride, offset,
                                  _ptr(C), _ptr(vpos), _ptr(tpos), _ptr(ppos), _ptr(aux),
                                  _ptr(ws), ws.numel(), _stream(dev))
    if rc != 0:
        raise SceError("sce_build_candidates", rc)
    return dict(C=C, target_pos=tpos[:T], prefix_pos=ppos[:T], vocab_pos=vpos, aux=aux,
                _tpos=tpos, _ppos=ppos, has_prefix=prefix_targets is not None)


def build_candidates_host(targets, prefix_targets, V, P, stride, offset, *, outputs=None):
    """The candidate build on the host (sce_build_candidates_host). targets / prefix_targets:
    int64 CPU tensors or numpy arrays (prefix may be None). Returns CPU tensors C, target_pos,
    prefix_pos (or None) and aux (int64 [4]); `outputs` may pass tensors to write into
    (pinned memory for an asynchronous upload). The call releases the interpreter lock while
    it builds, so a Python thread can run it beside the GPU's work."""
    import numpy as np

    lib = load_library()
    y = torch.as_tensor(np.ascontiguousarray(targets, dtype=np.int64)) if not torch.is_tensor(targets) else targets
    p = None
    if prefix_targets is not None:
        p = (torch.as_tensor(np.ascontiguousarray(prefix_targets, dtype=np.int64))
             if not torch.is_tensor(prefix_targets) else prefix_targets)
    for t in (y, p):
        if t is not None and (t.is_cuda or t.dtype != torch.int64 or not t.is_contiguous()):
            raise ValueError("labels must be contiguous int64 host tensors")
    T = y.shape[0]
    o = dict(outputs or {})
    if "C" not in o:
        o["C"] = torch.empty(P, dtype=torch.int32)
    if "target_pos" not in o:
        o["target_pos"] = torch.empty(max(T, 1), dtype=torch.int32)
    if "prefix_pos" not in o or (p is not None and o["prefix_pos"] is None):
        o["prefix_pos"] = torch.empty(max(T, 1), dtype=torch.int32) if p is not None else None
    if "aux" not in o:
        o["aux"] = torch.empty(4, dtype=torch.int64)
    rc = lib.sce_build_candidates_host(_ptr(y), _ptr(p), T, V, P, stride, offset, _ptr(o["C"]),
                                       _ptr(o["target_pos"]), _ptr(o["prefix_pos"]), _ptr(o["aux"]))
    if rc != 0:
        raise SceError("sce_build_candidates_host", rc)
    return o


def build_candidates_noalloc(targets, prefix_targets, V, P, stride, offset, *,
                             want_vocab_pos=False, want_prefix_pos=True):
    """The candidate build with the library's static scratch instead of a workspace
    (sce_build_candidates_noalloc). Same results as build_candidates; with
    want_prefix_pos=False no prefix positions are returned (the library keeps them in its
    scratch). Calls on one GPU must not overlap in time."""
    lib = load_library()
    dev = targets.device
    T = targets.shape[0]
    C = torch.empty(P, dtype=torch.int32, device=dev)
    tpos = torch.empty(max(T, 1), dtype=torch.int32, device=dev)
    ppos = torch.empty(max(T, 1), dtype=torch.int32, device=dev) if want_prefix_pos else None
    vpos = torch.empty(V, dtype=torch.int32, device=dev) if want_vocab_pos else None
    aux = torch.empty(4, dtype=torch.int64, device=dev)
    rc = lib.sce_build_candidates_noalloc(_ptr(targets), _ptr(prefix_targets), T, V, P, stride,
                                          offset, _ptr(C), _ptr(vpos), _ptr(tpos), _ptr(ppos),
                                          _ptr(aux), _stream(dev))
    if rc != 0:
        raise SceError("sce_build_candidates_noalloc", rc)
    return dict(C=C, target_pos=tpos[:T], prefix_pos=None if ppos is None else ppos[:T],
                vocab_pos=vpos, aux=aux, has_prefix=prefix_targets is not None)


def forward_backward(x, W, targets, prefix_targets, P, stride, offset, *, outputs=None, ws=None,
                     want_rows=False):
    """One sampled-CE step. x [T,d], W [V,d] (bf16 or fp32, contiguous, same dtype),
    targets / prefix_targets int64 [T] (prefix may be None).

    Returns dict: loss (fp32 [1]), dX, dW, C (int32 [P], ascending; None for P == 0),
    target_pos, prefix_pos (int32 [T]), aux (int64 [4]), and with want_rows the
    per-row log-sum-exp and loss terms (fp32 [T]). `outputs` may pass preallocated
    tensors under the same keys.
    """
    lib = load_library()
    dev = x.device
    T, d = x.shape
    V = W.shape[0]
    if W.dtype != x.dtype or W.shape[1] != d:
        raise ValueError("x and W must share dtype and hidden size")
    for name, t in (("x", x), ("W", W), ("targets", targets)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if targets.dtype != torch.int64 or (prefix_targets is not None and prefix_targets.dtype != torch.int64):
        raise ValueError("labels must be int64")
    o = dict(outputs or {})
    if "loss" not in o:
        o["loss"] = torch.empty(1, dtype=torch.float32, device=dev)
    if "dX" not in o:
        o["dX"] = torch.empty_like(x)
    if "dW" not in o:
        o["dW"] = torch.empty_like(W)
    if "C" not in o:
        o["C"] = torch.empty(max(P, 1), dtype=torch.int32, device=dev) if P > 0 else None
    for k in ("target_pos", "prefix_pos"):
        if k not in o:
            o[k] = torch.empty(max(T, 1), dtype=torch.int32, device=dev)
    if "aux" not in o:
        o["aux"] = torch.empty(4, dtype=torch.int64, device=dev)
    if want_rows:
        for k in ("row_lse", "row_loss"):
            if k not in o:
                o[k] = torch.empty(max(T, 1), dtype=torch.float32, device=dev)
    dt = dtype_code(x.dtype)
    nbytes = workspace_size(T, d, V, P, dt)
    if ws is None:
        ws = workspace(nbytes, dev)
    rc = lib.sampled_ce_forward_backward(
        _ptr(x), _ptr(W), _ptr(targets), _ptr(prefix_targets), T, d, V, P, stride, offset, dt,
        _ptr(o["loss"]), _ptr(o["dX"]), _ptr(o["dW"]), _ptr(o["C"]), _ptr(o["target_pos"]),
        _ptr(o["prefix_pos"]), _ptr(o.get("row_lse")), _ptr(o.get("row_loss")), _ptr(o["aux"]),
        _ptr(ws), ws.numel(), _stream(dev))
    if rc != 0:
        raise SceError("sampled_ce_forward_backward", rc)
    if o["C"] is not None:
        o["C"] = o["C"][:P]
    o["target_pos"] = o["target_pos"][:T]
    o["prefix_pos"] = o["prefix_pos"][:T]
    return o


def forward_backward_prebuilt(x, W, cand, *, outputs=None, ws=None, want_rows=False):
    """The step from a candidate set built beforehand: `cand` is the dict that
    build_candidates / build_candidates_noalloc returned (C, target_pos, prefix_pos or
    None, aux). Returns the keys of forward_backward except C and the positions."""
    lib = load_library()
    dev = x.device
    T, d = x.shape
    V = W.shape[0]
    P = cand["C"].shape[0]
    if W.dtype != x.dtype or W.shape[1] != d:
        raise ValueError("x and W must share dtype and hidden size")
    for name, t in (("x", x), ("W", W)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    for k in ("C", "target_pos", "prefix_pos"):
        t = cand.get(k)
        if t is not None and (t.dtype != torch.int32 or not t.is_contiguous()):
            raise ValueError(f"{k} must be contiguous int32")
    o = dict(outputs or {})
    if "loss" not in o:
        o["loss"] = torch.empty(1, dtype=torch.float32, device=dev)
    if "dX" not in o:
        o["dX"] = torch.empty_like(x)
    if "dW" not in o:
        o["dW"] = torch.empty_like(W)
    if "aux" not in o:
        o["aux"] = torch.empty(4, dtype=torch.int64, device=dev)
    if want_rows:
        for k in ("row_lse", "row_loss"):
            if k not in o:
                o[k] = torch.empty(max(T, 1), dtype=torch.float32, device=dev)
    dt = dtype_code(x.dtype)
    nbytes = workspace_size(T, d, V, P, dt)
    if ws is None:
        ws = workspace(nbytes, dev)
    rc = lib.sampled_ce_forward_backward_prebuilt(
        _ptr(x), _ptr(W), _ptr(cand["C"]), _ptr(cand["target_pos"]), _ptr(cand.get("prefix_pos")),
        _ptr(cand.get("aux")), T, d, V, P, dt, _ptr(o["loss"]), _ptr(o["dX"]), _ptr(o["dW"]),
        _ptr(o.get("row_lse")), _ptr(o.get("row_loss")), _ptr(o["aux"]), _ptr(ws), ws.numel(),
        _stream(dev))
    if rc != 0:
        raise SceError("sampled_ce_forward_backward_prebuilt", rc)
    return o


def _scale_args(w_scale, dev):
    """(host scale, device scale tensor or None) from a float or a float32 device tensor."""
    if isinstance(w_scale, torch.Tensor):
        if w_scale.dtype != torch.float32 or w_scale.device != dev or w_scale.numel() < 1:
            raise ValueError("a device w_scale is a float32 tensor on x's device")
        return 1.0, w_scale
    return float(w_scale), None


def forward_backward_fp8_prebuilt(x, W8, w_scale, cand, *, outputs=None, ws=None,
                                  want_rows=False):
    """The e4m3 step from a candidate set built beforehand (`cand` as for
    forward_backward_prebuilt); x, W8 and w_scale as for forward_backward_fp8. Returns
    its keys except C and the positions. The gradient's scale depends on whether the
    microbatch has prefix targets (n_max): a set built without them (cand["has_prefix"]
    False, or prefix_pos None) is stepped without prefix positions, as the one-call step
    is."""
    lib = load_library()
    dev = x.device
    T, d = x.shape
    V = W8.shape[0]
    P = cand["C"].shape[0]
    if x.dtype != torch.bfloat16 or W8.shape[1] != d or W8.element_size() != 1:
        raise ValueError("x must be bf16 and W8 one byte per element with x's hidden size")
    for name, t in (("x", x), ("W8", W8)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    for k in ("C", "target_pos", "prefix_pos"):
        t = cand.get(k)
        if t is not None and (t.dtype != torch.int32 or not t.is_contiguous()):
            raise ValueError(f"{k} must be contiguous int32")
    o = dict(outputs or {})
    if "loss" not in o:
        o["loss"] = torch.empty(1, dtype=torch.float32, device=dev)
    if "dX" not in o:
        o["dX"] = torch.empty_like(x)
    if "dW" not in o:
        o["dW"] = torch.empty(V, d, dtype=torch.bfloat16, device=dev)
    if "aux" not in o:
        o["aux"] = torch.empty(4, dtype=torch.int64, device=dev)
    if "scales" not in o:
        o["scales"] = torch.empty(2, dtype=torch.float32, device=dev)
    if want_rows:
        for k in ("row_lse", "row_loss"):
            if k not in o:
                o[k] = torch.empty(max(T, 1), dtype=torch.float32, device=dev)
    host_scale, dev_scale = _scale_args(w_scale, dev)
    nbytes = workspace_size(T, d, V, P, SCE_E4M3)
    if ws is None:
        ws = workspace(nbytes, dev)
    rc = lib.sampled_ce_forward_backward_fp8_prebuilt(
        _ptr(x), _ptr(W8), ctypes.c_float(host_scale), _ptr(dev_scale), _ptr(cand["C"]),
        _ptr(cand["target_pos"]), _ptr(cand.get("prefix_pos") if cand.get("has_prefix", True) else None),
        _ptr(cand.get("aux")), T, d, V, P,
        _ptr(o["loss"]), _ptr(o["dX"]), _ptr(o["dW"]), _ptr(o.get("row_lse")),
        _ptr(o.get("row_loss")), _ptr(o["aux"]), _ptr(o["scales"]), _ptr(ws), ws.numel(),
        _stream(dev))
    if rc != 0:
        raise SceError("sampled_ce_forward_backward_fp8_prebuilt", rc)
    return o


def forward_backward_fp8(x, W8, w_scale, targets, prefix_targets, P, stride, offset, *,
                         outputs=None, ws=None, want_rows=False):
    """One sampled-CE step with e4m3 product operands. x [T,d] bf16, W8 [V,d] the lm_head
    as e4m3 codes (torch.uint8 or torch.float8_e4m3fn), w_scale its dequantisation scale:
    a Python float, or a one-element float32 device tensor that the step reads on the
    device (refresh_e4m3_cache's "w_scale"), labels as in forward_backward.

    Returns the keys of forward_backward (dX and dW bf16) plus `scales` (fp32 [2]:
    s_x, s_g).
    """
    lib = load_library()
    dev = x.device
    T, d = x.shape
    V = W8.shape[0]
    if x.dtype != torch.bfloat16 or W8.shape[1] != d or W8.element_size() != 1:
        raise ValueError("x must be bf16 and W8 one byte per element with x's hidden size")
    for name, t in (("x", x), ("W8", W8), ("targets", targets)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if targets.dtype != torch.int64 or (prefix_targets is not None and prefix_targets.dtype != torch.int64):
        raise ValueError("labels must be int64")
    o = dict(outputs or {})
    if "loss" not in o:
        o["loss"] = torch.empty(1, dtype=torch.float32, device=dev)
    if "dX" not in o:
        o["dX"] = torch.empty_like(x)
    if "dW" not in o:
        o["dW"] = torch.empty(V, d, dtype=torch.bfloat16, device=dev)
    if "C" not in o:
        o["C"] = torch.empty(max(P, 1), dtype=torch.int32, device=dev) if P > 0 else None
    for k in ("target_pos", "prefix_pos"):
        if k not in o:
            o[k] = torch.empty(max(T, 1), dtype=torch.int32, device=dev)
    if "aux" not in o:
        o["aux"] = torch.empty(4, dtype=torch.int64, device=dev)
    if "scales" not in o:
        o["scales"] = torch.empty(2, dtype=torch.float32, device=dev)
    if want_rows:
        for k in ("row_lse", "row_loss"):
            if k not in o:
                o[k] = torch.empty(max(T, 1), dtype=torch.float32, device=dev)
    nbytes = workspace_size(T, d, V, P, SCE_E4M3)
    if ws is None:
        ws = workspace(nbytes, dev)
    host_scale, dev_scale = _scale_args(w_scale, dev)
    rc = lib.sampled_ce_forward_backward_fp8(
        _ptr(x), _ptr(W8), ctypes.c_float(host_scale), _ptr(dev_scale), _ptr(targets), _ptr(prefix_targets), T, d, V,
        P, stride, offset, _ptr(o["loss"]), _ptr(o["dX"]), _ptr(o["dW"]), _ptr(o["C"]),
        _ptr(o["target_pos"]), _ptr(o["prefix_pos"]), _ptr(o.get("row_lse")),
        _ptr(o.get("row_loss")), _ptr(o["aux"]), _ptr(o["scales"]), _ptr(ws), ws.numel(),
        _stream(dev))
    if rc != 0:
        raise SceError("sampled_ce_forward_backward_fp8", rc)
    if o["C"] is not None:
        o["C"] = o["C"][:P]
    o["target_pos"] = o["target_pos"][:T]
    o["prefix_pos"] = o["prefix_pos"][:T]
    return o


REFRESH_WORKSPACE_BYTES = 8192  # SCE_REFRESH_WORKSPACE_BYTES


def refresh_e4m3_cache(W, *, outputs=None, ws=None):
    """Rebuild the e4m3 lm_head cache on the device from W [V, d] bf16: returns dict
    W8 (uint8 [V, d] codes), w_scale (float32 [1], s_w = max|W| / 448) and status
    (int32 [1]: 0, or DEV_SCALE_RANGE for a non-finite W). `outputs` may pass a previous
    result to overwrite (same shape)."""
    lib = load_library()
    dev = W.device
    if W.dtype != torch.bfloat16 or W.dim() != 2 or not W.is_contiguous():
        raise ValueError("W must be a contiguous bf16 [V, d] tensor")
    V, d = W.shape
    o = dict(outputs or {})
    if "W8" not in o:
        o["W8"] = torch.empty(V, d, dtype=torch.uint8, device=dev)
    if "w_scale" not in o:
        o["w_scale"] = torch.empty(1, dtype=torch.float32, device=dev)
    if "status" not in o:
        o["status"] = torch.empty(1, dtype=torch.int32, device=dev)
    if ws is None:
        ws = workspace(REFRESH_WORKSPACE_BYTES, dev)
    rc = lib.sce_refresh_e4m3_cache(_ptr(W), V, d, _ptr(o["W8"]), _ptr(o["w_scale"]),
                                    _ptr(o["status"]), _ptr(ws), ws.numel(), _stream(dev))
    if rc != 0:
        raise SceError("sce_refresh_e4m3_cache", rc)
    return o


def forward_backward_fp8_bf16w(x, W, targets, prefix_targets, P, stride, offset, *,
                               outputs=None, ws=None, want_rows=False):
    """The e4m3 step from bf16 weights W [V, d], the cache refresh folded in (the scale
    and the candidate rows' codes formed inside the step). Returns the keys of
    forward_backward_fp8, with `scales` fp32 [3]: s_x, s_g, s_w."""
    lib = load_library()
    dev = x.device
    T, d = x.shape
    V = W.shape[0]
    if x.dtype != torch.bfloat16 or W.dtype != torch.bfloat16 or W.shape[1] != d:
        raise ValueError("x and W must be bf16 with the same hidden size")
    for name, t in (("x", x), ("W", W), ("targets", targets)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if targets.dtype != torch.int64 or (prefix_targets is not None and prefix_targets.dtype != torch.int64):
        raise ValueError("labels must be int64")
    o = dict(outputs or {})
    if "loss" not in o:
        o["loss"] = torch.empty(1, dtype=torch.float32, device=dev)
    if "dX" not in o:
        o["dX"] = torch.empty_like(x)
    if "dW" not in o:
        o["dW"] = torch.empty(V, d, dtype=torch.bfloat16, device=dev)
    if "C" not in o:
        o["C"] = torch.empty(max(P, 1), dtype=torch.int32, device=dev) if P > 0 else None
    for k in ("target_pos", "prefix_pos"):
        if k not in o:
            o[k] = torch.empty(max(T, 1), dtype=torch.int32, device=dev)
    if "aux" not in o:
        o["aux"] = torch.empty(4, dtype=torch.int64, device=dev)
    if "scales" not in o:
        o["scales"] = torch.empty(3, dtype=torch.float32, device=dev)
    if want_rows:
        for k in ("row_lse", "row_loss"):
            if k not in o:
                o[k] = torch.empty(max(T, 1), dtype=torch.float32, device=dev)
    nbytes = workspace_size(T, d, V, P, SCE_E4M3_BF16W)
    if ws is None:
        ws = workspace(nbytes, dev)
    rc = lib.sampled_ce_forward_backward_fp8_bf16w(
        _ptr(x), _ptr(W), _ptr(targets), _ptr(prefix_targets), T, d, V, P, stride, offset,
        _ptr(o["loss"]), _ptr(o["dX"]), _ptr(o["dW"]), _ptr(o["C"]), _ptr(o["target_pos"]),
        _ptr(o["prefix_pos"]), _ptr(o.get("row_lse")), _ptr(o.get("row_loss")), _ptr(o["aux"]),
        _ptr(o["scales"]), _ptr(ws), ws.numel(), _stream(dev))
    if rc != 0:
        raise SceError("sampled_ce_forward_backward_fp8_bf16w", rc)
    if o["C"] is not None:
        o["C"] = o["C"][:P]
    o["target_pos"] = o["target_pos"][:T]
    o["prefix_pos"] = o["prefix_pos"][:T]
    return o


def ce_rows(Z, P, target_pos, prefix_pos=None, *, want_rows=False, ws=None):
    """The fused CE forward/backward alone, in place: Z [T, ldz] (bf16 or fp32,
    contiguous, ldz % 8 == 0) holds logits in columns [0, P) and is overwritten with
    their gradient. target_pos / prefix_pos are int32 [T] positions in [0, P) or -1.
    Returns dict: loss (fp32 [1]), aux (int64 [4]: 0, N, 0, device status) and with
    want_rows row_lse, row_loss (fp32 [T])."""
    lib = load_library()
    dev = Z.device
    T, ldz = Z.shape
    if not Z.is_contiguous():
        raise ValueError("Z must be contiguous")
    for t in (target_pos, prefix_pos):
        if t is not None and (t.dtype != torch.int32 or not t.is_contiguous() or t.shape[0] != T):
            raise ValueError("label positions must be contiguous int32 [T]")
    o = {"loss": torch.empty(1, dtype=torch.float32, device=dev),
         "aux": torch.empty(4, dtype=torch.int64, device=dev)}
    if want_rows:
        o["row_lse"] = torch.empty(max(T, 1), dtype=torch.float32, device=dev)
        o["row_loss"] = torch.empty(max(T, 1), dtype=torch.float32, device=dev)
    out = ctypes.c_size_t(0)
    rc = lib.sce_ce_rows_workspace_size(T, ctypes.byref(out))
    if rc != 0:
        raise SceError("sce_ce_rows_workspace_size", rc)
    if ws is None:
        ws = workspace(out.value, dev)
    rc = lib.sce_ce_rows(_ptr(Z), ldz, T, P, dtype_code(Z.dtype), _ptr(target_pos),
                         _ptr(prefix_pos), _ptr(o["loss"]), _ptr(o.get("row_loss")),
                         _ptr(o.get("row_lse")), _ptr(o["aux"]), _ptr(ws), ws.numel(), _stream(dev))
    if rc != 0:
        raise SceError("sce_ce_rows", rc)
    return o


def gather_rows(W, idx, *, out=None, status=None):
    """out[i] = W[idx[i]] (bit for bit) for W [V, d] (bf16 or fp32, contiguous) and
    int32 idx [n]; rows of out may be padded (out [n, ld_out], ld_out % 8 == 0). An
    index outside [0, V) gives zeros and, with a zeroed int32 [1] `status`, sets
    DEV_LABEL_RANGE in it."""
    lib = load_library()
    dev = W.device
    V, d = W.shape
    n = idx.shape[0]
    if not W.is_contiguous() or idx.dtype != torch.int32 or not idx.is_contiguous():
        raise ValueError("W must be contiguous and idx contiguous int32")
    if out is None:
        out = torch.empty(n, d, dtype=W.dtype, device=dev)
    if out.dtype != W.dtype or out.shape[0] != n or out.stride(1) != 1 or out.shape[1] < d:
        raise ValueError("out must be [n, >= d] with unit column stride, dtype of W")
    rc = lib.sce_gather_rows(_ptr(W), V, d, _ptr(idx), n, dtype_code(W.dtype), _ptr(out),
                             out.stride(0), _ptr(status), _stream(dev))
    if rc != 0:
        raise SceError("sce_gather_rows", rc)
    return out


def profile_enable(on: bool) -> None:
    """Start/stop per-stage HIP-event timing inside the library."""
    load_library().sce_profile_enable(1 if on else 0)


def profile_collect():
    """(milliseconds per stage summed over the timed calls, number of calls)."""
    lib = load_library()
    arr = (ctypes.c_double * len(STAGES))()
    n = ctypes.c_int(0)
    rc = lib.sce_profile_collect(arr, len(STAGES), ctypes.byref(n))
    if rc != 0:
        raise SceError("sce_profile_collect", rc)
    return {k: arr[i] for i, k in enumerate(STAGES)}, n.value
