"""Helpers for the GPU parity tests: device transfer and error measures."""
import numpy as np
import torch

from sampled_softmax_cross_amd import synth


def to_dev(a, dtype):
    """numpy input (bf16 bits as uint16, or float32) -> device tensor of that dtype."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def labels_dev(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.int64)).cuda()


def to_f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def max_rel(got, ref):
    """max |got - ref| / max |ref| over the tensor (the tolerance measure for dX, dW)."""
    den = np.abs(ref).max()
    num = np.abs(got - ref).max()
    return num / den if den > 0 else num


def max_row_rel(got, ref, floor=1e-3, scale=None):
    """Largest per-row max-relative error max|got_r - ref_r| / max|ref_r| over the rows whose
    largest oracle entry is at least `floor` times `scale` (default: the tensor's largest
    entry). A row of small values is held to its own magnitude, not to the tensor's
    largest row. Returns (worst ratio, number of rows checked)."""
    ref = np.asarray(ref)
    got = np.asarray(got)
    row_max = np.abs(ref).max(axis=1)
    top = np.abs(ref).max() if scale is None else scale
    sel = row_max >= floor * top
    if not sel.any():
        return 0.0, 0
    err = np.abs(got[sel] - ref[sel]).max(axis=1) / row_max[sel]
    return float(err.max()), int(sel.sum())


TOL = {"bf16": dict(loss=1e-3, grad=2e-2), "f32": dict(loss=1e-5, grad=1e-5)}


def inputs_f64(x, W, dtype):
    return synth.to_f64(x, dtype), synth.to_f64(W, dtype)
