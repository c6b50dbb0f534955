"""The on-device e4m3 lm_head cache refresh (sce_refresh_e4m3_cache) against the oracle's
cache (oracle.fp8.e4m3_cache, itself pinned to torch's float8_e4m3fn cast): scale and
every code bit for bit, and the e4m3 step reading the refreshed scale on the device."""
import numpy as np
import pytest
import torch

from oracle import build_candidates, fp8
from sampled_softmax_cross_amd import binding, synth
from tests.gpu_util import labels_dev, to_dev

pytestmark = pytest.mark.gpu


def _weights(seed, V, d, sd):
    return synth.normal(seed, 7, (V, d), sd, "bf16")


def _check(Wbits, label):
    V, d = Wbits.shape
    print(f"refresh {label} V={V} d={d}", flush=True)
    Wd = to_dev(Wbits, "bf16")
    out = binding.refresh_e4m3_cache(Wd)
    torch.cuda.synchronize()
    codes, s_w = fp8.e4m3_cache(synth.to_f64(Wbits, "bf16"))
    assert out["status"].item() == 0
    assert out["w_scale"].item() == s_w
    got = out["W8"].cpu().numpy()
    bad = np.argwhere(got != codes)
    assert bad.shape[0] == 0, (f"{bad.shape[0]} codes differ, first at {tuple(bad[0])}: "
                               f"{got[tuple(bad[0])]:#x} vs {codes[tuple(bad[0])]:#x}")
    return out


@pytest.mark.parametrize("V,d,sd,seed", [
    (50304, 768, 0.02, 1),        # the lm_head of the stage-0/1 workload
    (777, 144, 1.0, 2),           # ragged: V * d not a multiple of any launch's tile
    (3, 16, 3e-3, 3),             # smaller than one workgroup
    (131072, 64, 0.5, 4),         # V = SCE_MAX_V_SAMPLED
    (40, 16384, 0.05, 5),         # d = SCE_MAX_D
    (1048576, 16, 1e-2, 6),       # V = SCE_MAX_V
])
def test_refresh_bitwise(V, d, sd, seed):
    _check(_weights(seed, V, d, sd), "normal")


def test_refresh_edge_values():
    # zeros of both signs, values that land on e4m3 subnormals, on ties and on +-448
    W = _weights(11, 300, 64, 0.3)
    W[0, :] = 0
    W[1, :] = 0x8000                                 # -0.0
    # e4m3 subnormals after the scaling (|W| / s_w < 2^-6)
    W[2, :8] = (np.array([2.0 ** -16, -3 * 2.0 ** -18, 5 * 2.0 ** -19, 2.0 ** -20] * 2,
                         np.float32).view(np.uint32) >> 16).astype(np.uint16)
    out = _check(W, "edge")
    assert (out["W8"][1].cpu() == 0x80).all()        # -0 keeps its sign
    # all zeros: scale 1, every code 0
    Z = np.zeros((64, 32), np.uint16)
    out = _check(Z, "zeros")
    assert out["w_scale"].item() == 1.0


def test_refresh_flags_non_finite():
    W = _weights(12, 64, 32, 0.1)
    W[5, 7] = 0x7FC0                                 # a bf16 NaN
    out = binding.refresh_e4m3_cache(to_dev(W, "bf16"))
    torch.cuda.synchronize()
    assert out["status"].item() == binding.DEV_SCALE_RANGE
    assert out["w_scale"].item() == 1.0


def test_refresh_twice_reuses_outputs():
    """A second refresh into the same outputs (smaller magnitudes, new scale) leaves
    nothing of the first."""
    W1 = _weights(13, 1000, 96, 2.0)
    W2 = _weights(14, 1000, 96, 0.01)
    out = binding.refresh_e4m3_cache(to_dev(W1, "bf16"))
    out = binding.refresh_e4m3_cache(to_dev(W2, "bf16"), outputs=out)
    torch.cuda.synchronize()
    codes, s_w = fp8.e4m3_cache(synth.to_f64(W2, "bf16"))
    assert out["w_scale"].item() == s_w
    assert np.array_equal(out["W8"].cpu().numpy(), codes)


def test_step_reads_the_refreshed_scale_on_device():
    """The e4m3 step with the refresh's device scale gives, bit for bit, what it gives with
    the same scale passed from the host; a bad device scale is flagged."""
    T, d, V, P = 700, 384, 3000, 1111
    x, W, y, p = synth.small_case(21, T, d, V, "bf16", prefix=True, ignore_frac=0.05)
    xd, yd, pd = to_dev(x, "bf16"), labels_dev(y), labels_dev(p)
    cache = binding.refresh_e4m3_cache(to_dev(W, "bf16"))
    dev_out = binding.forward_backward_fp8(xd, cache["W8"], cache["w_scale"], yd, pd, P, 7, 3,
                                           want_rows=True)
    torch.cuda.synchronize()
    host_out = binding.forward_backward_fp8(xd, cache["W8"], cache["w_scale"].item(), yd, pd, P,
                                            7, 3, want_rows=True)
    torch.cuda.synchronize()
    for k in ("loss", "dX", "dW", "C", "target_pos", "prefix_pos", "row_lse", "row_loss", "aux",
              "scales"):
        a, b = dev_out[k], host_out[k]
        assert torch.equal(a.view(torch.uint8) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.uint8) if b.dtype == torch.bfloat16 else b), k
    assert dev_out["aux"][3].item() == 0
    # the candidate set agrees with the oracle's build (the refreshed step is the same step)
    cand = build_candidates(V, P, 7, 3, y, p)
    assert np.array_equal(dev_out["C"].cpu().numpy(), cand["C"])
    bad = torch.zeros(1, dtype=torch.float32, device=xd.device)
    out = binding.forward_backward_fp8(xd, cache["W8"], bad, yd, pd, P, 7, 3)
    torch.cuda.synchronize()
    assert out["aux"][3].item() & binding.DEV_SCALE_RANGE


BF16W_CASES = [
    # T, d, V, P, prefix, stride
    (300, 64, 1000, 333, True, 7),
    (2050, 96, 2500, 1601, False, 3),
    (257, 144, 777, 0, True, 1),               # full softmax: every row encoded, ragged V
    (1024, 16, 70000, 66000, True, 3),         # dW with more tiles than compute units
    (48, 64, 1048576, 0, True, 1),             # V = SCE_MAX_V, full softmax
    (16384, 768, 50304, 10240, False, 20011),  # the stage-0/1 workload
    (0, 64, 1000, 333, True, 7),               # no tokens
]


@pytest.mark.parametrize("T,d,V,P,prefix,stride", BF16W_CASES)
def test_step_from_bf16_weights_equals_refresh_then_step(T, d, V, P, prefix, stride):
    """The e4m3 step that encodes the candidate rows itself gives, bit for bit, what the
    cache refresh followed by the e4m3 step with the refreshed scale gives."""
    print(f"fp8 from bf16 W T={T} d={d} V={V} P={P}", flush=True)
    x, W, y, p = synth.small_case(T + V + P + 9, max(T, 1), d, V, "bf16", prefix=prefix,
                                  ignore_frac=0.05)
    x, y = x[:T], y[:T]
    p = None if p is None else p[:T]
    xd, Wd, yd, pd = to_dev(x, "bf16"), to_dev(W, "bf16"), labels_dev(y), labels_dev(p)
    off = (T * 7) % V
    cache = binding.refresh_e4m3_cache(Wd)
    ref = binding.forward_backward_fp8(xd, cache["W8"], cache["w_scale"], yd, pd, P, stride, off,
                                       want_rows=True)
    got = binding.forward_backward_fp8_bf16w(xd, Wd, yd, pd, P, stride, off, want_rows=True)
    torch.cuda.synchronize()
    keys = ["loss", "dX", "dW", "target_pos", "prefix_pos", "aux"] + (["row_lse", "row_loss"] if T else [])
    if P > 0:
        keys.append("C")
    for k in keys:
        a, b = got[k], ref[k]
        if a.dtype == torch.bfloat16:
            a, b = a.view(torch.int16), b.view(torch.int16)
        assert torch.equal(a, b), k
    assert torch.equal(got["scales"][:2], ref["scales"]), "s_x, s_g"
    assert got["scales"][2].item() == cache["w_scale"].item()
    assert got["aux"][3].item() == 0


def test_step_from_bf16_weights_flags_non_finite():
    T, d, V, P = 300, 64, 1000, 333
    x, W, y, p = synth.small_case(91, T, d, V, "bf16", prefix=True)
    W[17, 3] = 0x7F80                                # +inf in bf16
    out = binding.forward_backward_fp8_bf16w(to_dev(x, "bf16"), to_dev(W, "bf16"), labels_dev(y),
                                             labels_dev(p), P, 7, 3)
    torch.cuda.synchronize()
    assert out["aux"][3].item() & binding.DEV_SCALE_RANGE
    assert out["scales"][2].item() == 1.0
