"""The step under HIP graph capture: the library allocates, clears and synchronises
nothing inside a call, so one call can be captured and replayed. Each replay, with
other eager work on the device in between, must reproduce the eager call bit for bit
(every kernel of the step is deterministic)."""
import pytest
import torch

from oracle import fp8
from sampled_softmax_cross_amd import binding, synth
from tests.gpu_util import labels_dev, to_dev

pytestmark = pytest.mark.gpu

KEYS = ("loss", "dX", "dW", "C", "target_pos", "prefix_pos", "aux", "row_lse", "row_loss")


def _inputs(dtype, T=300, d=64, V=1000, P=333):
    x, W, y, p = synth.small_case(11, T, d, V, "bf16" if dtype.startswith("e4m3") else dtype,
                                  prefix=True, ignore_frac=0.05)
    return x, W, y, p, P


def _call(fn, outs, ws):
    return fn(outputs=outs, ws=ws, want_rows=True)


@pytest.mark.parametrize("dtype", ["bf16", "f32", "e4m3", "e4m3_refresh", "e4m3_bf16w"])
def test_captured_step_replays_bitwise(dtype):
    """e4m3_refresh: the cache refresh from bf16 W and the e4m3 step reading its scale on
    the device, captured together; e4m3_bf16w: the e4m3 step that encodes the candidate
    rows of bf16 W itself."""
    print(f"graph capture {dtype}", flush=True)
    x, W, y, p, P = _inputs(dtype)
    T, d = x.shape
    V = W.shape[0]
    xd = to_dev(x, "bf16" if dtype.startswith("e4m3") else dtype)
    yd, pd = labels_dev(y), labels_dev(p)
    if dtype == "e4m3_refresh":
        Wd = to_dev(W, "bf16")
        cache = dict(W8=torch.empty(V, d, dtype=torch.uint8, device=xd.device),
                     w_scale=torch.empty(1, dtype=torch.float32, device=xd.device),
                     status=torch.empty(1, dtype=torch.int32, device=xd.device))
        rws = torch.empty(binding.REFRESH_WORKSPACE_BYTES, dtype=torch.uint8, device=xd.device)

        def fn(**kw):
            binding.refresh_e4m3_cache(Wd, outputs=cache, ws=rws)
            return binding.forward_backward_fp8(xd, cache["W8"], cache["w_scale"], yd, pd, P, 7, 3,
                                                **kw)
        nbytes = binding.workspace_size(T, d, V, P, binding.SCE_E4M3)
    elif dtype == "e4m3_bf16w":
        Wd = to_dev(W, "bf16")
        fn = lambda **kw: binding.forward_backward_fp8_bf16w(xd, Wd, yd, pd, P, 7, 3, **kw)
        nbytes = binding.workspace_size(T, d, V, P, binding.SCE_E4M3_BF16W)
    elif dtype == "e4m3":
        codes, scale = fp8.e4m3_cache(synth.to_f64(W, "bf16"))
        W8 = torch.from_numpy(codes).cuda()
        fn = lambda **kw: binding.forward_backward_fp8(xd, W8, scale, yd, pd, P, 7, 3, **kw)
        nbytes = binding.workspace_size(T, d, V, P, binding.SCE_E4M3)
    else:
        Wd = to_dev(W, dtype)
        fn = lambda **kw: binding.forward_backward(xd, Wd, yd, pd, P, 7, 3, **kw)
        nbytes = binding.workspace_size(T, d, V, P, binding.dtype_code(xd.dtype))
    ws = binding.workspace(nbytes, xd.device)
    eager = _call(fn, None, ws)
    torch.cuda.synchronize()
    ref = {k: eager[k].clone() for k in KEYS if eager.get(k) is not None}
    outs = {k: torch.empty_like(v) for k, v in eager.items() if torch.is_tensor(v)}
    # warm up on a side stream (as torch's capture requires), then capture one call
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _call(fn, outs, ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _call(fn, outs, ws)
    noise = torch.randn(1 << 20, device=xd.device)
    for rep in range(4):
        for v in outs.values():
            v.fill_(7)                         # a replay must write every output again
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in ref.items():
            assert torch.equal(outs[k], v), (rep, k)
        # other work on the device between replays, including the library itself
        noise.mul_(1.0001).add_(0.5)
        _call(fn, None, binding.workspace(nbytes, xd.device))
        torch.cuda.synchronize()
