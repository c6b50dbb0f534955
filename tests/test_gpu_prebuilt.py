"""The step from a candidate set built beforehand (sampled_ce_forward_backward_prebuilt):
bit for bit the one-call step; two steps on two streams with distinct workspaces at the
same time, each bit for bit its serial run; the next microbatch's build on a second
stream overlapping the current step; bad sets and positions flagged, not faulted."""
import numpy as np
import pytest
import torch

from sampled_softmax_cross_amd import binding, synth
from tests.gpu_util import labels_dev, to_dev

pytestmark = pytest.mark.gpu

KEYS = ("loss", "dX", "dW", "row_lse", "row_loss", "aux")


def _inputs(seed, T, d, V, dtype, prefix, ign=0.05):
    x, W, y, p = synth.small_case(seed, T, d, V, dtype, prefix=prefix, ignore_frac=ign)
    return to_dev(x, dtype), to_dev(W, dtype), labels_dev(y), labels_dev(p)


CASES = [
    # T, d, V, P, dtype, prefix, stride
    (300, 64, 1000, 333, "bf16", True, 7),
    (512, 128, 4096, 2048, "f32", False, 1021),
    (2050, 96, 2500, 1601, "bf16", False, 3),
    (700, 384, 3000, 1111, "bf16", True, 7),
    (16384, 768, 50304, 10240, "bf16", False, 20011),
]


@pytest.mark.parametrize("T,d,V,P,dtype,prefix,stride", CASES)
def test_prebuilt_equals_one_call_bitwise(T, d, V, P, dtype, prefix, stride):
    print(f"prebuilt T={T} d={d} V={V} P={P} {dtype}", flush=True)
    x, W, y, p = _inputs(T + P, T, d, V, dtype, prefix)
    off = (T * 5) % V
    ref = binding.forward_backward(x, W, y, p, P, stride, off, want_rows=True)
    cand = binding.build_candidates(y, p, V, P, stride, off)
    got = binding.forward_backward_prebuilt(x, W, cand, want_rows=True)
    torch.cuda.synchronize()
    for k in KEYS:
        assert torch.equal(got[k], ref[k]), k
    assert got["aux"][3].item() == 0


def test_noalloc_build_feeds_the_step():
    x, W, y, p = _inputs(5, 300, 64, 1000, "bf16", True)
    ref = binding.forward_backward(x, W, y, p, 333, 7, 11, want_rows=True)
    cand = binding.build_candidates_noalloc(y, p, 1000, 333, 7, 11)
    got = binding.forward_backward_prebuilt(x, W, cand, want_rows=True)
    torch.cuda.synchronize()
    for k in KEYS:
        assert torch.equal(got[k], ref[k]), k


def test_two_streams_distinct_workspaces():
    """Two microbatches, each built and stepped on its own stream with its own workspaces
    and outputs, launched together; each result equals its serial run bit for bit."""
    T, d, V, P = 4096, 256, 8192, 3000
    mb = [_inputs(11 + i, T, d, V, "bf16", True) for i in range(2)]
    serial = []
    for i, (x, W, y, p) in enumerate(mb):
        serial.append(binding.forward_backward(x, W, y, p, P, 97, 100 * i, want_rows=True))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    nbytes = binding.workspace_size(T, d, V, P, binding.SCE_BF16)
    nb = binding.workspace_size(T, 8, V, P, binding.SCE_F32)
    wss = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(2)]
    bws = [torch.empty(nb, dtype=torch.uint8, device="cuda") for _ in range(2)]
    torch.cuda.synchronize()
    outs = [None, None]
    for rep in range(3):
        for i, (x, W, y, p) in enumerate(mb):
            with torch.cuda.stream(streams[i]):
                if i == 0:
                    outs[i] = binding.forward_backward(x, W, y, p, P, 97, 100 * i, ws=wss[i],
                                                       want_rows=True)
                else:
                    cand = binding.build_candidates(y, p, V, P, 97, 100 * i, ws=bws[i])
                    outs[i] = binding.forward_backward_prebuilt(x, W, cand, ws=wss[i],
                                                                want_rows=True)
        torch.cuda.synchronize()
        for i in range(2):
            for k in KEYS:
                assert torch.equal(outs[i][k], serial[i][k]), (rep, i, k)


def test_next_build_overlaps_the_step():
    """The overlapped pattern: the build of microbatch i + 1 on a side stream while the step
    of microbatch i runs on the main stream (events order the two), four microbatches in a
    row, each step bit for bit its one-call result."""
    T, d, V, P = 8192, 768, 50304, 10240
    x, W, _, _ = _inputs(21, T, d, V, "bf16", False)
    w = synth.workload("stage01")
    labels = [labels_dev(synth.make_labels(w, c)[0][:T]) for c in range(4)]
    offs = [(1000 + c * P) % V for c in range(4)]
    ref = [binding.forward_backward(x, W, labels[c], None, P, 20011, offs[c]) for c in range(4)]
    ref = [{k: r[k].clone() for k in ("loss", "dX", "dW", "aux")} for r in ref]
    torch.cuda.synchronize()
    main, side = torch.cuda.current_stream(), torch.cuda.Stream()
    nb = binding.workspace_size(T, 8, V, P, binding.SCE_F32)
    bws = [torch.empty(nb, dtype=torch.uint8, device="cuda") for _ in range(2)]
    built = [torch.cuda.Event(), torch.cuda.Event()]
    used = [torch.cuda.Event(), torch.cuda.Event()]
    bufs = [None, None]
    with torch.cuda.stream(side):
        bufs[0] = binding.build_candidates(labels[0], None, V, P, 20011, offs[0], ws=bws[0])
        built[0].record(side)
    outs = None
    for c in range(4):
        if c + 1 < 4:
            with torch.cuda.stream(side):
                if c >= 1:
                    side.wait_event(used[(c + 1) % 2])  # the step that read this slot is done
                bufs[(c + 1) % 2] = binding.build_candidates(labels[c + 1], None, V, P, 20011,
                                                             offs[c + 1], ws=bws[(c + 1) % 2],
                                                             outputs=bufs[(c + 1) % 2])
                built[(c + 1) % 2].record(side)
        main.wait_event(built[c % 2])
        outs = binding.forward_backward_prebuilt(x, W, bufs[c % 2], outputs=outs)
        used[c % 2].record(main)
        got = {k: outs[k].clone() for k in ("loss", "dX", "dW", "aux")}
        torch.cuda.synchronize()
        for k in got:
            assert torch.equal(got[k], ref[c][k]), (c, k)


def test_bad_sets_are_flagged():
    T, d, V, P = 64, 64, 500, 100
    x, W, y, p = _inputs(7, T, d, V, "bf16", True)
    cand = binding.build_candidates(y, p, V, P, 7, 0)
    good = {k: v.clone() if torch.is_tensor(v) else v for k, v in cand.items()}
    for mutate in ("range", "order", "position"):
        c = {k: v.clone() if torch.is_tensor(v) else v for k, v in good.items()}
        if mutate == "range":
            c["C"][P - 1] = V + 7
        elif mutate == "order":
            c["C"][5] = c["C"][4]
        else:
            c["target_pos"][3] = P + 2
        c["aux"] = None
        out = binding.forward_backward_prebuilt(x, W, c)
        torch.cuda.synchronize()
        assert out["aux"][3].item() & binding.DEV_LABEL_RANGE, mutate


def test_host_build_feeds_the_step():
    """The set built on the host (sce_build_candidates_host) and uploaded equals the device
    build, and the step from it equals the one-call step, bit for bit."""
    T, d, V, P = 2048, 256, 8192, 2000
    x, W, y, p = _inputs(31, T, d, V, "bf16", True)
    ref = binding.forward_backward(x, W, y, p, P, 97, 55, want_rows=True)
    hb = binding.build_candidates_host(y.cpu(), p.cpu(), V, P, 97, 55)
    dev = {k: (v.cuda() if v is not None else None) for k, v in hb.items()}
    got = binding.forward_backward_prebuilt(x, W, dev, want_rows=True)
    db = binding.build_candidates(y, p, V, P, 97, 55)
    torch.cuda.synchronize()
    assert torch.equal(dev["C"], db["C"]) and torch.equal(dev["aux"], db["aux"])
    for k in KEYS:
        assert torch.equal(got[k], ref[k]), k


FP8_CASES = [
    # T, d, V, P, prefix, stride
    (300, 64, 1000, 333, True, 7),
    (2050, 96, 2500, 1601, False, 3),
    (1024, 16, 70000, 66000, True, 3),     # dW with more tiles than compute units
    (16384, 768, 50304, 10240, False, 20011),
]


@pytest.mark.parametrize("T,d,V,P,prefix,stride", FP8_CASES)
def test_fp8_prebuilt_equals_one_call_bitwise(T, d, V, P, prefix, stride):
    """The e4m3 step from a device-built set, with the refreshed cache's scale read on the
    device, equals the one-call e4m3 step bit for bit."""
    print(f"fp8 prebuilt T={T} d={d} V={V} P={P}", flush=True)
    x, W, y, p = _inputs(T + P + 3, T, d, V, "bf16", prefix)
    cache = binding.refresh_e4m3_cache(W)
    off = (T * 5) % V
    ref = binding.forward_backward_fp8(x, cache["W8"], cache["w_scale"], y, p, P, stride, off,
                                       want_rows=True)
    cand = binding.build_candidates(y, p, V, P, stride, off)
    got = binding.forward_backward_fp8_prebuilt(x, cache["W8"], cache["w_scale"], cand,
                                                want_rows=True)
    torch.cuda.synchronize()
    for k in KEYS + ("scales",):
        assert torch.equal(got[k], ref[k]), k
    assert got["aux"][3].item() == 0


def test_fp8_host_build_feeds_the_step():
    """The page's arrangement end to end: candidate set built on the host, uploaded, the
    e4m3 cache refreshed on the device, the e4m3 step from the uploaded set."""
    T, d, V, P, stride, off = 2000, 128, 6000, 2500, 7, 123
    x, W, y, p = _inputs(77, T, d, V, "bf16", True)
    host = binding.build_candidates_host(y.cpu(), p.cpu(), V, P, stride, off)
    cand = {k: (v.to(x.device) if v is not None else None) for k, v in host.items()}
    cache = binding.refresh_e4m3_cache(W)
    got = binding.forward_backward_fp8_prebuilt(x, cache["W8"], cache["w_scale"], cand,
                                                want_rows=True)
    ref = binding.forward_backward_fp8(x, cache["W8"], cache["w_scale"], y, p, P, stride, off,
                                       want_rows=True)
    torch.cuda.synchronize()
    for k in KEYS + ("scales",):
        assert torch.equal(got[k], ref[k]), k


def test_fp8_prebuilt_bad_set_is_flagged():
    T, d, V, P = 300, 64, 1000, 333
    x, W, y, p = _inputs(78, T, d, V, "bf16", True)
    cache = binding.refresh_e4m3_cache(W)
    cand = binding.build_candidates(y, p, V, P, 7, 0)
    C = cand["C"].clone()
    C[5] = C[4]                          # not ascending
    bad = dict(cand, C=C)
    out = binding.forward_backward_fp8_prebuilt(x, cache["W8"], cache["w_scale"], bad)
    torch.cuda.synchronize()
    assert out["aux"][3].item() & binding.DEV_LABEL_RANGE
