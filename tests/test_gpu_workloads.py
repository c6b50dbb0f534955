"""The five named workloads at full size, in the launch configuration the benchmark
times. Integers are compared exactly; the loss against the oracle's full float64
evaluation; dX and dW on sampled rows the oracle computes one by one; every row of
dW outside C must be exactly zero."""
import numpy as np
import pytest
import torch

from oracle import build_candidates, ce_c
from sampled_softmax_cross_amd import binding, synth
from tests.gpu_util import TOL, inputs_f64, labels_dev, max_rel, max_row_rel, to_dev, to_f64

pytestmark = pytest.mark.gpu


def _window_members(V, stride, offset, draw):
    """Classes in the sweep window [offset, offset + draw): via the inverse of the stride."""
    inv = pow(stride % V, -1, V)
    k = (np.arange(V, dtype=object) * inv % V).astype(np.int64)  # sweep index of each class
    return ((k - offset) % V) < draw


@pytest.mark.parametrize("name", ["tiny", "stage01", "s2early", "s2late", "full"])
def test_workload(name):
    w = synth.workload(name)
    print(f"workload {name}: T={w.T} d={w.d} V={w.V} P={w.P} {w.dtype}", flush=True)
    x, W = synth.make_weights(w)
    xd, Wd = to_dev(x, w.dtype), to_dev(W, w.dtype)
    xf, Wf = inputs_f64(x, W, w.dtype)
    tol = TOL[w.dtype]
    rng = np.random.default_rng(123)
    neg_hits = np.zeros(w.V, dtype=np.int64)
    win_hits = np.zeros(w.V, dtype=np.int64)
    for call in range(w.calls):
        y, p = synth.make_labels(w, call)
        off = w.call_offset(call)
        print(f"  call {call} offset {off}", flush=True)
        out = binding.forward_backward(xd, Wd, labels_dev(y), labels_dev(p), w.P, w.stride, off,
                                       want_rows=True)
        torch.cuda.synchronize()
        cand = build_candidates(w.V, w.P, w.stride, off, y, p)
        # candidate set, positions, counters: exact
        if w.P > 0:
            C = out["C"].cpu().numpy()
            assert np.array_equal(C, cand["C"])
        assert np.array_equal(out["target_pos"].cpu().numpy(), cand["target_pos"])
        assert np.array_equal(out["prefix_pos"].cpu().numpy(), cand["prefix_pos"])
        aux = out["aux"].cpu().numpy().tolist()
        assert aux == [cand["num_targets"], cand["N"], cand["next_offset"], 0]
        assert not cand["fallback"]
        if w.P > 0:
            negs = np.setdiff1d(cand["C"], y)
            inside = _window_members(w.V, w.stride, off, cand["draw"])
            assert inside[negs].all()  # every negative comes from this call's window
            neg_hits[negs] += 1
            win_hits += inside
        Cc = None if w.P == 0 else cand["C"]
        P_eff = w.V if w.P == 0 else w.P
        tpos, ppos = cand["target_pos"], (cand["prefix_pos"] if p is not None else None)
        N = cand["N"]
        L_rows = np.zeros(w.T)
        rows = np.unique(np.concatenate([[0, 1, w.T - 1], rng.integers(0, w.T, 29)]))
        gl = to_f64(out["row_lse"])
        if call == 0:
            L = ce_c.lse_rows(xf, Wf, Cc)
            loss, row_loss, N2 = ce_c.loss_from_lse(xf, Wf, Cc, L, tpos, ppos)
            assert N2 == N
            got = float(out["loss"].item())
            print(f"  loss {got:.7f} oracle {loss:.7f} rel {abs(got - loss) / abs(loss):.2e}", flush=True)
            assert abs(got - loss) <= tol["loss"] * abs(loss), (got, loss)
            np.testing.assert_allclose(gl, L, rtol=tol["loss"], atol=0)
            assert max_rel(to_f64(out["row_loss"]), row_loss) <= 10 * tol["loss"]
            # dW on sampled candidate rows: ends, random, and the most frequent targets
            top = np.bincount(tpos[tpos >= 0], minlength=P_eff).argsort()[-8:]
            js = np.unique(np.concatenate([[0, P_eff - 1], rng.integers(0, P_eff, 22), top]))
            ref = ce_c.dwc_rows(xf, Wf, Cc, L, tpos, ppos, N, js)
            cls = js if w.P == 0 else cand["C"][js]
            gW_rows = to_f64(out["dW"][torch.from_numpy(cls).cuda()])
            # each sampled row against its own magnitude (every one of them: floor 0)
            worst, _ = max_row_rel(gW_rows, ref, floor=0.0)
            print(f"  dW rows max-rel {max_rel(gW_rows, ref):.2e}, worst row {worst:.2e}", flush=True)
            assert max_rel(gW_rows, ref) <= tol["grad"], max_rel(gW_rows, ref)
            assert worst <= tol["grad"], worst
            L_rows = L
        else:
            L_rows[rows] = ce_c.lse_rows(xf, Wf, Cc, rows)
            np.testing.assert_allclose(gl[rows], L_rows[rows], rtol=tol["loss"], atol=0)
        ref = ce_c.dx_rows(xf, Wf, Cc, L_rows, tpos, ppos, N, rows)
        gX_rows = to_f64(out["dX"][torch.from_numpy(rows).cuda()])
        worst, _ = max_row_rel(gX_rows, ref, floor=0.0)
        print(f"  dX rows max-rel {max_rel(gX_rows, ref):.2e}, worst row {worst:.2e}", flush=True)
        assert max_rel(gX_rows, ref) <= tol["grad"], max_rel(gX_rows, ref)
        assert worst <= tol["grad"], worst
        if w.P > 0:
            outside = np.setdiff1d(np.arange(w.V), cand["C"])
            raw = out["dW"].view(torch.int16 if w.dtype == "bf16" else torch.int32).cpu().numpy()
            assert (raw[outside] == 0).all()
        del out
        torch.cuda.empty_cache()
    if w.calls > 1:
        # a class is drawn as a negative at most as often as a window covered it
        assert (neg_hits <= win_hits).all()


def test_dx_split_sampled():
    """A shape whose dX product is split along k (260 tiles of 256 x 192 on the chip's
    256 compute units, so four splits reduced in fp32): sampled rows of dX, their L_t
    and loss terms against the oracle, the candidate set exactly."""
    T, d, V, P, stride, off = 16640, 768, 12000, 4608, 7919, 123
    print(f"dx split: T={T} d={d} V={V} P={P} bf16", flush=True)
    x, W, y, p = synth.small_case(11, T, d, V, "bf16", prefix=True, ignore_frac=0.02)
    out = binding.forward_backward(to_dev(x, "bf16"), to_dev(W, "bf16"), labels_dev(y), labels_dev(p),
                                   P, stride, off, want_rows=True)
    torch.cuda.synchronize()
    cand = build_candidates(V, P, stride, off, y, p)
    assert np.array_equal(out["C"].cpu().numpy(), cand["C"])
    xf, Wf = inputs_f64(x, W, "bf16")
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([[0, 255, 256, T - 257, T - 1], rng.integers(0, T, 27)]))
    L = np.zeros(T)
    L[rows] = ce_c.lse_rows(xf, Wf, cand["C"], rows)
    tol = TOL["bf16"]
    np.testing.assert_allclose(to_f64(out["row_lse"])[rows], L[rows], rtol=tol["loss"], atol=0)
    ref = ce_c.dx_rows(xf, Wf, cand["C"], L, cand["target_pos"], cand["prefix_pos"], cand["N"], rows)
    got = to_f64(out["dX"][torch.from_numpy(rows).cuda()])
    assert max_rel(got, ref) <= tol["grad"], max_rel(got, ref)
    assert max_row_rel(got, ref, floor=0.0)[0] <= tol["grad"]
