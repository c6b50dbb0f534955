"""The step's building blocks through their own C entry points: the fused CE
forward/backward over caller-given logits (against the oracle's dense evaluation) and
the row gather (bit for bit against numpy indexing)."""
import numpy as np
import pytest
import torch

from oracle import ce
from sampled_softmax_cross_amd import binding, synth
from tests.gpu_util import TOL, max_rel, to_f64

pytestmark = pytest.mark.gpu

CE_CASES = [
    # T, P, ldz, dtype, prefix, ignore_frac
    (300, 333, 336, "bf16", True, 0.05),
    (300, 333, 400, "f32", True, 0.0),
    (129, 2048, 2048, "bf16", False, 0.2),
    (64, 8, 8, "f32", True, 0.0),
    # either side of the row-shape choice: 256 lanes while 40 values each, then 512
    # lanes with the values kept, then 512 lanes evaluating the exponential twice
    (40, 10248, 10248, "bf16", True, 0.0),      # 1281 vectors: 512 lanes, kept
    (24, 20488, 20488, "bf16", False, 0.1),     # 2561 vectors: 512 lanes, evaluated twice
    (32, 9000, 9000, "f32", True, 0.0),         # 2250 vectors: 256 lanes x 9, kept
    (24, 20488, 20488, "f32", False, 0.0),      # 5122 vectors: 512 lanes x 11, evaluated twice
    (17, 50304, 50304, "bf16", True, 0.0),      # a row of the full vocabulary
    (3, 140000, 140000, "bf16", False, 0.0),    # rows beyond what registers hold
]


def _labels(seed, T, P, frac):
    r = np.random.default_rng(seed)
    y = r.integers(0, P, T).astype(np.int32)
    y[r.random(T) < frac] = -1
    return y


@pytest.mark.parametrize("T,P,ldz,dtype,prefix,frac", CE_CASES)
def test_ce_rows_matches_oracle(T, P, ldz, dtype, prefix, frac):
    print(f"ce_rows T={T} P={P} ldz={ldz} {dtype}", flush=True)
    z = synth.normal(T + P, 7, (T, P), 2.0, dtype)          # logits, rounded to the dtype
    tp = _labels(T, T, P, frac)
    pp = _labels(T + 1, T, P, frac) if prefix else None
    zf = synth.to_f64(z, dtype)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    Z = torch.zeros(T, ldz, dtype=tdt, device="cuda")
    Z[:, :P] = torch.from_numpy(zf).to(tdt).cuda()
    out = binding.ce_rows(Z, P, torch.from_numpy(tp).cuda(),
                          None if pp is None else torch.from_numpy(pp).cuda(), want_rows=True)
    torch.cuda.synchronize()
    loss, g, L, row_loss, _ = ce.ce_rows(zf, tp, pp)
    tol = TOL[dtype]
    got = to_f64(Z)
    assert max_rel(got[:, :P], g) <= tol["grad"], max_rel(got[:, :P], g)
    assert (got[:, P:] == 0).all()
    assert abs(out["loss"].item() - loss) <= tol["loss"] * max(abs(loss), 1e-30)
    np.testing.assert_allclose(to_f64(out["row_lse"])[:T], L, rtol=tol["loss"], atol=0)
    assert max_rel(to_f64(out["row_loss"])[:T], row_loss) <= 10 * tol["loss"]
    assert out["aux"].cpu().tolist() == [0, ce.num_labels(tp, pp), 0, 0]


def test_ce_rows_label_range_flag():
    T, P = 40, 64
    Z = torch.randn(T, P, device="cuda")
    tp = torch.full((T,), 3, dtype=torch.int32, device="cuda")
    tp[5] = P          # out of range: flagged, treated as no label
    tp[6] = -2
    out = binding.ce_rows(Z, P, tp)
    torch.cuda.synchronize()
    aux = out["aux"].cpu().tolist()
    assert aux[1] == T - 2 and aux[3] == binding.DEV_LABEL_RANGE
    assert torch.isfinite(Z).all()


def test_ce_rows_no_labels():
    Z = torch.randn(10, 16, device="cuda")
    out = binding.ce_rows(Z, 16, torch.full((10,), -1, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert out["loss"].item() == 0.0 and (Z == 0).all()


@pytest.mark.parametrize("V,d,n,ld,dtype", [(1000, 64, 777, 64, "bf16"), (4096, 4096, 512, 4096, "bf16"),
                                            (300, 136, 1000, 200, "f32"), (50, 8, 0, 8, "bf16")])
def test_gather_rows_bitwise(V, d, n, ld, dtype):
    print(f"gather V={V} d={d} n={n} ld={ld} {dtype}", flush=True)
    w = synth.normal(V + d, 3, (V, d), 1.0, dtype)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    W = torch.from_numpy(synth.to_f64(w, dtype)).to(tdt).cuda()
    idx = np.random.default_rng(n).integers(0, V, n).astype(np.int32)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = torch.full((n, ld), 7.0, dtype=tdt, device="cuda")
    binding.gather_rows(W, torch.from_numpy(idx).cuda(), out=out, status=status)
    torch.cuda.synchronize()
    ref = W.cpu()[torch.from_numpy(idx).long()]
    assert torch.equal(out[:, :d].cpu(), ref)
    assert (out[:, d:].cpu() == 7.0).all()           # padding columns untouched
    assert status.item() == 0


def test_gather_rows_out_of_range():
    W = torch.randn(20, 16, device="cuda").to(torch.bfloat16)
    idx = torch.tensor([0, 19, 20, -1, 5], dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = binding.gather_rows(W, idx, status=status)
    torch.cuda.synchronize()
    assert torch.equal(out[[0, 1, 4]], W[[0, 19, 5]])
    assert (out[[2, 3]] == 0).all() and status.item() == binding.DEV_LABEL_RANGE
