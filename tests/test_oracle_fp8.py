"""Pins of the fp8 (e4m3) oracle against references that do not share its code:
torch's float8_e4m3fn and bfloat16 conversions (library routines), values fixed by
the format's definition, and a pure-Python brute force of the whole step on tiny
inputs (exhaustive nearest-code search, exact rational rounding, scalar loops)."""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import fp8

# ---------------------------------------------------------------------------
# e4m3 codec
# ---------------------------------------------------------------------------


def test_decode_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = fp8.e4m3_decode(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    assert np.array_equal(np.signbit(ref[ok]), np.signbit(got[ok]))


def test_encode_matches_torch():
    rng = np.random.default_rng(1)
    finite = np.unique(fp8.e4m3_decode(np.arange(256, dtype=np.uint8)))
    finite = finite[np.isfinite(finite)]
    mids = ((finite[1:] + finite[:-1]) / 2).astype(np.float32)  # every tie
    v = np.concatenate([
        rng.uniform(-448, 448, 50000), rng.uniform(-0.05, 0.05, 50000),
        rng.standard_normal(50000) * 3, finite]).astype(np.float32)
    v = np.concatenate([v, mids, np.nextafter(mids, np.float32(1e9)), np.nextafter(mids, np.float32(-1e9))])
    v = v[np.abs(v) <= 448]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(fp8.e4m3_encode(v.astype(np.float64)), ref)


def test_codec_values_fixed_by_the_format():
    dec = lambda c: float(fp8.e4m3_decode(np.uint8(c)))
    assert dec(0x7E) == 448.0 and dec(0xFE) == -448.0          # largest finite
    assert dec(0x08) == 2.0 ** -6 and dec(0x01) == 2.0 ** -9   # min normal, min subnormal
    assert dec(0x38) == 1.0 and dec(0x3F) == 1.875
    assert math.isnan(dec(0x7F)) and math.isnan(dec(0xFF))
    enc = lambda v: int(fp8.e4m3_encode(np.float64(v)))
    assert enc(1.0) == 0x38 and enc(-2.0) == 0xC0 and enc(448.0) == 0x7E
    assert enc(1.0625) == 0x38          # halfway 1 | 1.125 -> even mantissa (1)
    assert enc(1.1875) == 0x3A          # halfway 1.125 | 1.25 -> 1.25
    assert enc(2.0 ** -10) == 0x00      # halfway 0 | 2^-9 -> 0
    assert enc(3 * 2.0 ** -10) == 0x02  # halfway 2^-9 | 2^-8 -> 2^-8
    assert enc(-1e-5) == 0x80           # rounds to -0, sign kept
    for c in range(256):                # every finite code is its own encoding
        if (c & 0x7F) != 0x7F:
            assert enc(dec(c)) == c or (c == 0x80 and enc(dec(c)) == 0x80)
    with pytest.raises(ValueError):
        fp8.e4m3_encode(np.float64(464.0 + 1))


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(2)
    v = np.concatenate([rng.standard_normal(100000) * 10, rng.uniform(-1e-3, 1e-3, 10000)]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(fp8.bf16_round(v.astype(np.float64)), ref)


def test_scale_rules():
    # smallest power of two s with amax <= 448 s
    assert fp8.pow2_scale(448.0) == 1.0
    assert fp8.pow2_scale(np.nextafter(448.0, 1e9)) == 2.0
    assert fp8.pow2_scale(1.0) == 2.0 ** -8        # 448 / 256 = 1.75 >= 1 > 0.875
    assert fp8.pow2_scale(1.75) == 2.0 ** -8
    assert fp8.pow2_scale(1.7500001) == 2.0 ** -7
    assert fp8.pow2_scale(0.0) == 1.0
    assert fp8.pow2_scale(5.25) == 2.0 ** -6       # 448 / 64 = 7 >= 5.25 > 3.5
    # smallest power of two s with n_max / N <= 448 s
    assert fp8.grad_scale(16384, 1) == 2.0 ** -22  # 2^-14 <= 448 * 2^-22 = 1.07e-4
    assert fp8.grad_scale(1, 2) == 2.0 ** -7       # 2 <= 448 / 128 = 3.5, > 1.75
    assert fp8.grad_scale(0, 1) == 1.0
    for N in (1, 3, 7, 100, 98304):
        for n in (1, 2):
            s = fp8.grad_scale(N, n)
            assert n / N <= 448 * s and n / N > 224 * s


# ---------------------------------------------------------------------------
# Whole step: brute force on tiny inputs
# ---------------------------------------------------------------------------

def _bf_decode(c):
    s, e, m = c >> 7, (c >> 3) & 15, c & 7
    v = math.ldexp(m, -9) if e == 0 else math.ldexp(8 + m, e - 10)
    return -v if s else v


_BF_CODES = [c for c in range(256) if (c & 0x7F) != 0x7F]


def _bf_encode(v):
    """Nearest finite code by exhaustive search; ties to the even code; sign kept."""
    best, bd = None, None
    for c in _BF_CODES:
        dv = abs(_bf_decode(c) - v)
        if best is None or dv < bd or (dv == bd and c % 2 == 0 and best % 2 == 1):
            best, bd = c, dv
    if _bf_decode(best) == 0.0:
        best = 0x80 if v < 0 or (v == 0 and math.copysign(1.0, v) < 0) else 0x00
    return best


def _bf_bf16(v):
    """Nearest bfloat16 of a float by exact rational arithmetic, ties to even."""
    if v == 0.0:
        return 0.0
    fv = Fraction(v)
    a = abs(fv)
    e = 0
    while a >= 2:
        a /= 2
        e += 1
    while a < 1:
        a *= 2
        e -= 1
    step = Fraction(2) ** (e - 7)                   # 8 significant bits
    lo = (abs(fv) // step) * step
    hi = lo + step
    dl, dh = abs(fv) - lo, hi - abs(fv)
    q = lo if dl < dh or (dl == dh and (lo / step) % 2 == 0) else hi
    return float(q) if v > 0 else -float(q)


def _bf_pow2(amax):
    for k in range(-60, 60):
        if amax <= 448.0 * 2.0 ** k:
            return 2.0 ** k


def _bf_step(x, W8, w_scale, C, tpos, ppos):
    T, d = len(x), len(x[0])
    P = len(C)
    WC = [[_bf_decode(int(W8[c][k])) for k in range(d)] for c in C]
    s_x = _bf_pow2(max(abs(v) for row in x for v in row)) if T else 1.0
    x8 = [[_bf_encode(v / s_x) for v in row] for row in x]
    xv = [[_bf_decode(c) for c in row] for row in x8]
    z = [[_bf_bf16(s_x * w_scale * sum(xv[t][k] * WC[j][k] for k in range(d))) for j in range(P)]
         for t in range(T)]
    N = sum(int(tpos[t] >= 0) + int(ppos is not None and ppos[t] >= 0) for t in range(T))
    n_max = 2 if ppos is not None else 1
    s_g = next(2.0 ** -k for k in range(200, -1, -1) if n_max / N <= 448.0 * 2.0 ** -k) if N else 1.0
    loss = 0.0
    g8 = [[0] * P for _ in range(T)]
    for t in range(T):
        m = max(z[t])
        L = m + math.log(sum(math.exp(v - m) for v in z[t]))
        labels = [p for p in (tpos[t], ppos[t] if ppos is not None else -1) if p >= 0]
        for p in labels:
            loss += L - z[t][p]
        for j in range(P):
            g = (len(labels) * math.exp(z[t][j] - L) - sum(1 for p in labels if p == j)) / N if N else 0.0
            g8[t][j] = _bf_encode(g / s_g)
    gv = [[_bf_decode(c) for c in row] for row in g8]
    dX = [[s_g * w_scale * sum(gv[t][j] * WC[j][k] for j in range(P)) for k in range(d)] for t in range(T)]
    dWC = [[s_g * s_x * sum(gv[t][j] * xv[t][k] for t in range(T)) for k in range(d)] for j in range(P)]
    return dict(loss=loss / N if N else 0.0, z=np.array(z), x8=np.array(x8, dtype=np.uint8),
                g8=np.array(g8, dtype=np.uint8), dX=np.array(dX), dWC=np.array(dWC), s_x=s_x, s_g=s_g)


def _tiny(seed, T, d, V, P, with_prefix, full):
    rng = np.random.default_rng(seed)
    x = torch.from_numpy(rng.standard_normal((T, d)) * 1.7).to(torch.bfloat16).to(torch.float64).numpy()
    W8 = rng.choice(np.array(_BF_CODES, dtype=np.uint8), size=(V, d))
    w_scale = float(np.float32(0.0123))
    C = np.arange(V) if full else np.sort(rng.choice(V, size=P, replace=False))
    P = len(C)
    tpos = rng.integers(-1, P, size=T)
    ppos = rng.integers(-1, P, size=T) if with_prefix else None
    if with_prefix:
        ppos[0] = tpos[0] = 2               # a duplicated label: coefficient -2
    return x, W8, w_scale, C, tpos, ppos


@pytest.mark.parametrize("case", [
    dict(seed=3, T=7, d=16, V=20, P=9, with_prefix=True, full=False),
    dict(seed=4, T=5, d=8, V=11, P=11, with_prefix=False, full=True),
    dict(seed=5, T=6, d=24, V=30, P=4, with_prefix=True, full=False),
])
def test_step_matches_brute_force(case):
    x, W8, w_scale, C, tpos, ppos = _tiny(**case)
    ref = _bf_step(x.tolist(), W8, w_scale, list(C), list(tpos), None if ppos is None else list(ppos))
    got = fp8.forward_backward(x, W8, w_scale, None if case["full"] else C, tpos, ppos)
    assert got["s_x"] == ref["s_x"] and got["s_g"] == ref["s_g"]
    assert np.array_equal(got["x8"], ref["x8"])
    assert np.array_equal(got["z"], ref["z"])
    assert np.array_equal(got["g8"], ref["g8"])
    assert got["loss"] == pytest.approx(ref["loss"], rel=1e-13, abs=1e-15)
    np.testing.assert_allclose(got["dX"], ref["dX"], rtol=1e-13, atol=1e-18)
    np.testing.assert_allclose(got["dW"][C], ref["dWC"], rtol=1e-13, atol=1e-18)
    outside = np.ones(len(W8), bool)
    outside[C] = False
    assert not got["dW"][outside].any()


def test_row_helpers_agree_with_dense():
    x, W8, w_scale, C, tpos, ppos = _tiny(seed=6, T=40, d=32, V=90, P=37, with_prefix=True, full=False)
    dense = fp8.forward_backward(x, W8, w_scale, C, tpos, ppos)
    WCv = fp8.e4m3_decode(W8[C])
    xv = fp8.e4m3_decode(dense["x8"])
    s_xw = dense["s_x"] * float(np.float32(w_scale))
    L = fp8.lse_rows(xv, WCv, s_xw)
    np.testing.assert_allclose(L, dense["L"], rtol=1e-14)
    rows = np.array([0, 5, 39])
    np.testing.assert_allclose(
        fp8.dx_rows(xv, WCv, s_xw, L, tpos, ppos, dense["N"], dense["s_g"], w_scale, rows),
        dense["dX"][rows], rtol=1e-13, atol=1e-18)
    cols = np.array([0, 17, 36])
    np.testing.assert_allclose(
        fp8.dwc_rows(xv, WCv, s_xw, L, tpos, ppos, dense["N"], dense["s_g"], dense["s_x"], cols),
        dense["dW"][C[cols]], rtol=1e-13, atol=1e-18)


def test_full_size_helpers_run_every_block_loop_twice():
    """fp8.lse_rows (2048-row blocks) and fp8.dwc_rows (8192-token blocks), and the
    full-size bounds (fp8_tol.sampled_bounds, 2048-row blocks) against their dense forms
    (fp8.forward_backward, fp8_tol.step_bounds) at T = 9000, where every loop runs
    more than once."""
    from tests import fp8_tol

    x, W8, w_scale, C, tpos, ppos = _tiny(seed=22, T=9000, d=32, V=700, P=320, with_prefix=True,
                                          full=False)
    dense = fp8.forward_backward(x, W8, w_scale, C, tpos, ppos)
    WCv = fp8.e4m3_decode(W8[C])
    xv = fp8.e4m3_decode(dense["x8"])
    s_xw = dense["s_x"] * float(np.float32(w_scale))
    L = fp8.lse_rows(xv, WCv, s_xw)
    np.testing.assert_allclose(L, dense["L"], rtol=1e-14)
    cols = np.arange(0, 320, 3)
    np.testing.assert_allclose(
        fp8.dwc_rows(xv, WCv, s_xw, L, tpos, ppos, dense["N"], dense["s_g"], dense["s_x"], cols),
        dense["dW"][C[cols]], rtol=1e-13, atol=1e-18)
    rows = np.array([0, 2047, 2048, 8191, 8192, 8999])
    np.testing.assert_allclose(
        fp8.dx_rows(xv, WCv, s_xw, L, tpos, ppos, dense["N"], dense["s_g"], w_scale, rows),
        dense["dX"][rows], rtol=1e-13, atol=1e-18)
    full = fp8_tol.step_bounds(dense, dense["x8"], W8[C], w_scale, C, tpos, ppos)
    samp = fp8_tol.sampled_bounds(dense["x8"], W8[C], w_scale, dense["s_x"], dense["s_g"], dense["N"],
                                  tpos, ppos, dense["L"], rows, cols, dense["dX"][rows],
                                  dense["dW"][C[cols]], dense["row_loss"], dense["loss"])
    np.testing.assert_allclose(samp["row_lse"], full["row_lse"], rtol=1e-12, atol=0)
    np.testing.assert_allclose(samp["dX"], full["dX"][rows], rtol=1e-12, atol=0)
    np.testing.assert_allclose(samp["dWC"], full["dWC"][cols], rtol=1e-12, atol=0)
    assert samp["loss"] == pytest.approx(full["loss"], rel=1e-12)
    assert full["dX"].min() > 0 and full["dWC"].min() > 0 and full["loss"] > 0


# ---------------------------------------------------------------------------
# The e4m3 lm_head cache (scale max|W| / 448, codes of the float32 quotient)
# ---------------------------------------------------------------------------

def _bf_f32_quotient(a, b):
    """Nearest float32 (normal range) of the exact rational a / b, ties to even."""
    q = Fraction(a) / Fraction(b)
    if q == 0:
        return 0.0
    m = abs(q)
    e = 0
    while m >= 2:
        m /= 2
        e += 1
    while m < 1:
        m *= 2
        e -= 1
    step = Fraction(2) ** (e - 23)                  # 24 significant bits
    lo = (abs(q) // step) * step
    hi = lo + step
    dl, dh = abs(q) - lo, hi - abs(q)
    r = lo if dl < dh or (dl == dh and (lo / step) % 2 == 0) else hi
    return float(r) if q > 0 else -float(r)


def _bf16_values(seed, shape, scale):
    v = np.random.default_rng(seed).standard_normal(shape) * scale
    return torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def test_cache_matches_torch_cast():
    """Scale and codes against torch: float32 max / 448 and the float8_e4m3fn cast of the
    float32 quotient, all in torch's float32 arithmetic."""
    for seed, shape, sc in ((3, (513, 64), 0.02), (4, (97, 48), 3.0), (5, (64, 16), 1e-3)):
        W = _bf16_values(seed, shape, sc)
        Wt = torch.from_numpy(W.astype(np.float32))
        s_ref = (Wt.abs().max() / torch.tensor(448.0, dtype=torch.float32)).item()
        codes_ref = (Wt / torch.tensor(s_ref, dtype=torch.float32)).to(torch.float8_e4m3fn)
        codes, s = fp8.e4m3_cache(W)
        assert s == s_ref
        assert np.array_equal(codes, codes_ref.view(torch.uint8).numpy())


def test_cache_brute_force():
    """Tiny tensors: the scale by exact rational rounding to float32, each code by
    exhaustive nearest-code search over the exactly rounded float32 quotient."""
    for seed in range(4):
        W = _bf16_values(10 + seed, (5, 16), 10.0 ** (seed - 2))
        amax = float(np.abs(W).max())
        s = _bf_f32_quotient(amax, 448)
        codes, s_o = fp8.e4m3_cache(W)
        assert s_o == s
        ref = np.array([[_bf_encode(_bf_f32_quotient(v, s)) for v in row] for row in W], np.uint8)
        assert np.array_equal(codes, ref)


def test_cache_values_fixed_by_the_definition():
    # all zeros: scale 1, every code +0
    codes, s = fp8.e4m3_cache(np.zeros((4, 16)))
    assert s == 1.0 and not codes.any()
    # the largest magnitude lands on +-448 (0x7e / 0xfe) whatever its value
    W = _bf16_values(20, (33, 32), 0.7)
    i = np.unravel_index(np.abs(W).argmax(), W.shape)
    codes, s = fp8.e4m3_cache(W)
    assert codes[i] == (0xFE if W[i] < 0 else 0x7E)
    assert np.all(np.abs(fp8.e4m3_decode(codes)) <= 448)
    # values that are e4m3 values times 2^k, with 448 2^k present, come back unchanged
    rng = np.random.default_rng(21)
    c = rng.choice([c for c in range(256) if (c & 0x7F) != 0x7F], size=(16, 32)).astype(np.uint8)
    c[3, 5] = 0xFE
    for k in (-12, 0, 7):
        codes, s = fp8.e4m3_cache(fp8.e4m3_decode(c) * 2.0 ** k)
        assert s == 2.0 ** k and np.array_equal(codes, c)
    # error bound: |s_w decode(code) - W| <= half an e4m3 step of W / s_w, times s_w
    W = _bf16_values(22, (64, 64), 0.05)
    codes, s = fp8.e4m3_cache(W)
    q = np.abs(W / s)
    step = np.where(q >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(q, 1e-300))) - 3), 2.0 ** -9)
    assert np.all(np.abs(fp8.e4m3_decode(codes) * s - W) <= 0.5 * step * s * (1 + 2.0 ** -20))
