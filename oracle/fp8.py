"""fp8 (e4m3) operand variant of the step in float64 numpy -- TEST INFRASTRUCTURE ONLY.

"sampled_softmax.py" keeps the lm_head as an fp8 cache: the candidate rows it gathers
(and their transposed copy, the backward's operand) are float8_e4m3fn tensors, and
the products are scaled fp8 matrix products. The page does not state the scaling
rules or which other operands are fp8. The readings implemented here:

* e4m3 is the OCP 8-bit format E4M3 (torch's float8_e4m3fn): sign bit, 4 exponent
  bits with bias 7, 3 mantissa bits, subnormals below 2^-6, no infinities, the
  all-ones magnitude (0x7f) is NaN, largest finite magnitude 448. Encoding rounds to
  nearest, ties to even.
* W is given as e4m3 codes with one float32 dequantisation scale for the tensor
  (W ~ w_scale * W8); gathering candidate rows copies their bytes.
* x is quantised per tensor: s_x is the smallest power of two with
  max|x| <= 448 s_x, and x8 = e4m3(x / s_x) (a power-of-two scale keeps x / s_x
  exact, so the encoding is the only rounding).
* logits z = bf16(s_x w_scale (x8 . W8_C)): a scaled fp8 product with a bf16
  result, rounded to nearest even; the cross-entropy then acts on these bf16
  logits as in the bf16 step (oracle.ce.ce_rows).
* the logit gradient g is quantised per tensor with a scale fixed before it is
  computed: every |g[t, j]| <= n_t / N <= n_max / N (n_max = 2 when prefix targets
  are given, else 1), so s_g is the smallest power of two with n_max / N <= 448 s_g
  and g8 = e4m3(g / s_g) never overflows;
* dX = s_g w_scale (g8 . W8_C) and dW_C = s_g s_x (g8^T . x8), both fp8 products;
  the dense dW holds dW_C in the rows of C and zeros elsewhere, as in the bf16 step.

Matrix products are numpy float64 matmuls of the decoded values (exact: every
e4m3 product has at most 8 significant bits and the sums stay far inside float64's
53). Nothing else is blocked, fused or reordered.
"""
import numpy as np

from . import ce as _ce

E4M3_MAX = 448.0
_MIN_NORMAL = 2.0 ** -6
_SUB_STEP = 2.0 ** -9  # spacing of the subnormals (and of the first binade)


def _decode_table():
    t = np.empty(256)
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            v = np.nan
        elif e == 0:
            v = m * _SUB_STEP
        else:
            v = (1.0 + m / 8.0) * 2.0 ** (e - 7)
        t[c] = -v if s else v
    return t


_TABLE = _decode_table()


def e4m3_decode(codes):
    """Values (float64) of e4m3 codes (uint8)."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(v):
    """Nearest e4m3 code of each finite value with |v| <= 448 + half a step; ties go to
    the even mantissa. The sign is kept (a tiny negative value encodes as -0)."""
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("e4m3_encode: non-finite input")
    a = np.abs(v)
    # normal: a = f * 2^e with f in [0.5, 1); the binade [2^(e-1), 2^e) holds 8 steps of 2^(e-4)
    f, e = np.frexp(a)
    normal = a >= _MIN_NORMAL
    step = np.where(normal, np.ldexp(1.0, e - 4), _SUB_STEP)
    q = np.rint(a / step) * step                    # exact: a / step is a power-of-two rescaling
    if np.any(q > E4M3_MAX):
        raise ValueError("e4m3_encode: value beyond 448")
    # code of q: exponent field and mantissa field from q's own binade
    fq, eq = np.frexp(q)
    qn = q >= _MIN_NORMAL
    exp_field = np.where(qn, eq - 1 + 7, 0)
    man_field = np.where(qn, np.rint((fq * 2.0 - 1.0) * 8.0), np.rint(q / _SUB_STEP))
    codes = (exp_field.astype(np.int64) << 3) | man_field.astype(np.int64)
    codes = codes | (np.signbit(v).astype(np.int64) << 7)
    return codes.astype(np.uint8)


def bf16_round(v):
    """v rounded to the nearest bfloat16 (8 significant bits), ties to even, as float64."""
    v = np.asarray(v, dtype=np.float64)
    f, e = np.frexp(v)                              # |f| in [0.5, 1)
    sub = np.abs(v) < 2.0 ** -126
    step = np.where(sub, 2.0 ** -133, np.ldexp(1.0, e - 8))
    return np.rint(v / step) * step


def pow2_scale(amax):
    """Smallest power of two s with amax <= 448 s (1.0 when amax == 0)."""
    a = float(amax)
    if a == 0.0:
        return 1.0
    f, e = np.frexp(a)                              # a = f 2^e, f in [0.5, 1)
    s = float(np.ldexp(1.0, int(e) - 9))            # 448 * 2^(e-9) = 0.875 * 2^e: just below or at a
    while a > E4M3_MAX * s:
        s *= 2.0
    while a <= E4M3_MAX * s / 2.0:
        s /= 2.0
    return s


def grad_scale(N, n_max):
    """Smallest power of two s with n_max / N <= 448 s (1.0 when N == 0). With
    n_max <= 2 <= 448 N it is 2^-k for the largest k with n_max 2^k <= 448 N, found in
    integers."""
    N, n_max = int(N), int(n_max)
    if N == 0:
        return 1.0
    k = 0
    while n_max << (k + 1) <= 448 * N:
        k += 1
    return 2.0 ** -k


def quantize_x(x):
    """(x8 codes, s_x) for the per-tensor quantisation of x (float64 values)."""
    x = np.asarray(x, dtype=np.float64)
    s = pow2_scale(np.abs(x).max() if x.size else 0.0)
    return e4m3_encode(x / s), s


def cache_scale(amax):
    """The e4m3 cache's scale for a weight tensor whose largest magnitude is amax (a
    float32 value): float32(amax / 448), the largest magnitude landing on e4m3's largest
    finite value; 1.0 when amax == 0. The float64 quotient rounded to float32 is the
    correctly rounded float32 quotient (double rounding of a quotient through a format
    with at least 2p + 2 bits, 53 >= 2 * 24 + 2, is innocuous: Figueroa, "When is double
    rounding innocuous?", SIGNUM Newsletter 1995)."""
    s = np.float32(np.float64(np.float32(amax)) / E4M3_MAX)
    return 1.0 if s == 0 else float(s)


def e4m3_cache(W):
    """The lm_head's e4m3 cache ("sampled_softmax.py" keeps the weights as a float8_e4m3fn
    copy, refreshed before the candidate rows are gathered; the page does not give the
    encoding, the reading here is one per-tensor scale): W [V, d] float64 values (exact
    widenings of bf16 or float32 weights). Returns (codes uint8 [V, d], s_w) with
    s_w = cache_scale(max|W|) and codes = e4m3 of the float32 quotient W / s_w (the
    correctly rounded float32 division, by the same double-rounding argument)."""
    W = np.asarray(W, dtype=np.float64)
    s_w = cache_scale(np.abs(W).max() if W.size else 0.0)
    q = (W / s_w).astype(np.float32).astype(np.float64)
    return e4m3_encode(q), s_w


def forward_backward(x, W8, w_scale, C, target_pos, prefix_pos=None):
    """Dense fp8 oracle. x [T,d] float64 (exact widening of the bf16 input), W8 [V,d]
    e4m3 codes, w_scale the float32 dequantisation scale, C the candidate classes
    (None: full softmax). Returns a dict: loss, dX [T,d], dW [V,d], L, row_loss,
    z (bf16 logits), s_x, s_g, x8, g8, N, and the values before their roundings:
    z_exact (the scaled product) and g_scaled (g / s_g)."""
    x = np.asarray(x, dtype=np.float64)
    T, d = x.shape
    W8 = np.asarray(W8, dtype=np.uint8)
    V = W8.shape[0]
    w_scale = float(np.float32(w_scale))
    W8C = W8 if C is None else W8[np.asarray(C, dtype=np.int64)]
    WCv = e4m3_decode(W8C)
    x8, s_x = quantize_x(x) if T else (np.zeros((0, d), np.uint8), 1.0)
    xv = e4m3_decode(x8)
    z_exact = (s_x * w_scale) * (xv @ WCv.T)
    z = bf16_round(z_exact)
    loss, g, L, row_loss, N = _ce.ce_rows(z, target_pos, prefix_pos)
    n_max = 2 if prefix_pos is not None else 1
    s_g = grad_scale(N, n_max)
    g8 = e4m3_encode(g / s_g) if T else np.zeros((0, W8C.shape[0]), np.uint8)
    gv = e4m3_decode(g8)
    dX = (s_g * w_scale) * (gv @ WCv)
    dWC = (s_g * s_x) * (gv.T @ xv)
    dW = np.zeros((V, d))
    if C is None:
        dW[:] = dWC
    else:
        dW[np.asarray(C, dtype=np.int64)] = dWC
    return dict(loss=loss, dX=dX, dW=dW, L=L, row_loss=row_loss, z=z, s_x=s_x, s_g=s_g,
                x8=x8, g8=g8, N=N, z_exact=z_exact, g_scaled=g / s_g)


# ---------------------------------------------------------------------------
# Row-by-row evaluation of the same definition, for full-size shapes.
# ---------------------------------------------------------------------------

def logits_rows(xv, WCv, s_xw, rows):
    """bf16 logits of the given rows: xv, WCv decoded operands, s_xw = s_x w_scale."""
    return bf16_round(s_xw * (xv[np.asarray(rows, dtype=np.int64)] @ WCv.T))


def lse_rows(xv, WCv, s_xw, block=2048):
    """L[t] of every row from the bf16 logits."""
    T = xv.shape[0]
    out = np.empty(T)
    for s in range(0, T, block):
        out[s:s + block] = _ce.logsumexp_rows(logits_rows(xv, WCv, s_xw, np.arange(s, min(T, s + block))))
    return out


def label_logits(xv, WCv, s_xw, pos):
    """bf16 logit z[t, pos[t]] for every t with pos[t] >= 0 (0 elsewhere)."""
    pos = np.asarray(pos, dtype=np.int64)
    out = np.zeros(pos.shape[0])
    ok = pos >= 0
    out[ok] = bf16_round(s_xw * np.einsum("td,td->t", xv[ok], WCv[pos[ok]]))
    return out


def loss_from_lse(xv, WCv, s_xw, L, target_pos, prefix_pos=None):
    """(loss, row_loss, N) given every row's L: the label terms L - z over the bf16 logits."""
    tpos = np.asarray(target_pos, dtype=np.int64)
    row_loss = np.where(tpos >= 0, L - label_logits(xv, WCv, s_xw, tpos), 0.0)
    N = int((tpos >= 0).sum())
    if prefix_pos is not None:
        ppos = np.asarray(prefix_pos, dtype=np.int64)
        row_loss = row_loss + np.where(ppos >= 0, L - label_logits(xv, WCv, s_xw, ppos), 0.0)
        N += int((ppos >= 0).sum())
    return (float(row_loss.sum() / N) if N else 0.0), row_loss, N


def g8_rows(z, L, tpos, ppos, N, s_g):
    """e4m3 codes of g / s_g for rows whose bf16 logits z and row log-sum-exp L are given."""
    tpos = np.asarray(tpos, dtype=np.int64)
    n = (tpos >= 0).astype(np.int64)
    if ppos is not None:
        ppos = np.asarray(ppos, dtype=np.int64)
        n = n + (ppos >= 0)
    g = n[:, None] * np.exp(z - L[:, None])
    i = np.arange(z.shape[0])
    np.add.at(g, (i[tpos >= 0], tpos[tpos >= 0]), -1.0)
    if ppos is not None:
        np.add.at(g, (i[ppos >= 0], ppos[ppos >= 0]), -1.0)
    return e4m3_encode((g / N) / s_g) if N else np.zeros(z.shape, np.uint8)


def dx_rows(xv, WCv, s_xw, L, target_pos, prefix_pos, N, s_g, w_scale, rows):
    """dX[t] of the given rows."""
    rows = np.asarray(rows, dtype=np.int64)
    z = logits_rows(xv, WCv, s_xw, rows)
    tp = np.asarray(target_pos)[rows]
    pp = None if prefix_pos is None else np.asarray(prefix_pos)[rows]
    g8 = g8_rows(z, L[rows], tp, pp, N, s_g)
    return (s_g * float(np.float32(w_scale))) * (e4m3_decode(g8) @ WCv)


def dwc_rows(xv, WCv, s_xw, L, target_pos, prefix_pos, N, s_g, s_x, cand_rows, block=8192):
    """dW_C[j] of the given candidate positions (sum over every token)."""
    cand_rows = np.asarray(cand_rows, dtype=np.int64)
    T = xv.shape[0]
    acc = np.zeros((cand_rows.shape[0], xv.shape[1]))
    tpos = np.asarray(target_pos, dtype=np.int64)
    ppos = None if prefix_pos is None else np.asarray(prefix_pos, dtype=np.int64)
    for t0 in range(0, T, block):
        r = np.arange(t0, min(T, t0 + block))
        z = logits_rows(xv, WCv, s_xw, r)
        g8 = g8_rows(z, L[r], tpos[r], None if ppos is None else ppos[r], N, s_g)
        acc += e4m3_decode(g8[:, cand_rows]).T @ xv[r]
    return (s_g * s_x) * acc
