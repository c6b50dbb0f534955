"""Loss and gradient oracle in float64 numpy -- TEST INFRASTRUCTURE ONLY.

What is computed (one microbatch of T tokens, hidden size d, candidate set C of
P classes; P == 0 means C is the whole vocabulary):

* logits  z[t, j] = x[t] . W[C[j]]                 ("sampled_softmax.py",
  module docstring: logits are x @ lm_head[C].T, each label replaced by its
  position in C);
* row log-sum-exp  L[t] = m[t] + ln sum_j exp(z[t, j] - m[t]),  m[t] = max_j z[t, j]
  ("Learning Triton one kernel at a time: softmax", the softmax definition and
  the max-subtraction section: subtracting the row maximum leaves the softmax
  unchanged and keeps exp in range);
* per-token loss  l[t] = [y'>=0](L[t] - z[t, y']) + [p'>=0](L[t] - z[t, p'])
  where y', p' are the target and prefix-target positions, -1 meaning "no label"
  (the page's no-op);
* N = number of labels with position >= 0; loss = sum_t l[t] / N, and 0 when
  N == 0 ("16_optimization_checks.py", lm_gradient: the summed token loss divided
  by the count of non-ignored targets);
* g[t, j] = (n_t * softmax(z[t])_j - [j == y'] - [j == p']) / N with
  n_t = [y'>=0] + [p'>=0] (the softmax-gradient section of the Triton softmax
  article, applied to cross-entropy: d loss / d z = softmax - one-hot);
* dX = g @ W_C,  dW_C = g^T @ x, and the dense dW [V, d] holds dW_C in the rows
  of C and exactly zero elsewhere ("sampled_softmax.py", module docstring: the
  lm_head gradient is dense with zeros outside C).

Matrix products are numpy's float64 matmul (a library primitive); nothing else is
blocked, fused or reordered. The "sampled" helpers evaluate single rows or
single columns of the same definition for shapes too large to hold [T, P].
"""
import numpy as np


def _wc(W, C):
    return W if C is None else W[np.asarray(C, dtype=np.int64)]


def _label_counts(target_pos, prefix_pos):
    n = (np.asarray(target_pos) >= 0).astype(np.int64)
    if prefix_pos is not None:
        n = n + (np.asarray(prefix_pos) >= 0).astype(np.int64)
    return n


def num_labels(target_pos, prefix_pos):
    """N: labels whose position is >= 0 (targets plus surviving prefix targets)."""
    return int(_label_counts(target_pos, prefix_pos).sum())


def logsumexp_rows(z):
    """Row log-sum-exp with the row maximum subtracted first."""
    m = z.max(axis=1, keepdims=True)
    return m[:, 0] + np.log(np.exp(z - m).sum(axis=1))


def ce_rows(z, target_pos, prefix_pos=None):
    """The cross-entropy part of the definition from the logits z [T, P] (float64):
    returns (loss, g [T, P], L [T], row_loss [T], N)."""
    z = np.asarray(z, dtype=np.float64)
    T, P = z.shape
    tpos = np.asarray(target_pos, dtype=np.int64)
    ppos = None if prefix_pos is None else np.asarray(prefix_pos, dtype=np.int64)
    n = _label_counts(tpos, ppos)
    N = int(n.sum())
    if T == 0:
        return 0.0, np.zeros((0, P)), np.zeros(0), np.zeros(0), N
    L = logsumexp_rows(z)
    rows = np.arange(T)
    row_loss = np.zeros(T)
    onehot = np.zeros((T, P))
    has_t = tpos >= 0
    row_loss[has_t] += L[has_t] - z[rows[has_t], tpos[has_t]]
    np.add.at(onehot, (rows[has_t], tpos[has_t]), 1.0)
    if ppos is not None:
        has_p = ppos >= 0
        row_loss[has_p] += L[has_p] - z[rows[has_p], ppos[has_p]]
        np.add.at(onehot, (rows[has_p], ppos[has_p]), 1.0)
    if N == 0:
        return 0.0, np.zeros((T, P)), L, row_loss, N
    g = (n[:, None] * np.exp(z - L[:, None]) - onehot) / N
    return float(row_loss.sum() / N), g, L, row_loss, N


def forward_backward(x, W, C, target_pos, prefix_pos=None):
    """Dense oracle: returns (loss, dX [T,d], dW [V,d], L [T], row_loss [T]).

    x [T,d] and W [V,d] are float64 (exact widenings of the inputs); C is the
    int array of candidate classes (None for the full softmax).
    """
    x = np.asarray(x, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    T, d = x.shape
    V = W.shape[0]
    WC = _wc(W, C)
    if T == 0:
        return 0.0, np.zeros((0, d)), np.zeros((V, d)), np.zeros(0), np.zeros(0)
    loss, g, L, row_loss, N = ce_rows(x @ WC.T, target_pos, prefix_pos)
    dX = g @ WC
    dWC = g.T @ x
    dW = np.zeros((V, d))
    if C is None:
        dW[:] = dWC
    else:
        dW[np.asarray(C, dtype=np.int64)] = dWC
    return loss, dX, dW, L, row_loss


# ---------------------------------------------------------------------------
# Entry-by-entry evaluation of the same definition, for full-size shapes.
# ---------------------------------------------------------------------------

def lse_rows(x, WC, rows=None, block=2048):
    """L[t] for the given rows (all rows when None); each row is independent, so
    rows are taken a block at a time only to bound memory."""
    x = np.asarray(x)
    rows = np.arange(x.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty(rows.shape[0])
    for s in range(0, rows.shape[0], block):
        r = rows[s:s + block]
        z = np.asarray(x[r], dtype=np.float64) @ WC.T
        out[s:s + block] = logsumexp_rows(z)
    return out


def label_logits(x, WC, pos):
    """z[t, pos[t]] for every t with pos[t] >= 0 (0 elsewhere)."""
    pos = np.asarray(pos, dtype=np.int64)
    out = np.zeros(pos.shape[0])
    ok = pos >= 0
    out[ok] = np.einsum("td,td->t", np.asarray(x[ok], dtype=np.float64),
                        WC[pos[ok]])
    return out


def loss_from_lse(x, WC, L, target_pos, prefix_pos=None):
    """(loss, row_loss, N) given every row's L."""
    tpos = np.asarray(target_pos, dtype=np.int64)
    row_loss = np.where(tpos >= 0, L - label_logits(x, WC, tpos), 0.0)
    if prefix_pos is not None:
        ppos = np.asarray(prefix_pos, dtype=np.int64)
        row_loss = row_loss + np.where(ppos >= 0, L - label_logits(x, WC, ppos), 0.0)
    N = num_labels(tpos, prefix_pos)
    return (float(row_loss.sum() / N) if N else 0.0), row_loss, N


def dx_rows(x, WC, L, target_pos, prefix_pos, N, rows):
    """dX[t] for the given rows: (n_t softmax(z_t) - one-hots) / N, times W_C."""
    rows = np.asarray(rows, dtype=np.int64)
    if N == 0:
        return np.zeros((rows.shape[0], WC.shape[1]))
    z = np.asarray(x[rows], dtype=np.float64) @ WC.T
    tpos = np.asarray(target_pos, dtype=np.int64)[rows]
    ppos = None if prefix_pos is None else np.asarray(prefix_pos, dtype=np.int64)[rows]
    n = _label_counts(tpos, ppos)
    g = n[:, None] * np.exp(z - L[rows][:, None])
    i = np.arange(rows.shape[0])
    np.add.at(g, (i[tpos >= 0], tpos[tpos >= 0]), -1.0)
    if ppos is not None:
        np.add.at(g, (i[ppos >= 0], ppos[ppos >= 0]), -1.0)
    return (g / N) @ WC


def dwc_rows(x, WC, L, target_pos, prefix_pos, N, cand_rows, block=256, tblock=8192):
    """dW_C[j] for the given candidate positions j: sum over tokens of g[t, j] x[t].
    Columns are taken `block` at a time and tokens `tblock` at a time, only to bound
    memory."""
    cand_rows = np.asarray(cand_rows, dtype=np.int64)
    d = WC.shape[1]
    out = np.zeros((cand_rows.shape[0], d))
    if N == 0:
        return out
    tpos = np.asarray(target_pos, dtype=np.int64)
    ppos = None if prefix_pos is None else np.asarray(prefix_pos, dtype=np.int64)
    n = _label_counts(tpos, ppos)
    for s in range(0, cand_rows.shape[0], block):
        j = cand_rows[s:s + block]
        T = x.shape[0]
        acc = np.zeros((j.shape[0], d))
        for t0 in range(0, T, tblock):
            t1 = t0 + tblock
            xb = np.asarray(x[t0:t1], dtype=np.float64)
            zc = xb @ WC[j].T                                  # [tb, |j|]
            g = n[t0:t1, None] * np.exp(zc - L[t0:t1, None])
            g -= (tpos[t0:t1, None] == j[None, :])
            if ppos is not None:
                g -= (ppos[t0:t1, None] == j[None, :])
            acc += g.T @ xb
        out[s:s + block] = acc / N
    return out
