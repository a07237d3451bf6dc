"""Offline calibration and the synthetic error chain, in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Calibration (MarkTechPost article, "What OSCAR Does Differently"; ModelScope/
CSDN page, section on OSCAR's design):
  C1  query covariance of a KV head: C_Q = (1/N) sum_n q_n^T q_n over the
      calibration queries of all query heads that read the KV head;
  C2  score-weighted value covariance C_S = (1/N) V^T S^T S V with S the
      causal softmax score matrix (scale 1/sqrt(D)) of the calibration draw,
      averaged over the KV head's query heads;
  C3  U = eigenvectors of C (numpy's symmetric eigensolver), columns ordered
      by descending eigenvalue, each column's largest-magnitude entry made
      positive (the first one where two tie);
  C4  R = U H P_br: H the Sylvester Walsh-Hadamard matrix scaled by
      1/sqrt(D), P_br the bit-reversal permutation, (y P_br)[j] = y[br(j)];
      row-vector convention x' = x R with R stored [D_in][D_out];
  C5  clip threshold tau = the 0.995 quantile of |x R| over every rotated
      calibration value of the head, with linear interpolation between order
      statistics (Hyndman and Fan's definition 7), rounded to fp32.

Error chain (ModelScope/CSDN page, motivation section and its Figure 1, which
compares rotations by attention-score KL and attention output MSE rather
than by K/V reconstruction error; MarkTechPost article, same section, for the
logit error ||Q K^T - Q K^^T||_F^2):
  E1  quantize the bf16 calibration keys and values with the write path
      (rotate, clip, INT2, the oracle's ``quantize_tokens``) and dequantize
      them back to the model basis: k^ = [s (q - z)] R^T;
  E2  for every query row n and key t <= n (causal):
        logit error      d_nt = sm q_n . (k^_t - k_t),  summed squares per row;
        score KL         KL(p_n || p^_n) with p = softmax(sm q k^T) rows;
        output error     ||o_n - o^_n||^2, o = p V, o^ = p^ V^;
      the summaries are the mean squared logit error over causal pairs, the
      mean KL over rows and sum ||o - o^||^2 / sum ||o||^2.

The rotation, the thresholds and the error metrics are pinned by
``tests/test_oracle_calibration.py``.
"""

import math

import numpy as np

from .quant import dequantize, quantize_tokens

CLIP_QUANTILE = 0.995


def query_covariance(q):
    """C1: q [..., N, D] (all leading axes are pooled) -> C_Q [D, D] fp64."""
    x = np.asarray(q, np.float64).reshape(-1, np.shape(q)[-1])
    return x.T @ x / x.shape[0]


def causal_attention(q, k, v, sm=None):
    """Causal softmax attention of N queries over N keys (row n sees keys
    0..n).  q, k, v: [N, D].  Returns (o [N, D], lse [N]) in fp64."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    n, d = q.shape
    sm = 1.0 / math.sqrt(d) if sm is None else sm
    logits = sm * (q @ k.T)
    logits = np.where(np.tril(np.ones((n, n), dtype=bool)), logits, -np.inf)
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m)
    z = e.sum(axis=1, keepdims=True)
    return (e @ v) / z, (m + np.log(z))[:, 0]


def score_weighted_covariance(q, k, v, sm=None):
    """C2: q [g, N, D] (the KV head's query heads), k, v [N, D] -> C_S."""
    q = np.asarray(q, np.float64)
    c = np.zeros((q.shape[-1], q.shape[-1]))
    for h in range(q.shape[0]):
        o, _ = causal_attention(q[h], k, v, sm)
        c += o.T @ o / o.shape[0]
    return c / q.shape[0]


def eigenbasis(c):
    """C3: (U, eigenvalues), eigenvalues descending, U's columns signed so
    that each column's largest-magnitude entry is positive."""
    w, u = np.linalg.eigh(np.asarray(c, np.float64))
    order = np.argsort(w)[::-1]
    w, u = w[order], u[:, order]
    top = np.argmax(np.abs(u), axis=0)
    return u * np.sign(u[top, np.arange(u.shape[1])]), w


def hadamard_matrix(d):
    """Sylvester-ordered Walsh-Hadamard matrix scaled by 1/sqrt(d)."""
    assert d > 0 and d & (d - 1) == 0
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h / math.sqrt(d)


def bit_reversal_permutation(d):
    """br[i] = i with its log2(d) bits in reverse order."""
    bits = int(round(math.log2(d)))
    assert 1 << bits == d
    return np.array([int(format(i, f"0{bits}b")[::-1], 2) if bits else 0 for i in range(d)])


def mix_matrix(d):
    """H P_br as one matrix: column j of H P_br is column br(j) of H."""
    return hadamard_matrix(d)[:, bit_reversal_permutation(d)]


def rotation(c=None, d=None):
    """C4: R = U H P_br for the covariance c; with c None, the Hadamard-only
    rotation H P_br (U = I) of size d.  fp64."""
    if c is None:
        return mix_matrix(d)
    u, _ = eigenbasis(c)
    return u @ mix_matrix(u.shape[0])


def clip_threshold(x, r, quantile=CLIP_QUANTILE):
    """C5: x [..., D] calibration vectors, r [D, D] (None: no rotation)."""
    x = np.asarray(x, np.float64).reshape(-1, np.shape(x)[-1])
    y = x if r is None else x @ np.asarray(r, np.float64)
    return np.float32(np.quantile(np.abs(y), quantile, method="linear"))


def calibrate_head(q, k, v, sm=None):
    """C1-C5 for one KV head.  q [g, N, D], k, v [N, D] calibration
    activations (values in the model basis).  R is returned in fp64 and in the
    fp32 form the hot path takes; tau from the fp64 R."""
    c_q = query_covariance(q)
    c_s = score_weighted_covariance(q, k, v, sm)
    r_k = rotation(c_q)
    r_v = rotation(c_s)
    return {
        "c_q": c_q, "c_s": c_s, "r_k64": r_k, "r_v64": r_v,
        "eig_q": eigenbasis(c_q)[1], "eig_s": eigenbasis(c_s)[1],
        "r_k": r_k.astype(np.float32), "r_v": r_v.astype(np.float32),
        "tau_k": clip_threshold(k, r_k), "tau_v": clip_threshold(v, r_v),
    }


def calibrate(draws, sm=None):
    """``calibrate_head`` over a list of per-KV-head (q, k, v) triples; the
    per-head results stacked along a leading KV-head axis."""
    heads = [calibrate_head(q, k, v, sm) for q, k, v in draws]
    return {key: np.stack([h[key] for h in heads]) for key in heads[0]}


# --------------------------------------------------------------------------
# error chain
# --------------------------------------------------------------------------

def quantize_roundtrip(x, r, tau, group_size):
    """E1: x [N, D] bf16 values -> k^ [N, D] fp64 in the model basis.  r
    None quantizes without rotation."""
    codes, s, z = quantize_tokens(x, r, tau, group_size)
    y_hat = dequantize(codes, s, z, group_size)
    if r is None:
        return y_hat
    return y_hat @ np.asarray(r, np.float32).astype(np.float64).T


def kl_divergence(p, p_hat):
    """KL(p || p^) = sum_t p_t ln(p_t / p^_t) over the last axis (terms with
    p_t = 0 contribute 0)."""
    p = np.asarray(p, np.float64)
    p_hat = np.asarray(p_hat, np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.where(p > 0, p * (np.log(p) - np.log(p_hat)), 0.0)
    return t.sum(axis=-1)


def attention_error_rows(q, k, v, k_hat, v_hat, sm=None):
    """E2 for one query head: q, k, v, k_hat, v_hat [N, D].  Returns per row
    n: kl [N], logit squared error summed over t <= n [N], ||o - o^||^2 [N],
    ||o||^2 [N]."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    k_hat = np.asarray(k_hat, np.float64)
    v_hat = np.asarray(v_hat, np.float64)
    n, d = q.shape
    sm = 1.0 / math.sqrt(d) if sm is None else sm
    mask = np.tril(np.ones((n, n), dtype=bool))
    logits = sm * (q @ k.T)
    logits_hat = sm * (q @ k_hat.T)
    p = _softmax_rows(np.where(mask, logits, -np.inf))
    p_hat = _softmax_rows(np.where(mask, logits_hat, -np.inf))
    o = p @ v
    o_hat = p_hat @ v_hat
    return (kl_divergence(p, p_hat),
            np.where(mask, (logits_hat - logits) ** 2, 0.0).sum(axis=1),
            ((o - o_hat) ** 2).sum(axis=1), (o ** 2).sum(axis=1))


def _softmax_rows(x):
    e = np.exp(x - x.max(axis=1, keepdims=True))
    return e / e.sum(axis=1, keepdims=True)


def summarize(rows):
    """Means over a stack of ``attention_error_rows`` results (leading axes
    any): mean squared logit error per causal pair, mean KL per row, relative
    output MSE."""
    kl, lse2, ose, osq = (np.asarray(a, np.float64) for a in rows)
    n = kl.shape[-1]
    pairs = kl.size // n * n * (n + 1) // 2
    return {"logit_mse": lse2.sum() / pairs, "kl": kl.mean(), "out_rel_mse": ose.sum() / osq.sum()}


def error_chain(q, k, v, r_k, r_v, tau_k, tau_v, group_size, sm=None):
    """E1 + E2 for one KV head: q [g, N, D], k, v [N, D] bf16 values (the
    cache's content before quantization).  r None = no rotation (tau still
    clips).  Returns (per-row results stacked [4, g, N], summary)."""
    k_hat = quantize_roundtrip(k, r_k, tau_k, group_size)
    v_hat = quantize_roundtrip(v, r_v, tau_v, group_size)
    rows = [attention_error_rows(qh, k, v, k_hat, v_hat, sm) for qh in np.asarray(q)]
    stacked = np.stack([np.stack(r) for r in rows], axis=1)  # [4, g, N]
    return stacked, summarize(stacked)
