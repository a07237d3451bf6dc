"""Log-sum-exp merge of partial attentions.

The ModelScope/CSDN page (design section, decode paragraph) attends the INT2
and BF16 segments separately and merges the two results by online softmax.
Each partial i carries its normalised output o_i and the natural-log
log-sum-exp lse_i of its logits; the merged output is

    LSE = ln sum_i exp(lse_i),   O = sum_i exp(lse_i - LSE) o_i.

An empty partial has lse = -inf and weight 0; if every partial is empty the
output is 0 and LSE = -inf.
"""

import math

import numpy as np


def merge_partials(o_parts, lse_parts):
    o = np.asarray(o_parts, np.float64)
    lse = np.asarray(lse_parts, np.float64)
    if lse.size == 0 or np.all(np.isneginf(lse)):
        return np.zeros(o.shape[-1]), -np.inf
    m = lse.max()
    w = np.exp(lse - m)
    tot = w.sum()
    return (w[:, None] * o).sum(axis=0) / tot, m + math.log(tot)
