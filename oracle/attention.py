"""Decode attention over the three-segment pool, in fp64.

Read path (MarkTechPost article, "The Serving System": the INT2 kernel
unpacks, dequantizes and inverse-rotates before attention; ModelScope/CSDN
page, design section: INT2 and BF16 segments attended separately and merged
by online softmax).  The oracle does not split anything: it builds the full
key and value sequence and takes one softmax over it.

  R1  history: k^ = [s_K (q_K - z_K)] R_K^T and v^ = s_V (q_V - z_V)
      (absorbed V; otherwise times R_V^T), all fp64; with a four-level
      codebook L the code value q is replaced by L[q].
  R2  logits l_t = sm * (q . k_t) with sm = 1/sqrt(D) unless given; sink and
      recent keys are the stored bf16 values, unrotated.
  R3  p = softmax(l) over the concatenation sink | history | recent, with max
      subtraction; o = sum_t p_t v_t; lse = max + ln(sum exp(l - max)).

Query head h reads KV head floor(h / g), g = Hq / Hkv.
"""

import math

import numpy as np

from . import codebook
from .quant import dequantize


def attention_one_head(keys, values, q, sm):
    """Softmax attention of one query over [T, D] keys/values (fp64).
    Returns (o [D], lse).  T = 0 gives (zeros, -inf)."""
    keys = np.asarray(keys, np.float64)
    values = np.asarray(values, np.float64)
    if keys.shape[0] == 0:
        return np.zeros(values.shape[1]), -np.inf
    logits = sm * (keys @ np.asarray(q, np.float64))
    m = logits.max()
    e = np.exp(logits - m)
    tot = e.sum()
    return (e @ values) / tot, m + math.log(tot)


def _dequant(codes, s, z, g, levels):
    if levels is None:
        return dequantize(codes, s, z, g)
    return codebook.dequantize(codes, s, z, g, levels)


def _history_kv(seq, kv, r_k, r_v):
    lk, lv = getattr(seq, "levels_k", None), getattr(seq, "levels_v", None)
    k_hat = _dequant(seq.kc[:, kv], seq.ks[:, kv], seq.kz[:, kv], seq.g, lk)
    k_hat = k_hat @ np.asarray(r_k[kv], np.float32).astype(np.float64).T
    v_hat = _dequant(seq.vc[:, kv], seq.vs[:, kv], seq.vz[:, kv], seq.g, lv)
    if not seq.v_absorbed:
        v_hat = v_hat @ np.asarray(r_v[kv], np.float32).astype(np.float64).T
    return k_hat, v_hat


def decode_attention(seqs, q, r_k, r_v=None, sm_scale=None, pairs=None):
    """Decode one step for every sequence.

    seqs: list of oracle SeqPool; q: [B, Hq, D] bf16 values.
    pairs: optional iterable of (b, h) to compute (others left NaN).
    Returns (out [B, Hq, D] fp64, lse [B, Hq] natural log).
    """
    q = np.asarray(q, np.float64)
    bsz, hq, d = q.shape
    sm = 1.0 / math.sqrt(d) if not sm_scale else float(sm_scale)
    out = np.full((bsz, hq, d), np.nan)
    lse = np.full((bsz, hq), np.nan)
    want = None if pairs is None else set(pairs)
    for b, seq in enumerate(seqs):
        g = hq // seq.hkv
        sink, _, recent = seq.segments()
        for kv in range(seq.hkv):
            heads = [h for h in range(kv * g, (kv + 1) * g) if want is None or (b, h) in want]
            if not heads:
                continue
            k_hat, v_hat = _history_kv(seq, kv, r_k, r_v)
            keys = np.concatenate([seq.k[sink, kv], k_hat, seq.k[recent, kv]]).astype(np.float64)
            vals = np.concatenate([seq.v[sink, kv], v_hat, seq.v[recent, kv]]).astype(np.float64)
            for h in heads:
                out[b, h], lse[b, h] = attention_one_head(keys, vals, q[b, h], sm)
    return out, lse


def bf16_decode_attention(k, v, q, seq_lens, sm_scale=None, pairs=None):
    """All-BF16 decode (the comparator): softmax attention over every stored
    bf16 key/value of each sequence.  k[b], v[b]: [L_b, Hkv, D]."""
    q = np.asarray(q, np.float64)
    bsz, hq, d = q.shape
    sm = 1.0 / math.sqrt(d) if not sm_scale else float(sm_scale)
    out = np.full((bsz, hq, d), np.nan)
    lse = np.full((bsz, hq), np.nan)
    want = None if pairs is None else set(pairs)
    for b in range(bsz):
        kb = np.asarray(k[b], np.float64)[: seq_lens[b]]
        vb = np.asarray(v[b], np.float64)[: seq_lens[b]]
        g = hq // kb.shape[1]
        for h in range(hq):
            if want is not None and (b, h) not in want:
                continue
            out[b, h], lse[b, h] = attention_one_head(kb[:, h // g], vb[:, h // g], q[b, h], sm)
    return out, lse
