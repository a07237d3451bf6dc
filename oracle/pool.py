"""Logical three-segment token pool of one sequence.

Segments (MarkTechPost article, "The Serving System"; ModelScope/CSDN page,
design section): a BF16 sink of the first S0 tokens, an INT2 history, and a
BF16 recent window of the last W tokens.  New tokens enter the recent window;
as decoding advances, the oldest recent token is rotated, clipped, quantized,
packed and demoted into the history (ModelScope/CSDN page, same section).

Readings where the pages are silent:
  * the length L counts the token appended this step; append first, then
    demote, then attend;
  * positions: sink [0, min(L, S0)), history [S0, max(S0, L - W)), recent
    [max(S0, L - W), L); after appending position L-1, token d = L-1-W is
    demoted when d >= S0;
  * keys in the BF16 segments are unrotated (only demotion rotates); values
    are stored in the V basis of the pool in all three segments (R_V is
    absorbed into the projection weights, MarkTechPost article, "The Serving
    System"), so with ``v_absorbed`` the history V is quantized without a
    rotation, otherwise it is rotated by R_V at demotion.

The oracle holds logical arrays, not pages: dense bf16 K/V per position and
per-token history codes, scales and zeros.  With ``levels_k`` / ``levels_v``
(four-level codebooks, ``codebook``) the history is quantized with the
codebook quantizer instead of the uniform one.
"""

import numpy as np

from . import codebook
from .quant import quantize_tokens


class SeqPool:
    def __init__(self, num_kv_heads, head_dim, group_size, sink=64, recent=256,
                 v_absorbed=True, levels_k=None, levels_v=None):
        self.hkv, self.d, self.g = num_kv_heads, head_dim, group_size
        self.ng = head_dim // group_size
        self.sink, self.recent, self.v_absorbed = sink, recent, v_absorbed
        self.levels_k, self.levels_v = levels_k, levels_v
        self.L = 0
        self.k = np.zeros((0, self.hkv, self.d), np.float32)
        self.v = np.zeros((0, self.hkv, self.d), np.float32)
        z3 = lambda: np.zeros((0, self.hkv, self.d), np.uint8)  # noqa: E731
        zs = lambda: np.zeros((0, self.hkv, self.ng), np.float32)  # noqa: E731
        self.kc, self.ks, self.kz = z3(), zs(), zs()
        self.vc, self.vs, self.vz = z3(), zs(), zs()

    # ---- segment arithmetic ------------------------------------------------
    def recent_start(self, L=None):
        L = self.L if L is None else L
        return max(self.sink, L - self.recent)

    @property
    def n_hist(self):
        return self.kc.shape[0]

    def segments(self):
        """(sink positions, history positions, recent positions)."""
        r0 = self.recent_start()
        return (np.arange(min(self.L, self.sink)), np.arange(self.sink, r0),
                np.arange(r0, self.L))

    # ---- write path ----------------------------------------------------------
    def _quantize(self, pos, r_k, tau_k, r_v, tau_v):
        """Quantize tokens at positions ``pos`` (all KV heads)."""
        outs = {n: [] for n in ("kc", "ks", "kz", "vc", "vs", "vz")}
        def quant(x, r, tau, levels):
            if levels is None:
                return quantize_tokens(x, r, tau, self.g)
            return codebook.quantize_tokens(x, r, tau, self.g, levels)
        for h in range(self.hkv):
            kc, ks, kz = quant(self.k[pos, h], r_k[h], tau_k[h], self.levels_k)
            rv = None if self.v_absorbed else r_v[h]
            vc, vs, vz = quant(self.v[pos, h], rv, tau_v[h], self.levels_v)
            for n, a in zip(outs, (kc, ks, kz, vc, vs, vz)):
                outs[n].append(a)
        return {n: np.stack(a, axis=1) for n, a in outs.items()}

    def _append_hist(self, q):
        for n in q:
            setattr(self, n, np.concatenate([getattr(self, n), q[n]]))

    def prefill(self, k, v, r_k, tau_k, tau_v, r_v=None):
        """State of a sequence after ``len(k)`` tokens, with its history
        quantized token by token (the per-token map makes bulk and one-by-one
        demotion identical)."""
        self.k = np.asarray(k, np.float32).copy()
        self.v = np.asarray(v, np.float32).copy()
        self.L = self.k.shape[0]
        hist = np.arange(self.sink, self.recent_start())
        self.kc = np.zeros((0, self.hkv, self.d), np.uint8)
        self.ks = self.kz = self.vs = self.vz = np.zeros((0, self.hkv, self.ng), np.float32)
        self.vc = np.zeros((0, self.hkv, self.d), np.uint8)
        if len(hist):
            self._append_hist(self._quantize(hist, r_k, tau_k, r_v, tau_v))
        return self

    def append_demote(self, k_new, v_new, r_k, tau_k, tau_v, r_v=None):
        """Append one token (k_new, v_new: [Hkv, D]) and demote the oldest
        recent token if it leaves the window.  Returns the demoted position
        or None."""
        self.k = np.concatenate([self.k, np.asarray(k_new, np.float32)[None]])
        self.v = np.concatenate([self.v, np.asarray(v_new, np.float32)[None]])
        self.L += 1
        d = self.L - 1 - self.recent
        if d >= self.sink:
            assert d == self.sink + self.n_hist
            self._append_hist(self._quantize(np.array([d]), r_k, tau_k, r_v, tau_v))
            return d
        return None

