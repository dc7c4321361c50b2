"""Empirical entropy of BF16 tensors (test infrastructure only).

The bits/weight target is stated against the plug-in (maximum-likelihood)
conditional entropy H(S) + H(F | S) of the joint (sign, exponent) symbol S and
the 7-bit fraction F [Qwen3.8-27B-BF16-NVLC-Lossless card, codec paragraph:
the fraction is coded conditionally on the decoded sign/exponent symbol].

Three independent routes are provided so that each pins the others:
  * ``conditional_entropy_bits``: numpy fp64 from the two field histograms;
  * ``word_entropy_bits``: H(W) over the 65,536-bin word histogram (chain rule:
    H(W) = H(S) + H(F|S) exactly, because W <-> (S, F) is a bijection);
  * ``exact_bits``: exact rational arithmetic for tiny hand-computable cases.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np


def _h(counts: np.ndarray) -> float:
    c = np.asarray(counts, dtype=np.float64).ravel()
    c = c[c > 0]
    if c.size == 0:
        return 0.0
    n = c.sum()
    p = c / n
    return float(-(p * np.log2(p)).sum())


def split(words: np.ndarray):
    w = np.asarray(words, dtype=np.uint16).astype(np.int64)
    return w >> 7, w & 0x7F


def field_histograms(words: np.ndarray):
    s, f = split(words)
    cs = np.bincount(s, minlength=512).astype(np.int64)
    cf = np.bincount(s * 128 + f, minlength=512 * 128).astype(np.int64).reshape(512, 128)
    return cs, cf


def conditional_entropy_bits(words: np.ndarray):
    """(H_S, H_F|S) in bits per weight, plug-in estimator, fp64."""
    cs, cf = field_histograms(words)
    n = cs.sum()
    if n == 0:
        return 0.0, 0.0
    hs = _h(cs)
    hfs = 0.0
    for s in np.nonzero(cs)[0]:
        hfs += cs[s] / n * _h(cf[s])
    return hs, float(hfs)


def word_entropy_bits(words: np.ndarray) -> float:
    w = np.asarray(words, dtype=np.uint16).astype(np.int64)
    return _h(np.bincount(w, minlength=65536))


def exact_bits(words) -> Fraction:
    """Exact H_S + H_F|S for tiny inputs whose probabilities are powers of two.

    Raises ValueError when a probability is not a power of two (log2 would be
    irrational)."""
    ws = [int(w) & 0xFFFF for w in words]
    n = len(ws)
    cs, cf = {}, {}
    for w in ws:
        s, f = w >> 7, w & 0x7F
        cs[s] = cs.get(s, 0) + 1
        cf[(s, f)] = cf.get((s, f), 0) + 1

    def lg(fr: Fraction) -> int:
        # exact log2 of a power-of-two fraction
        num, den = fr.numerator, fr.denominator
        if num & (num - 1) or den & (den - 1):
            raise ValueError("not a power of two")
        return num.bit_length() - den.bit_length()

    hs = sum(-Fraction(c, n) * lg(Fraction(c, n)) for c in cs.values())
    hfs = Fraction(0)
    for (s, f), c in cf.items():
        p_s = Fraction(cs[s], n)
        p_f = Fraction(c, cs[s])
        hfs += p_s * (-p_f * lg(p_f))
    return hs + hfs


def gaussian_entropy_bits(sigma: float):
    """Closed form H_S, H_F|S for i.i.d. N(0, sigma^2) rounded to BF16 (RNE).

    Each finite BF16 value v owns the real interval between the midpoints to
    its neighbours (ties go to the even mantissa, a measure-zero detail); the
    probability of v is the Gaussian mass of that interval.  +0 and -0 own
    (0, m1) and (-m1, 0)."""
    from scipy.stats import norm

    # all non-negative finite BF16 values in increasing order: words 0x0000..0x7F7F
    pos_words = np.arange(0, 0x7F80, dtype=np.int64)
    vals = (pos_words.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    mids = np.empty(vals.size + 1)
    mids[0] = 0.0
    mids[1:-1] = 0.5 * (vals[:-1] + vals[1:])
    mids[-1] = np.inf
    # scaled CDF differences, tail handled with sf for accuracy
    lo = mids[:-1] / sigma
    hi = mids[1:] / sigma
    p_pos = norm.sf(lo) - norm.sf(hi)  # mass of (lo, hi) on the positive side
    # word probability: positive word w gets p_pos, its negative twin w|0x8000 the same
    P = np.zeros(65536)
    P[pos_words] = p_pos
    P[pos_words | 0x8000] = p_pos
    P /= P.sum()
    s = np.arange(65536) >> 7
    ps = np.bincount(s, weights=P, minlength=512)
    nz = P > 0
    H_w = float(-(P[nz] * np.log2(P[nz])).sum())
    nzs = ps > 0
    H_s = float(-(ps[nzs] * np.log2(ps[nzs])).sum())
    return H_s, H_w - H_s


def bits_per_weight(container_bf16_bytes: int, n_weights: int) -> float:
    return 8.0 * container_bf16_bytes / n_weights if n_weights else math.nan
