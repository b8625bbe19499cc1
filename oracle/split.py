"""Split-KV attention: partial outputs over key ranges and their merge, in float64.

TEST INFRASTRUCTURE ONLY (see the package header).

Sources (page titles and sections):
- "FlashAttention: Fast and Memory-Efficient Exact Attention with IO-Awareness"
  (summary page of arXiv 2205.14135), Method, incremental softmax tracking: for a
  vector split into x1 and x2, m(x) = max(m(x1), m(x2)) and
  l(x) = e^{m(x1) - m(x)} l(x1) + e^{m(x2) - m(x)} l(x2); the running output of the
  block update is rescaled the same way, O <- diag(l_new)^-1 (diag(l) e^{m - m_new} O
  + e^{m~ - m_new} P~ V). Splitting the key axis into ranges and merging their
  (O, m, l) with this rule is the same computation with the key blocks processed
  apart instead of one after the other.

Readings (where the pages are silent):
- A split is a contiguous key range [p*L, min(N, (p+1)*L)) of a fixed length L; the
  masks (causal, key padding) apply inside it unchanged.
- A query row that sees no key of a range has an empty partial: O_p = 0 and
  LSE_p = -inf (m = -inf, l = 0: the state that holds nothing). It contributes
  exactly nothing to the merge.
- The partial output is normalised (O_p = P_p V over its range) and carries
  LSE_p = m_p + ln l_p, so a merge needs only (O_p, LSE_p): with m = LSE_p and l = 1
  the page's rule applies as written.
"""
from __future__ import annotations

import math

import numpy as np

from .attention import allowed_mask

NEG_INF = -math.inf


def split_ranges(n: int, split_len: int) -> list:
    """Key ranges [(begin, end)] of length split_len covering [0, n)."""
    if split_len <= 0:
        raise ValueError("split_len must be positive")
    return [(b, min(n, b + split_len)) for b in range(0, n, split_len)]


def head_forward_range(q, k, v, scale, causal, kv_len_b, kbeg, kend):
    """Attention of every query row of one head over keys [kbeg, kend) only.

    The definition with the key set restricted: S = scale * q k^T, masked (causal,
    key padding, and every key outside the range) to -inf; rows with a visible key get
    the safe softmax O = P V and LSE = m + ln l; rows without one get O = 0, LSE = -inf.
    """
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    n = q.shape[0]
    a = allowed_mask(n, k.shape[0], causal, kv_len_b)
    inside = np.zeros(k.shape[0], dtype=bool)
    inside[kbeg:kend] = True
    a &= inside[None, :]
    s = np.where(a, scale * (q @ k.T), -np.inf)
    o = np.zeros((n, v.shape[1]))
    lse = np.full(n, -np.inf)
    rows = a.any(axis=1)
    if rows.any():
        sr = s[rows]
        m = sr.max(axis=1)
        e = np.exp(sr - m[:, None])
        l = e.sum(axis=1)
        o[rows] = (e / l[:, None]) @ v
        lse[rows] = m + np.log(l)
    return o, lse


def attention_forward_split(q, k, v, scale, causal=False, kv_len=None, split_len=64):
    """[B,H,N,d] (queries and keys alike) -> (O_parts [P,B,H,N,d], LSE_parts [P,B,H,N]),
    one partial per key range of split_len keys."""
    B, H, N, d = q.shape
    ranges = split_ranges(N, split_len)
    o = np.zeros((len(ranges), B, H, N, v.shape[3]))
    lse = np.full((len(ranges), B, H, N), -np.inf)
    for p, (kb, ke) in enumerate(ranges):
        for b in range(B):
            kvb = None if kv_len is None else int(kv_len[b])
            for h in range(H):
                o[p, b, h], lse[p, b, h] = head_forward_range(
                    q[b, h], k[b, h], v[b, h], scale, causal, kvb, kb, ke)
    return o, lse


def merge_pair(o1, lse1, o2, lse2):
    """One application of the incremental tracking rule to two normalised partials.

    Per row: (m1, l1) = (LSE1, 1), (m2, l2) = (LSE2, 1); m = max(m1, m2);
    l = e^{m1 - m} l1 + e^{m2 - m} l2; O = (e^{m1 - m} l1 O1 + e^{m2 - m} l2 O2) / l;
    the merged partial is (O, m + ln l). A side whose LSE is -inf weighs 0; two empty
    sides stay empty (O = 0, LSE = -inf).
    """
    o1, o2 = np.asarray(o1, dtype=np.float64), np.asarray(o2, dtype=np.float64)
    lse1, lse2 = np.asarray(lse1, dtype=np.float64), np.asarray(lse2, dtype=np.float64)
    m = np.maximum(lse1, lse2)
    empty = m == -np.inf
    m_safe = np.where(empty, 0.0, m)
    w1 = np.where(lse1 == -np.inf, 0.0, np.exp(lse1 - m_safe))
    w2 = np.where(lse2 == -np.inf, 0.0, np.exp(lse2 - m_safe))
    l = w1 + w2
    l_safe = np.where(empty, 1.0, l)
    o = (w1[..., None] * o1 + w2[..., None] * o2) / l_safe[..., None]
    lse = np.where(empty, -np.inf, m_safe + np.log(l_safe))
    return np.where(empty[..., None], 0.0, o), lse


def merge_partials(o_parts, lse_parts):
    """Fold merge_pair over the splits in order: (O [..., N, d], LSE [..., N])."""
    o, lse = o_parts[0], lse_parts[0]
    for p in range(1, len(o_parts)):
        o, lse = merge_pair(o, lse, o_parts[p], lse_parts[p])
    return np.asarray(o, dtype=np.float64), np.asarray(lse, dtype=np.float64)
