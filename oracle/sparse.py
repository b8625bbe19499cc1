"""Block-sparse attention: the definition with a block mask, in float64.

TEST INFRASTRUCTURE ONLY (see the package header).

Source: "FlashAttention: Fast and Memory-Efficient Exact Attention with IO-Awareness"
(summary page of arXiv 2205.14135), Extension: Block-Sparse FlashAttention -- a fixed
mask M in {0,1}^{(N/Br) x (N/Bc)} restricts evaluation to its nonzero blocks. The
method evaluates only those blocks; what it computes is attention whose scores outside
them are -inf, which is what this module writes out.

Readings (where the page is silent):
- Br = Bc = `block` (128 for the library); the last block row/column is ragged when
  `block` does not divide N. The mask is shared by every batch and head.
- M hides key j from query i when M[i // block][j // block] == 0, on top of the causal
  and key-padding rules.
- A query row that sees no key at all (possible now) gets O = 0 and LSE = -inf, and
  contributes nothing to any gradient (its P row is 0); its dQ is 0.
"""
from __future__ import annotations

import numpy as np

from .attention import allowed_mask


def block_allowed(n: int, causal: bool, kv_len_b, block_mask, block: int) -> np.ndarray:
    """Boolean [n, n]: key j visible to query i under the masks and the block mask."""
    bm = np.asarray(block_mask) != 0
    nb = -(-n // block)
    if bm.shape != (nb, nb):
        raise ValueError(f"block mask must be {nb} x {nb}")
    idx = np.arange(n) // block
    return allowed_mask(n, n, causal, kv_len_b) & bm[idx[:, None], idx[None, :]]


def _probs(q, k, scale, a):
    """P [n, n] (rows with no visible key all 0), m, l of the scaled, masked scores."""
    s = np.where(a, scale * (q @ k.T), -np.inf)
    rows = a.any(axis=1)
    m = np.where(rows, s.max(axis=1, initial=-np.inf), 0.0)
    e = np.where(a, np.exp(s - m[:, None]), 0.0)
    l = e.sum(axis=1)
    p = e / np.where(rows, l, 1.0)[:, None]
    return p, m, l, rows


def head_forward_sparse(q, k, v, scale, causal, kv_len_b, block_mask, block=128):
    """One head: (O [N,d], LSE [N]); empty rows O = 0, LSE = -inf."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    a = block_allowed(q.shape[0], causal, kv_len_b, block_mask, block)
    p, m, l, rows = _probs(q, k, scale, a)
    lse = np.where(rows, m + np.log(np.where(rows, l, 1.0)), -np.inf)
    return p @ v, lse


def head_backward_sparse(q, k, v, dout, scale, causal, kv_len_b, block_mask, block=128):
    """One head: gradient of sum(dout * O) -> (dQ, dK, dV), the chain rule of the
    definition (dV = P^T dO, dP = dO V^T, D = rowsum(P * dP), dS = P * (dP - D),
    dQ = scale dS K, dK = scale dS^T Q) with P rows of empty queries equal to 0."""
    q, k, v, dout = (np.asarray(x, dtype=np.float64) for x in (q, k, v, dout))
    a = block_allowed(q.shape[0], causal, kv_len_b, block_mask, block)
    p, _, _, _ = _probs(q, k, scale, a)
    dv = p.T @ dout
    dp = dout @ v.T
    dsum = (p * dp).sum(axis=1)
    ds = p * (dp - dsum[:, None])
    return scale * (ds @ k), scale * (ds.T @ q), dv


def attention_forward_sparse(q, k, v, scale, causal=False, kv_len=None, block_mask=None,
                             block=128):
    """[B,H,N,d] -> (O [B,H,N,d], LSE [B,H,N])."""
    B, H, N, d = q.shape
    o = np.empty((B, H, N, v.shape[3]))
    lse = np.empty((B, H, N))
    for b in range(B):
        kvb = None if kv_len is None else int(kv_len[b])
        for h in range(H):
            o[b, h], lse[b, h] = head_forward_sparse(q[b, h], k[b, h], v[b, h], scale,
                                                     causal, kvb, block_mask, block)
    return o, lse


def attention_backward_sparse(q, k, v, dout, scale, causal=False, kv_len=None,
                              block_mask=None, block=128):
    """[B,H,N,d] -> (dQ, dK, dV)."""
    B, H, N, d = q.shape
    dq, dk, dv = (np.empty(q.shape), np.empty(k.shape), np.empty(v.shape))
    for b in range(B):
        kvb = None if kv_len is None else int(kv_len[b])
        for h in range(H):
            dq[b, h], dk[b, h], dv[b, h] = head_backward_sparse(
                q[b, h], k[b, h], v[b, h], dout[b, h], scale, causal, kvb, block_mask, block)
    return dq, dk, dv


def head_row_block_sparse(q, k, v, dout, scale, causal, kv_len_b, block_mask, r0, r1,
                          block=128):
    """Block-sparse attention restricted to query rows r0 .. r1-1 of one head, for heads
    too long to take whole: (O, LSE, dQ) of those rows and their contributions to dK and
    dV, under the same conventions as head_forward_sparse / head_backward_sparse (a row
    that sees no key: O = 0, LSE = -inf, P = 0)."""
    q, k, v, dout = (np.asarray(x, dtype=np.float64) for x in (q, k, v, dout))
    bm = np.asarray(block_mask) != 0
    n = k.shape[0]
    rows = np.arange(r0, r1)
    cols = np.arange(n)
    a = allowed_mask(r1 - r0, n, causal, kv_len_b, r0) & bm[(rows // block)[:, None],
                                                           (cols // block)[None, :]]
    p, m, l, seen = _probs(q[r0:r1], k, scale, a)
    lse = np.where(seen, m + np.log(np.where(seen, l, 1.0)), -np.inf)
    do = dout[r0:r1]
    dp = do @ v.T
    ds = p * (dp - (p * dp).sum(axis=1)[:, None])
    return p @ v, lse, scale * (ds @ k), scale * (ds.T @ q[r0:r1]), p.T @ do
