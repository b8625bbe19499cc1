"""Attention with dropout on the probabilities, and the counter-based generator behind
the dropout mask, in float64 / uint64.

TEST INFRASTRUCTURE ONLY (see the package header).

Sources:
- "FlashAttention: Fast and Memory-Efficient Exact Attention with IO-Awareness" (summary
  page of arXiv 2205.14135): Key ideas (kernel fusion) puts dropout inside the fused
  kernel; the FAQ says the method keeps, besides O and the softmax statistics, the state
  of a pseudo-random generator so the dropout mask can be regenerated on chip in the
  backward pass. The page names no generator.
- The generator chosen here is the published counter-based Philox4x64-10 (J. K. Salmon,
  M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel random numbers: as easy as 1, 2, 3",
  SC11): 10 rounds over a 4 x 64-bit counter with a 2 x 64-bit key; each round
  multiplies two counter words by fixed constants, keeps both halves of the 128-bit
  products and mixes them with the other words and the round key; the key advances by
  fixed Weyl increments between rounds.

Readings (where the pages are silent):
- Dropout acts on the normalised probabilities: O = (P * Z / keep) V with Z_ij in {0,1};
  the softmax statistics (and LSE) are those of the undropped scores.
- Random byte of element (b, h, i, j): the Philox4x64-10 block at counter
  (i, j >> 5, b*H + h, 0) with key (seed, offset) gives four 64-bit words; their 32
  little-endian bytes serve the 32 keys j = 32*(j >> 5) ... +31, key j taking byte j & 31.
- p is quantised to t = round(256 p) (0 <= t <= 255); Z_ij = 1 iff the byte >= t; the
  keep probability is (256 - t)/256 and the kept probabilities are scaled by its inverse
  256/(256 - t), so E[Z / keep] = 1 exactly.
- Backward: the chain rule of L = sum(dO * O) through O = (P * Z / keep) V:
  dV = (P * Z / keep)^T dO, dP = (Z / keep) * (dO V^T), D_i = sum_j P_ij dP_ij
  (= sum_k dO_ik O_ik), dS = P * (dP - D), dQ = scale dS K, dK = scale dS^T Q.
"""
from __future__ import annotations

import numpy as np

from .attention import allowed_mask

_M0, _M1 = np.uint64(0xD2E7470EE14C6C93), np.uint64(0xCA5A826395121157)
_W0, _W1 = np.uint64(0x9E3779B97F4A7C15), np.uint64(0xBB67AE8584CAA73B)
_LO32 = np.uint64(0xFFFFFFFF)
_S32 = np.uint64(32)


def _mulhilo(a, m):
    """(hi, lo) 64-bit halves of the 128-bit product a * m (uint64 arrays)."""
    a0, a1 = a & _LO32, a >> _S32
    m0, m1 = m & _LO32, m >> _S32
    p00, p01, p10, p11 = a0 * m0, a0 * m1, a1 * m0, a1 * m1
    mid = (p00 >> _S32) + (p01 & _LO32) + (p10 & _LO32)
    hi = p11 + (p01 >> _S32) + (p10 >> _S32) + (mid >> _S32)
    return hi, a * m


def philox4x64(c0, c1, c2, c3, k0, k1, rounds=10):
    """Philox4x64 block function on uint64 arrays (broadcast): returns four uint64 words."""
    with np.errstate(over="ignore"):
        x0, x1, x2, x3 = (np.asarray(c, dtype=np.uint64) for c in (c0, c1, c2, c3))
        k0 = np.asarray(k0, dtype=np.uint64)
        k1 = np.asarray(k1, dtype=np.uint64)
        for r in range(rounds):
            if r:
                k0, k1 = k0 + _W0, k1 + _W1
            hi0, lo0 = _mulhilo(x0, _M0)
            hi1, lo1 = _mulhilo(x2, _M1)
            x0, x1, x2, x3 = hi1 ^ x1 ^ k0, lo1, hi0 ^ x3 ^ k1, lo0
    return x0, x1, x2, x3


def dropout_threshold(p: float) -> int:
    """t = round(256 p), the byte threshold (keep iff byte >= t)."""
    if not 0.0 <= p < 1.0:
        raise ValueError("dropout probability must be in [0, 1)")
    return min(255, int(np.floor(256.0 * p + 0.5)))


def random_bytes(n_q: int, n_k: int, bh: int, seed: int, offset: int) -> np.ndarray:
    """uint8 [n_q, n_k]: the random byte of every (query, key) element of head bh."""
    i = np.arange(n_q, dtype=np.uint64)[:, None]
    jb = np.arange(-(-n_k // 32), dtype=np.uint64)[None, :]
    words = philox4x64(i, jb, np.uint64(bh), np.uint64(0), np.uint64(seed), np.uint64(offset))
    w = np.stack(np.broadcast_arrays(*words), axis=-1)          # [n_q, n_jb, 4] uint64
    b = w.astype("<u8").view(np.uint8).reshape(n_q, -1)          # little-endian bytes
    return b[:, :n_k]


def keep_mask(n: int, bh: int, p: float, seed: int, offset: int) -> np.ndarray:
    """Boolean [n, n] dropout keep mask Z of head bh."""
    return random_bytes(n, n, bh, seed, offset) >= dropout_threshold(p)


def head_forward_dropout(q, k, v, scale, causal, kv_len_b, z, keep_scale):
    """One head: O = (P * Z * keep_scale) V, LSE of the undropped scores."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    a = allowed_mask(q.shape[0], k.shape[0], causal, kv_len_b)
    s = np.where(a, scale * (q @ k.T), -np.inf)
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    l = e.sum(axis=1)
    p = e / l[:, None]
    return (p * z * keep_scale) @ v, m + np.log(l)


def head_backward_dropout(q, k, v, dout, scale, causal, kv_len_b, z, keep_scale):
    """One head: the chain rule of sum(dout * O) for O = (P * Z * keep_scale) V."""
    q, k, v, dout = (np.asarray(x, dtype=np.float64) for x in (q, k, v, dout))
    a = allowed_mask(q.shape[0], k.shape[0], causal, kv_len_b)
    s = np.where(a, scale * (q @ k.T), -np.inf)
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    p = e / e.sum(axis=1)[:, None]
    pd = p * z * keep_scale
    dv = pd.T @ dout
    dp = (dout @ v.T) * z * keep_scale
    dsum = (p * dp).sum(axis=1)
    d_alt = (dout * (pd @ v)).sum(axis=1)
    if not np.allclose(dsum, d_alt, rtol=0.0, atol=1e-12 * max(1.0, float(np.abs(dsum).max()))):
        raise AssertionError("rowsum(P*dP) != rowsum(dO*O)")
    ds = p * (dp - dsum[:, None])
    return scale * (ds @ k), scale * (ds.T @ q), dv


def _masks(B, H, N, p, seed, offset):
    t = dropout_threshold(p)
    return [[random_bytes(N, N, b * H + h, seed, offset) >= t for h in range(H)]
            for b in range(B)], 256.0 / (256 - t)


def attention_forward_dropout(q, k, v, scale, causal=False, kv_len=None, p=0.0, seed=0,
                              offset=0):
    """[B,H,N,d] -> (O, LSE) with dropout p, generator (seed, offset)."""
    B, H, N, d = q.shape
    zs, ks = _masks(B, H, N, p, seed, offset)
    o = np.empty((B, H, N, v.shape[3]))
    lse = np.empty((B, H, N))
    for b in range(B):
        kvb = None if kv_len is None else int(kv_len[b])
        for h in range(H):
            o[b, h], lse[b, h] = head_forward_dropout(q[b, h], k[b, h], v[b, h], scale,
                                                      causal, kvb, zs[b][h], ks)
    return o, lse


def attention_backward_dropout(q, k, v, dout, scale, causal=False, kv_len=None, p=0.0,
                               seed=0, offset=0):
    """[B,H,N,d] -> (dQ, dK, dV) with the same dropout mask as the forward pass."""
    B, H, N, d = q.shape
    zs, ks = _masks(B, H, N, p, seed, offset)
    dq, dk, dv = (np.empty(q.shape), np.empty(k.shape), np.empty(v.shape))
    for b in range(B):
        kvb = None if kv_len is None else int(kv_len[b])
        for h in range(H):
            dq[b, h], dk[b, h], dv[b, h] = head_backward_dropout(
                q[b, h], k[b, h], v[b, h], dout[b, h], scale, causal, kvb, zs[b][h], ks)
    return dq, dk, dv
