"""Attention with dropout on the probabilities, and the counter-based generator behind
the dropout mask, in float64 / uint64.

TEST INFRASTRUCTURE ONLY (see the package header).

Sources:
- "FlashAttention: Fast and Memory-Efficient Exact Attention with IO-Awareness" (summary
  page of arXiv 2205.14135): Key ideas (kernel fusion) puts dropout inside the fused
  kernel; the FAQ says the method keeps, besides O and the softmax statistics, the state
  of a pseudo-random generator so the dropout mask can be regenerated on chip in the
  backward pass. The page names no generator.
- The generator chosen here is the published counter-based Philox4x32-10 (J. K. Salmon,
  M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel random numbers: as easy as 1, 2, 3",
  SC11): 10 rounds over a 4 x 32-bit counter with a 2 x 32-bit key; each round
  multiplies two counter words by fixed constants, keeps both halves of the 64-bit
  products and mixes them with the other words and the round key; the key advances by
  fixed Weyl increments between rounds.

Readings (where the pages are silent):
- Dropout acts on the normalised probabilities: O = (P * Z / keep) V with Z_ij in {0,1};
  the softmax statistics (and LSE) are those of the undropped scores.
- Random byte of element (b, h, i, j): keys fall in groups of 32 (g = j >> 5, u = j & 31).
  The group's 32 bytes come from two Philox4x32-10 blocks, at counters (i, 2g, b*H + h,
  offset) and (i, 2g + 1, b*H + h, offset) with key (seed mod 2^32, seed >> 32); each
  block gives 16 bytes (its four words, little-endian). Key u takes block 2g + ((u >> 3)
  & 1), byte 8*(u >> 4) + (u & 7): keys 0-7 and 16-23 of the group read bytes 0-7 and
  8-15 of the first block, keys 8-15 and 24-31 those of the second.
- p is quantised to the byte threshold t whose keep probability (256 - t)/256 lies
  nearest to 1 - p on the 1/256 grid, i.e. t = round(256 p) with halves rounded up,
  capped at 255; Z_ij = 1 iff the byte >= t; the kept probabilities are scaled by the
  inverse of the keep probability, 256/(256 - t), so E[Z / keep] = 1 exactly. p is a
  32-bit float parameter of the library's entry points, so t is derived from p rounded
  to float32 (then 256 p + 1/2 in float64, floored), the same arithmetic on both sides.
- Backward: the chain rule of L = sum(dO * O) through O = (P * Z / keep) V:
  dV = (P * Z / keep)^T dO, dP = (Z / keep) * (dO V^T), D_i = sum_j P_ij dP_ij
  (= sum_k dO_ik O_ik), dS = P * (dP - D), dQ = scale dS K, dK = scale dS^T Q.
"""
from __future__ import annotations

import numpy as np

from .attention import allowed_mask

_M0, _M1 = np.uint64(0xD2511F53), np.uint64(0xCD9E8D57)
_W0, _W1 = np.uint64(0x9E3779B9), np.uint64(0xBB67AE85)
_LO32 = np.uint64(0xFFFFFFFF)
_S32 = np.uint64(32)


def philox4x32(c0, c1, c2, c3, k0, k1, rounds=10):
    """Philox4x32 block function on arrays of 32-bit values (held in uint64, broadcast):
    returns the four output words as uint32 arrays."""
    x0, x1, x2, x3, k0, k1 = (np.asarray(c, dtype=np.uint64) & _LO32
                              for c in (c0, c1, c2, c3, k0, k1))
    for r in range(rounds):
        if r:
            k0, k1 = (k0 + _W0) & _LO32, (k1 + _W1) & _LO32
        p0 = x0 * _M0                      # exact: both factors are below 2^32
        p1 = x2 * _M1
        x0, x1, x2, x3 = (p1 >> _S32) ^ x1 ^ k0, p1 & _LO32, (p0 >> _S32) ^ x3 ^ k1, p0 & _LO32
    return tuple(x.astype(np.uint32) for x in (x0, x1, x2, x3))


def dropout_threshold(p: float) -> int:
    """The byte threshold t (keep iff byte >= t): round(256 p), halves up, at most 255,
    with p taken as the float32 the entry points receive."""
    p32 = float(np.float32(p))
    if not 0.0 <= p32 < 1.0:
        raise ValueError("dropout probability must be in [0, 1)")
    return min(255, int(np.floor(256.0 * p32 + 0.5)))


def keep_scale(p: float) -> float:
    """1 / keep probability = 256 / (256 - t): the factor on kept probabilities."""
    return 256.0 / (256 - dropout_threshold(p))


def _check_key(seed: int, offset: int):
    if not (0 <= seed < 1 << 64 and 0 <= offset < 1 << 32):
        raise ValueError("seed is an unsigned 64-bit and offset an unsigned 32-bit integer")


def random_bytes(n_q: int, n_k: int, bh: int, seed: int, offset: int) -> np.ndarray:
    """uint8 [n_q, n_k]: the random byte of every (query, key) element of head bh."""
    _check_key(seed, offset)
    n_blk = 2 * (-(-n_k // 32))
    i = np.arange(n_q, dtype=np.uint64)[:, None]
    jb = np.arange(n_blk, dtype=np.uint64)[None, :]
    words = philox4x32(i, jb, bh, offset, seed & 0xFFFFFFFF, seed >> 32)
    w = np.stack(np.broadcast_arrays(*words), axis=-1).astype("<u4")    # [n_q, n_blk, 4]
    blk_bytes = w.view(np.uint8).reshape(n_q, n_blk, 16)
    j = np.arange(n_k)
    u = j & 31
    block = 2 * (j >> 5) + ((u >> 3) & 1)
    byte = 8 * (u >> 4) + (u & 7)
    return blk_bytes[:, block, byte]


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
            for b in range(B)], keep_scale(p)


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
