"""The definition of exact attention and its gradient, in float64 on the CPU.

TEST INFRASTRUCTURE ONLY (see the package header).

Sources (page titles and sections):
- "FlashAttention: Fast and Memory-Efficient Exact Attention with IO-Awareness"
  (summary page of arXiv 2205.14135), Problem and motivation: standard attention
  computes S = Q K^T, P = softmax(S), O = P V; FAQ: FlashAttention returns the same
  output as this up to floating-point rounding, so the plain definition is the oracle.
- "[Review] From Online Softmax to Flash Attention", The Self-Attention (X = QK^T,
  A = softmax(X), O = AV) and (safe) softmax (subtracting the row maximum changes
  nothing mathematically and keeps every exponent argument <= 0).
- "Fewer matrix multiplications, same results" (flash-attention issue #941): the
  1/sqrt(head_dim) scale applied to the scores, the [batch, heads, seq, head_dim]
  layout and the causal convention tril(ones(S, S), 0) -- key j is visible to query i
  iff j <= i, diagonal included.
- Same review, the Triton listings: out-of-range keys get a score of -inf, so they
  contribute exactly zero. Per-sequence key padding (key j of batch b is visible iff
  j < kv_len[b]) is read the same way.

The backward pass is not printed on the pages; the summary's Key ideas only say S and
P are recomputed from O and the softmax statistics. It is the textbook chain rule of
L = sum(dO * O) through O = P V and the row softmax:
    dV = P^T dO,  dP = dO V^T,  D_i = sum_j P_ij dP_ij (= sum_k dO_ik O_ik),
    dS = P * (dP - D),  dQ = scale * dS K,  dK = scale * dS^T Q.
Finite differences pin it (tests).

The LSE written by the forward pass is m_i + ln(l_i) in natural log over the scaled,
masked scores (the summary stores l and m; their log-sum-exp is the one number the
backward pass needs).
"""
from __future__ import annotations

import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np

# Rows per block when materialising S: bounds the per-head footprint at long N
# (16384 x 1024 float64 = 128 MiB per S block).
ROW_BLOCK = 1024


def allowed_mask(n_q: int, n_k: int, causal: bool, kv_len_b: int | None,
                 row0: int = 0) -> np.ndarray:
    """Boolean [n_q, n_k] visibility of key j to query row0 + i.

    causal: j <= i (diagonal kept, top-left aligned). kv_len_b: j < kv_len_b.
    """
    i = np.arange(row0, row0 + n_q)[:, None]
    j = np.arange(n_k)[None, :]
    a = np.ones((n_q, n_k), dtype=bool)
    if causal:
        a &= j <= i
    if kv_len_b is not None:
        a &= j < int(kv_len_b)
    return a


def _probs(q_blk, k, scale, causal, kv_len_b, row0):
    """Scaled, masked scores of a block of query rows -> (P, m, l), safe softmax."""
    s = scale * (q_blk @ k.T)
    a = allowed_mask(q_blk.shape[0], k.shape[0], causal, kv_len_b, row0)
    if not a.any(axis=1).all():
        raise ValueError("a query row sees no key: kv_len must be >= 1")
    s = np.where(a, s, -np.inf)
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])  # exactly 0 where masked
    l = e.sum(axis=1)
    return e / l[:, None], m, l


def head_forward(q, k, v, scale, causal=False, kv_len_b=None):
    """One (batch, head): q [N,d], k [N,d], v [N,d] float64 -> (O [N,d], LSE [N])."""
    n = q.shape[0]
    o = np.empty((n, v.shape[1]), dtype=np.float64)
    lse = np.empty(n, dtype=np.float64)
    for r0 in range(0, n, ROW_BLOCK):
        r1 = min(n, r0 + ROW_BLOCK)
        p, m, l = _probs(q[r0:r1], k, scale, causal, kv_len_b, r0)
        o[r0:r1] = p @ v
        lse[r0:r1] = m + np.log(l)
    return o, lse


def head_backward(q, k, v, dout, scale, causal=False, kv_len_b=None, check_d=True):
    """One (batch, head) gradient of L = sum(dout * O) -> (dQ, dK, dV), all [N,d].

    Recomputes P from q, k, v; takes nothing from a forward pass.
    """
    n = q.shape[0]
    dq = np.empty_like(q, dtype=np.float64)
    dk = np.zeros_like(k, dtype=np.float64)
    dv = np.zeros_like(v, dtype=np.float64)
    for r0 in range(0, n, ROW_BLOCK):
        r1 = min(n, r0 + ROW_BLOCK)
        p, _, _ = _probs(q[r0:r1], k, scale, causal, kv_len_b, r0)
        do = dout[r0:r1]
        dv += p.T @ do
        dp = do @ v.T
        dsum = (p * dp).sum(axis=1)
        if check_d:
            # the same D from the forward output: D_i = sum_k dO_ik O_ik
            d_alt = (do * (p @ v)).sum(axis=1)
            tol = 1e-12 * max(1.0, float(np.abs(dsum).max(initial=0.0)))
            if not np.allclose(dsum, d_alt, rtol=0.0, atol=tol * 16):
                raise AssertionError("rowsum(P*dP) != rowsum(dO*O)")
        ds = p * (dp - dsum[:, None])
        dq[r0:r1] = scale * (ds @ k)
        dk += scale * (ds.T @ q[r0:r1])
    return dq, dk, dv


def head_row_block(q, k, v, dout, scale, causal, kv_len_b, r0, r1):
    """The definition restricted to query rows r0 .. r1-1 of one head, for heads too long
    to take whole: (O, LSE, dQ) of those rows, and their contributions to dK and dV
    (scale dS^T Q and P^T dO summed over those rows, for every key). It is the body of
    head_forward / head_backward for one row block; under the causal mask the last row
    block's contributions are the whole dK and dV of the keys inside it."""
    q, k, v, dout = (np.asarray(x, dtype=np.float64) for x in (q, k, v, dout))
    p, m, l = _probs(q[r0:r1], k, scale, causal, kv_len_b, r0)
    do = dout[r0:r1]
    dp = do @ v.T
    ds = p * (dp - (p * dp).sum(axis=1)[:, None])
    return (p @ v, m + np.log(l), scale * (ds @ k), scale * (ds.T @ q[r0:r1]), p.T @ do)


def _kv(kv_len, b):
    return None if kv_len is None else int(kv_len[b])


def attention_forward(q, k, v, scale, causal=False, kv_len=None):
    """[B,H,N,d] float64 -> (O [B,H,N,d], LSE [B,H,N]), serial over heads."""
    B, H, N, d = q.shape
    o = np.empty((B, H, N, v.shape[3]))
    lse = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h] = head_forward(q[b, h], k[b, h], v[b, h], scale,
                                              causal, _kv(kv_len, b))
    return o, lse


def attention_backward(q, k, v, dout, scale, causal=False, kv_len=None):
    """[B,H,N,d] float64 -> (dQ, dK, dV), serial over heads."""
    B, H, N, d = q.shape
    dq, dk, dv = (np.empty_like(q), np.empty_like(k), np.empty_like(v))
    for b in range(B):
        for h in range(H):
            dq[b, h], dk[b, h], dv[b, h] = head_backward(
                q[b, h], k[b, h], v[b, h], dout[b, h], scale, causal, _kv(kv_len, b))
    return dq, dk, dv


# ---- head-parallel drivers (process pool, one BLAS thread per worker) -------------

def _worker_init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # pragma: no cover - threadpoolctl is optional
        pass


def _fwd_job(args):
    q, k, v, scale, causal, kvb = args
    return head_forward(q, k, v, scale, causal, kvb)


def _bwd_job(args):
    q, k, v, do, scale, causal, kvb = args
    return head_backward(q, k, v, do, scale, causal, kvb)


def default_workers() -> int:
    """Worker processes for the per-head pools: the cores this process may run on, at
    most 16 (a GPU host's CPU share per GPU here, whatever the affinity mask shows)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def attention_forward_heads(q, k, v, scale, causal=False, kv_len=None, heads=None,
                            workers=None):
    """Forward for a list of (b, h) heads (all heads when None), in a process pool.

    Returns {(b, h): (O, LSE)}.
    """
    B, H = q.shape[:2]
    heads = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    jobs = [(q[b, h], k[b, h], v[b, h], scale, causal, _kv(kv_len, b)) for b, h in heads]
    workers = workers or default_workers()
    if workers <= 1 or len(jobs) <= 1:
        res = [_fwd_job(j) for j in jobs]
    else:
        with ProcessPoolExecutor(max_workers=min(workers, len(jobs)),
                                 initializer=_worker_init) as ex:
            res = list(ex.map(_fwd_job, jobs))
    return dict(zip(heads, res))


def attention_backward_heads(q, k, v, dout, scale, causal=False, kv_len=None, heads=None,
                             workers=None):
    """Backward for a list of (b, h) heads, in a process pool. Returns {(b,h): (dQ,dK,dV)}."""
    B, H = q.shape[:2]
    heads = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    jobs = [(q[b, h], k[b, h], v[b, h], dout[b, h], scale, causal, _kv(kv_len, b))
            for b, h in heads]
    workers = workers or default_workers()
    if workers <= 1 or len(jobs) <= 1:
        res = [_bwd_job(j) for j in jobs]
    else:
        with ProcessPoolExecutor(max_workers=min(workers, len(jobs)),
                                 initializer=_worker_init) as ex:
            res = list(ex.map(_bwd_job, jobs))
    return dict(zip(heads, res))
