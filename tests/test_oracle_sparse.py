"""The block-sparse oracle against facts other than itself: the dense definition (all-ones
mask, a mask that adds nothing to the causal rule), independent sub-problems (a
block-diagonal mask), scalar brute force, finite differences, closed forms for empty
rows, and planted mistakes that those pins must catch."""
import math

import numpy as np
import pytest

import oracle
from oracle import sparse as SP


def _inputs(B, H, N, d, seed, q_mult=1.0):
    rng = np.random.default_rng(seed)
    q, k, v, do = (rng.standard_normal((B, H, N, d)) for _ in range(4))
    return q * q_mult, k, v, do


def _close(a, b, tol, what):
    a, b = np.asarray(a), np.asarray(b)
    assert np.array_equal(np.isneginf(a), np.isneginf(b)), f"{what}: -inf pattern differs"
    f = ~np.isneginf(b)
    err = float(np.abs(a[f] - b[f]).max(initial=0.0))
    assert err <= tol, f"{what}: {err:.3e} > {tol:.1e}"


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("pad", [False, True])
def test_all_ones_mask_is_dense(causal, pad):
    B, H, N, d, blk = 2, 2, 23, 4, 5
    q, k, v, do = _inputs(B, H, N, d, 1, 2.0)
    kv = np.array([9, 23], np.int32) if pad else None
    nb = -(-N // blk)
    ones = np.ones((nb, nb), np.uint8)
    o, l = oracle.attention_forward_sparse(q, k, v, 0.6, causal, kv, ones, blk)
    ro, rl = oracle.attention_forward(q, k, v, 0.6, causal, kv)
    _close(o, ro, 1e-13, "O")
    _close(l, rl, 1e-13, "LSE")
    g = oracle.attention_backward_sparse(q, k, v, do, 0.6, causal, kv, ones, blk)
    rg = oracle.attention_backward(q, k, v, do, 0.6, causal, kv)
    for a, b, n in zip(g, rg, ("dQ", "dK", "dV")):
        _close(a, b, 1e-12, n)


def test_lower_block_triangle_adds_nothing_to_causal():
    B, H, N, d, blk = 1, 2, 30, 3, 7
    q, k, v, do = _inputs(B, H, N, d, 2)
    nb = -(-N // blk)
    tri = np.tril(np.ones((nb, nb), np.uint8))
    o, l = oracle.attention_forward_sparse(q, k, v, 0.5, True, None, tri, blk)
    ro, rl = oracle.attention_forward(q, k, v, 0.5, True)
    _close(o, ro, 1e-13, "O")
    _close(l, rl, 1e-13, "LSE")


@pytest.mark.parametrize("causal", [False, True])
def test_block_diagonal_is_independent_blocks(causal):
    """With only diagonal blocks on, each query block attends within its own key block:
    the same as running the dense definition on each block alone."""
    B, H, N, d, blk = 1, 2, 26, 4, 8
    q, k, v, do = _inputs(B, H, N, d, 3, 1.5)
    nb = -(-N // blk)
    diag = np.eye(nb, dtype=np.uint8)
    o, l = oracle.attention_forward_sparse(q, k, v, 0.7, causal, None, diag, blk)
    dq, dk, dv = oracle.attention_backward_sparse(q, k, v, do, 0.7, causal, None, diag, blk)
    for i0 in range(0, N, blk):
        sl = slice(i0, min(N, i0 + blk))
        ro, rl = oracle.attention_forward(q[:, :, sl], k[:, :, sl], v[:, :, sl], 0.7, causal)
        rq, rk, rv = oracle.attention_backward(q[:, :, sl], k[:, :, sl], v[:, :, sl],
                                               do[:, :, sl], 0.7, causal)
        _close(o[:, :, sl], ro, 1e-13, "O block")
        _close(l[:, :, sl], rl, 1e-13, "LSE block")
        for a, b, n in ((dq[:, :, sl], rq, "dQ"), (dk[:, :, sl], rk, "dK"),
                        (dv[:, :, sl], rv, "dV")):
            _close(a, b, 1e-12, n + " block")


def test_empty_rows():
    """A query block with every key block off: O = 0, LSE = -inf, dQ = 0, and its dO
    changes no dK or dV."""
    B, H, N, d, blk = 1, 1, 16, 3, 4
    q, k, v, do = _inputs(B, H, N, d, 4)
    bm = np.ones((4, 4), np.uint8)
    bm[2] = 0
    o, l = oracle.attention_forward_sparse(q, k, v, 0.5, False, None, bm, blk)
    assert np.all(np.isneginf(l[0, 0, 8:12])) and np.all(o[0, 0, 8:12] == 0)
    assert np.all(np.isfinite(l[0, 0, :8])) and np.all(np.isfinite(l[0, 0, 12:]))
    dq, dk, dv = oracle.attention_backward_sparse(q, k, v, do, 0.5, False, None, bm, blk)
    assert np.all(dq[0, 0, 8:12] == 0)
    do2 = do.copy()
    do2[0, 0, 8:12] = 123.0
    _, dk2, dv2 = oracle.attention_backward_sparse(q, k, v, do2, 0.5, False, None, bm, blk)
    assert np.array_equal(dk, dk2) and np.array_equal(dv, dv2)


def test_brute_force():
    B, H, N, d, blk = 1, 1, 11, 2, 3
    q, k, v, do = _inputs(B, H, N, d, 5, 2.0)
    rng = np.random.default_rng(6)
    bm = (rng.random((4, 4)) < 0.6).astype(np.uint8)
    kv = np.array([9], np.int32)
    for causal in (False, True):
        o, l = oracle.attention_forward_sparse(q, k, v, 0.8, causal, kv, bm, blk)
        for i in range(N):
            js = [j for j in range(N) if j < 9 and (not causal or j <= i)
                  and bm[i // blk, j // blk]]
            if not js:
                assert l[0, 0, i] == -math.inf and np.all(o[0, 0, i] == 0)
                continue
            s = [0.8 * math.fsum(q[0, 0, i, t] * k[0, 0, j, t] for t in range(d)) for j in js]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            z = math.fsum(w)
            assert abs(l[0, 0, i] - (m + math.log(z))) < 1e-13
            for t in range(d):
                ref = math.fsum(wj * v[0, 0, j, t] for wj, j in zip(w, js)) / z
                assert abs(o[0, 0, i, t] - ref) < 1e-13


def test_finite_differences():
    B, H, N, d, blk = 1, 1, 9, 3, 3
    q, k, v, do = _inputs(B, H, N, d, 7)
    bm = np.array([[1, 0, 1], [0, 1, 0], [1, 1, 0]], np.uint8)
    grads = oracle.attention_backward_sparse(q, k, v, do, 0.9, True, None, bm, blk)
    h = 1e-6
    for which in range(3):
        xs = [q, k, v]
        fd = np.zeros_like(xs[which])
        for idx in np.ndindex(*xs[which].shape):
            xp = [x.copy() for x in xs]
            xm = [x.copy() for x in xs]
            xp[which][idx] += h
            xm[which][idx] -= h
            lp = (oracle.attention_forward_sparse(*xp, 0.9, True, None, bm, blk)[0] * do).sum()
            lm = (oracle.attention_forward_sparse(*xm, 0.9, True, None, bm, blk)[0] * do).sum()
            fd[idx] = (lp - lm) / (2 * h)
        _close(grads[which], fd, 1e-7, "QKV"[which] + " finite differences")


# ---- planted mistakes ------------------------------------------------------------------

_block_allowed = SP.block_allowed


def _transposed(n, causal, kv_len_b, block_mask, block):
    return _block_allowed(n, causal, kv_len_b, np.asarray(block_mask).T, block)


def _block_off_by_one(n, causal, kv_len_b, block_mask, block):
    bm = np.asarray(block_mask) != 0
    idx = np.minimum(np.arange(n) // (block + 1), bm.shape[0] - 1)
    return oracle.allowed_mask(n, n, causal, kv_len_b) & bm[idx[:, None], idx[None, :]]


def _ignores_mask(n, causal, kv_len_b, block_mask, block):
    return oracle.allowed_mask(n, n, causal, kv_len_b)


@pytest.mark.parametrize("mutant", [_transposed, _block_off_by_one, _ignores_mask],
                         ids=lambda f: f.__name__)
def test_mask_mutants_are_caught(monkeypatch, mutant):
    monkeypatch.setattr(SP, "block_allowed", mutant)
    caught = False
    try:
        test_brute_force()
        test_block_diagonal_is_independent_blocks(False)
        test_empty_rows()
    except AssertionError:
        caught = True
    assert caught, f"{mutant.__name__} was not caught"


@pytest.mark.parametrize("causal,kvb", [(False, None), (True, None), (False, 23), (True, 30)])
def test_row_block_sparse_stitches_to_the_head_functions(causal, kvb):
    """head_row_block_sparse over row blocks (ragged, some rows with no visible key)
    reproduces head_forward_sparse and head_backward_sparse, which the tests above pin."""
    rng = np.random.default_rng(40)
    N, d, blk = 37, 5, 8
    q, k, v, do = (rng.standard_normal((N, d)) for _ in range(4))
    nb = -(-N // blk)
    m = (rng.random((nb, nb)) < 0.6).astype(np.uint8)
    m[1] = 0                                         # a block row with no visible key
    ro, rl = oracle.head_forward_sparse(q, k, v, 0.7, causal, kvb, m, blk)
    rq, rk, rv = oracle.head_backward_sparse(q, k, v, do, 0.7, causal, kvb, m, blk)
    o, lse, dq = np.empty_like(ro), np.empty_like(rl), np.empty_like(rq)
    dk, dv = np.zeros_like(rk), np.zeros_like(rv)
    for r0 in range(0, N, 6):
        r1 = min(N, r0 + 6)
        o[r0:r1], lse[r0:r1], dq[r0:r1], dkp, dvp = oracle.head_row_block_sparse(
            q, k, v, do, 0.7, causal, kvb, m, r0, r1, blk)
        dk += dkp
        dv += dvp
    assert np.array_equal(np.isneginf(lse), np.isneginf(rl))
    fin = ~np.isneginf(rl)
    assert np.abs(lse[fin] - rl[fin]).max() < 1e-12
    for a, b in ((o, ro), (dq, rq), (dk, rk), (dv, rv)):
        assert np.abs(a - b).max() < 1e-12
