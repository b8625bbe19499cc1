"""The oracle against facts other than itself (closed forms, invariants, library
routines, brute force, finite differences, hand-derived fixtures)."""
import numpy as np
import pytest

import oracle
from tests import pins


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check(oracle.attention_forward, oracle.attention_backward)


def test_row_blocking_is_invisible(monkeypatch):
    """Processing S in row blocks (used at long N) gives the unblocked result."""
    rng = np.random.default_rng(0)
    q, k, v, do = (rng.standard_normal((1, 2, 37, 6)) for _ in range(4))
    kv = np.array([30], np.int32)
    ref_o, ref_l = oracle.attention_forward(q, k, v, 0.4, True, kv)
    ref_g = oracle.attention_backward(q, k, v, do, 0.4, True, kv)
    monkeypatch.setattr("oracle.attention.ROW_BLOCK", 5)
    o, l = oracle.attention_forward(q, k, v, 0.4, True, kv)
    g = oracle.attention_backward(q, k, v, do, 0.4, True, kv)
    assert np.allclose(o, ref_o, atol=1e-14, rtol=0) and np.allclose(l, ref_l, atol=1e-14, rtol=0)
    for a, b in zip(g, ref_g):
        assert np.allclose(a, b, atol=1e-13, rtol=0)


def test_head_parallel_matches_serial():
    rng = np.random.default_rng(1)
    q, k, v, do = (rng.standard_normal((2, 3, 20, 4)) for _ in range(4))
    kv = np.array([7, 20], np.int32)
    o, l = oracle.attention_forward(q, k, v, 0.5, False, kv)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, 0.5, False, kv)
    fw = oracle.attention_forward_heads(q, k, v, 0.5, False, kv, workers=2)
    bw = oracle.attention_backward_heads(q, k, v, do, 0.5, False, kv, workers=2)
    for (b, h), (oh, lh) in fw.items():
        assert np.array_equal(oh, o[b, h]) and np.array_equal(lh, l[b, h])
    for (b, h), (a, bb, c) in bw.items():
        assert np.array_equal(a, dq[b, h]) and np.array_equal(bb, dk[b, h])
        assert np.array_equal(c, dv[b, h])


def test_empty_row_rejected():
    q = np.zeros((1, 1, 3, 2))
    with pytest.raises(ValueError):
        oracle.attention_forward(q, q, q, 1.0, False, np.array([0], np.int32))


def _row_block_fns(block):
    """attention_forward / attention_backward assembled from head_row_block calls over
    row blocks of `block` rows (dK, dV summed over the blocks)."""
    def fwd(q, k, v, scale, causal=False, kv_len=None):
        B, H, N, _ = q.shape
        o, lse = np.empty(q.shape[:3] + (v.shape[3],)), np.empty(q.shape[:3])
        for b in range(B):
            kvb = None if kv_len is None else int(kv_len[b])
            for h in range(H):
                z = np.zeros_like(q[b, h])
                for r0 in range(0, N, block):
                    r1 = min(N, r0 + block)
                    o[b, h, r0:r1], lse[b, h, r0:r1], *_ = oracle.head_row_block(
                        q[b, h], k[b, h], v[b, h], z, scale, causal, kvb, r0, r1)
        return o, lse

    def bwd(q, k, v, dout, scale, causal=False, kv_len=None):
        B, H, N, _ = q.shape
        dq, dk, dv = np.empty(q.shape), np.zeros(k.shape), np.zeros(v.shape)
        for b in range(B):
            kvb = None if kv_len is None else int(kv_len[b])
            for h in range(H):
                for r0 in range(0, N, block):
                    r1 = min(N, r0 + block)
                    _, _, dq[b, h, r0:r1], dkp, dvp = oracle.head_row_block(
                        q[b, h], k[b, h], v[b, h], dout[b, h], scale, causal, kvb, r0, r1)
                    dk[b, h] += dkp
                    dv[b, h] += dvp
        return dq, dk, dv
    return fwd, bwd


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_row_block_pin(check):
    """head_row_block (the definition for a block of query rows, used where a head is
    too long to take whole) meets every pin when the blocks are stitched together."""
    check(*_row_block_fns(3))
