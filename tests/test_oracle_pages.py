"""The recurrences the pages derive, written as scalar loops, reproduce the definition
(and the softmax helpers reproduce scipy's softmax) on tiny and adversarial inputs."""
import math

import numpy as np
import pytest
import scipy.special

import oracle
from oracle import page_algorithms as pa

NEG = -math.inf


def _vis(N, causal, kvb):
    return [[(not causal or j <= i) and (kvb is None or j < kvb) for j in range(N)]
            for i in range(N)]


def _adversarial_vectors(rng):
    out = [list(rng.standard_normal(9))]
    out.append(list(rng.standard_normal(12) * 1e3))          # overflows without the shift
    x = list(rng.standard_normal(10)); x[-1] = 50.0; out.append(x)   # max only at the end
    out.append([2.0, 5.0, 5.0, -1.0, 5.0])                     # tied maxima
    out.append([0.3, NEG, NEG, 1.2, NEG])                       # masked entries
    out.append([7.0])
    return out


@pytest.mark.parametrize("fn", [pa.softmax_three_pass, pa.softmax_online_two_pass])
def test_softmax_algorithms_match_scipy(fn):
    rng = np.random.default_rng(0)
    for x in _adversarial_vectors(rng):
        ref = scipy.special.softmax(np.array(x))
        got = np.array(fn(x))
        assert np.all(np.abs(got - ref) <= 1e-15 + 1e-13 * ref), (x, got, ref)
        assert abs(sum(got) - 1.0) < 1e-14


def test_merge_stats_matches_logsumexp():
    rng = np.random.default_rng(1)
    for _ in range(20):
        x = rng.standard_normal(11) * 5
        cut = int(rng.integers(1, 10))
        a, b = x[:cut], x[cut:]
        m1, l1 = a.max(), np.exp(a - a.max()).sum()
        m2, l2 = b.max(), np.exp(b - b.max()).sum()
        m, l = pa.merge_stats(m1, l1, m2, l2)
        assert m == x.max()
        assert abs(m + math.log(l) - scipy.special.logsumexp(x)) < 1e-13
    assert pa.merge_stats(NEG, 0.0, 1.5, 2.0) == (1.5, 2.0)


def _row_cases():
    rng = np.random.default_rng(2)
    for N, d, causal, kvb, qs in [(1, 1, False, None, 1.0), (7, 3, False, None, 1.0),
                                 (16, 4, True, None, 1.0), (13, 5, False, 9, 1.0),
                                 (12, 2, True, 5, 1.0), (10, 3, False, None, 300.0)]:
        q = rng.standard_normal((N, d)) * qs
        k = rng.standard_normal((N, d))
        v = rng.standard_normal((N, d))
        if N >= 10:
            k[-1] = q.mean(0) * 4  # a large score that appears only in the last key
        yield N, d, causal, kvb, q, k, v


@pytest.mark.parametrize("algo", ["two_pass", "one_pass", "tiled"])
def test_row_algorithms_match_definition(algo):
    for N, d, causal, kvb, q, k, v in _row_cases():
        scale = 0.55
        o_ref, l_ref = oracle.head_forward(q, k, v, scale, causal, kvb)
        vis = _vis(N, causal, kvb)
        widths = [1, 3, 4, N] if algo == "tiled" else [None]
        for b in widths:
            for r in range(N):
                if algo == "two_pass":
                    o, l = pa.attention_row_two_pass(q[r], k, v, scale, vis[r])
                elif algo == "one_pass":
                    o, l = pa.attention_row_one_pass(q[r], k, v, scale, vis[r])
                else:
                    o, l = pa.attention_row_tiled(q[r], k, v, b, scale, vis[r])
                tol = 1e-12 * max(1.0, abs(l_ref[r]))
                assert np.max(np.abs(np.array(o) - o_ref[r])) < 1e-12, (algo, N, b, r)
                assert abs(l - l_ref[r]) < tol, (algo, N, b, r)


def test_block_form_matches_definition():
    for N, d, causal, kvb, q, k, v in _row_cases():
        o_ref, l_ref = oracle.head_forward(q, k, v, 0.55, causal, kvb)
        vis = _vis(N, causal, kvb)
        for br, bc in [(1, 1), (3, 4), (4, 3), (5, 2), (N, N)]:
            o, l = pa.attention_blocks(q, k, v, br, bc, 0.55, vis)
            assert np.max(np.abs(o - o_ref)) < 1e-12, (N, br, bc)
            assert np.max(np.abs(l - l_ref)) < 1e-12 * max(1, np.abs(l_ref).max())


def test_flashatt_spec_is_attention_with_unit_head_dim():
    rng = np.random.default_rng(3)
    q, k, v = rng.standard_normal(6), rng.standard_normal(9), rng.standard_normal(9)
    z = np.array(pa.flashatt_spec(q, k, v))
    # one query row per entry of q, head_dim 1, scale 1, no mask, T = 9 keys
    o, _ = oracle.head_forward(q[:, None], k[:, None], v[:, None], 1.0)
    assert np.max(np.abs(z - o[:, 0])) < 1e-13
    # and against scipy's softmax written out
    ref = [(scipy.special.softmax(qi * k) * v).sum() for qi in q]
    assert np.max(np.abs(z - np.array(ref))) < 1e-13


def _rising_case(N=23, d=3, step=2.0):
    """Scores that rise along the keys, so every key block raises the running maximum
    and every earlier numerator block must be rescaled."""
    rng = np.random.default_rng(8)
    q = np.zeros((N, d))
    q[:, 0] = 1.0 + 0.1 * rng.random(N)
    k = 0.1 * rng.standard_normal((N, d))
    k[:, 0] = step * np.arange(N)
    v = rng.standard_normal((N, d))
    return q, k, v


def test_deferred_pv_matches_definition():
    cases = list(_row_cases())
    q, k, v = _rising_case()
    cases += [(23, 3, False, None, q, k, v), (23, 3, True, None, q, k, v),
              (23, 3, False, 17, q, k, v)]
    for N, d, causal, kvb, q, k, v in cases:
        o_ref, l_ref = oracle.head_forward(q, k, v, 0.55, causal, kvb)
        vis = _vis(N, causal, kvb)
        for blk in sorted({1, 3, 4, 5, N}):
            o, l = pa.attention_deferred_pv(q, k, v, blk, 0.55, vis)
            assert np.max(np.abs(o - o_ref)) < 1e-12, (N, blk)
            assert np.max(np.abs(l - l_ref)) < 1e-12 * max(1, np.abs(l_ref).max()), (N, blk)


def test_deferred_pv_needs_its_rescale():
    """The rising case separates the rule from a variant that leaves the earlier blocks
    unscaled (which stays exact only while the maximum never moves)."""
    q, k, v = _rising_case()
    vis = _vis(23, False, None)
    o_ref, _ = oracle.head_forward(q, k, v, 0.55, False, None)
    # the variant, by hand: numerators kept relative to their own block maximum
    blk = 4
    F, m_all = [], []
    for j0 in range(0, 23, blk):
        S = 0.55 * (q @ k[j0:j0 + blk].T)
        m_loc = S.max(axis=1)
        F.append(np.exp(S - m_loc[:, None]))
        m_all.append(m_loc)
    m_fin = np.max(np.stack(m_all, 1), axis=1)
    l_wrong = sum(f.sum(1) * np.exp(m - m_fin) for f, m in zip(F, m_all))
    o_wrong = (np.concatenate(F, 1) / l_wrong[:, None]) @ v
    assert np.max(np.abs(o_wrong - o_ref)) > 1e-3
    o, _ = pa.attention_deferred_pv(q, k, v, blk, 0.55, vis)
    assert np.max(np.abs(o - o_ref)) < 1e-12
