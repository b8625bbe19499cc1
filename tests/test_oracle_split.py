"""The split-KV oracle (partial attention over key ranges, merge of partials) against
facts other than itself: hand-derived cases, the unsplit definition, scalar brute force,
invariants of the merge, and planted mistakes that those pins must catch."""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import split as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "split_merge_cases.json")


def _ev(x):
    """A fixture entry: number, expression in +-*/ and ln(), or null (= -inf)."""
    if isinstance(x, list):
        return [_ev(e) for e in x]
    if x is None:
        return -math.inf
    if isinstance(x, str):
        return float(eval(x, {"__builtins__": {}}, {"ln": math.log}))  # noqa: S307
    return float(x)


def _same(a, b, tol, what):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    inf_a, inf_b = np.isneginf(a), np.isneginf(b)
    assert np.array_equal(inf_a, inf_b), f"{what}: -inf pattern differs"
    fin = ~inf_a
    err = float(np.abs(a[fin] - b[fin]).max(initial=0.0))
    assert err <= tol, f"{what}: max-abs error {err:.3e} > {tol:.1e}"


def _cases(kind):
    with open(GOLDEN) as f:
        return json.load(f)[kind]


@pytest.mark.parametrize("case", _cases("split_cases"), ids=lambda c: c["name"])
def test_golden_split(case):
    q, k, v = (np.array(_ev(case[n]))[None, None] for n in "qkv")
    kv = None if case["kv_len"] is None else np.array(case["kv_len"], np.int32)
    o_p, l_p = oracle.attention_forward_split(q, k, v, case["scale"], case["causal"], kv,
                                              case["split_len"])
    _same(o_p[:, 0, 0], _ev(case["O_parts"]), 1e-14, f"{case['name']}: O_parts")
    _same(l_p[:, 0, 0], _ev(case["LSE_parts"]), 1e-14, f"{case['name']}: LSE_parts")
    o, l = oracle.merge_partials(o_p, l_p)
    _same(o[0, 0], _ev(case["O"]), 1e-14, f"{case['name']}: merged O")
    _same(l[0, 0], _ev(case["LSE"]), 1e-14, f"{case['name']}: merged LSE")


@pytest.mark.parametrize("case", _cases("merge_cases"), ids=lambda c: c["name"])
def test_golden_merge(case):
    o_p = np.array(_ev(case["O_parts"]))
    l_p = np.array(_ev(case["LSE_parts"]))
    o, l = oracle.merge_partials(o_p, l_p)
    _same(o, _ev(case["O"]), 1e-12, f"{case['name']}: O")
    _same(l, _ev(case["LSE"]), 1e-12, f"{case['name']}: LSE")


def _inputs(B, H, N, d, seed, q_mult=1.0):
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal((B, H, N, d)) for _ in range(3))
    return q * q_mult, k, v


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("pad", [False, True])
@pytest.mark.parametrize("split_len", [1, 3, 7, 16, 40, 41, 100])
def test_merge_of_splits_is_unsplit_attention(causal, pad, split_len):
    """Merging the partials of every key range gives the definition's O and LSE."""
    B, H, N, d = 2, 2, 41, 5
    q, k, v = _inputs(B, H, N, d, 3 + split_len, q_mult=3.0)
    kv = np.array([17, 41], np.int32) if pad else None
    o_ref, l_ref = oracle.attention_forward(q, k, v, 0.45, causal, kv)
    o_p, l_p = oracle.attention_forward_split(q, k, v, 0.45, causal, kv, split_len)
    assert o_p.shape[0] == -(-N // split_len)
    o, l = oracle.merge_partials(o_p, l_p)
    _same(o, o_ref, 1e-12, "merged O vs unsplit O")
    _same(l, l_ref, 1e-12, "merged LSE vs unsplit LSE")


def test_partial_brute_force():
    """Each partial equals scalar sums over the range's visible keys (math.fsum)."""
    B, H, N, d = 1, 2, 13, 3
    q, k, v = _inputs(B, H, N, d, 11, q_mult=2.0)
    kv = np.array([11], np.int32)
    for causal in (False, True):
        o_p, l_p = oracle.attention_forward_split(q, k, v, 0.7, causal, kv, 4)
        for p, (kb, ke) in enumerate(S.split_ranges(N, 4)):
            for h in range(H):
                for i in range(N):
                    js = [j for j in range(kb, ke) if j < 11 and (not causal or j <= i)]
                    if not js:
                        assert l_p[p, 0, h, i] == -math.inf
                        assert np.all(o_p[p, 0, h, i] == 0.0)
                        continue
                    s = [0.7 * math.fsum(q[0, h, i, t] * k[0, h, j, t] for t in range(d))
                         for j in js]
                    m = max(s)
                    w = [math.exp(x - m) for x in s]
                    z = math.fsum(w)
                    for t in range(d):
                        ref = math.fsum(wj * v[0, h, j, t] for wj, j in zip(w, js)) / z
                        assert abs(o_p[p, 0, h, i, t] - ref) < 1e-13
                    assert abs(l_p[p, 0, h, i] - (m + math.log(z))) < 1e-13


def test_merge_order_and_grouping_do_not_matter():
    rng = np.random.default_rng(5)
    P, N, d = 5, 9, 4
    o_p = rng.standard_normal((P, N, d))
    l_p = 30.0 * rng.standard_normal((P, N))
    l_p[1, 2] = -np.inf
    o_p[1, 2] = 0.0
    o_ref, l_ref = oracle.merge_partials(o_p, l_p)
    perm = rng.permutation(P)
    o2, l2 = oracle.merge_partials(o_p[perm], l_p[perm])
    _same(o2, o_ref, 1e-12, "permuted O")
    _same(l2, l_ref, 1e-12, "permuted LSE")
    oa, la = oracle.merge_partials(o_p[:2], l_p[:2])
    ob, lb = oracle.merge_partials(o_p[2:], l_p[2:])
    o3, l3 = oracle.merge_pair(oa, la, ob, lb)
    _same(o3, o_ref, 1e-12, "grouped O")
    _same(l3, l_ref, 1e-12, "grouped LSE")


def test_single_split_and_empty_partials():
    q, k, v = _inputs(1, 1, 10, 4, 8)
    o_ref, l_ref = oracle.attention_forward(q, k, v, 0.5, True)
    o_p, l_p = oracle.attention_forward_split(q, k, v, 0.5, True, None, 10)
    assert o_p.shape[0] == 1
    _same(o_p[0], o_ref, 1e-14, "one split = unsplit O")
    _same(l_p[0], l_ref, 1e-14, "one split = unsplit LSE")
    # rows before the range start see nothing of it (causal)
    o_p, l_p = oracle.attention_forward_split(q, k, v, 0.5, True, None, 4)
    assert np.all(np.isneginf(l_p[1, 0, 0, :4])) and np.all(o_p[1, 0, 0, :4] == 0)
    assert np.all(np.isfinite(l_p[1, 0, 0, 4:]))


# ---- planted mistakes: each must make a pin above fail --------------------------------

_merge_pair = S.merge_pair  # the original, for mutants built on it

def _merge_no_shift(o1, l1, o2, l2):
    w1, w2 = np.exp(l1), np.exp(l2)
    return (w1[..., None] * o1 + w2[..., None] * o2) / (w1 + w2)[..., None], np.log(w1 + w2)


def _merge_no_normalise(o1, l1, o2, l2):
    m = np.maximum(l1, l2)
    w1, w2 = np.exp(l1 - m), np.exp(l2 - m)
    return w1[..., None] * o1 + w2[..., None] * o2, m + np.log(w1 + w2)


def _merge_lse_no_log(o1, l1, o2, l2):
    o, l = _merge_pair(o1, l1, o2, l2)
    m = np.maximum(l1, l2)
    return o, m + np.exp(l1 - m) + np.exp(l2 - m) - 1.0


def _merge_swapped(o1, l1, o2, l2):
    return _merge_pair(o2, l1, o1, l2)


@pytest.mark.parametrize("mutant", [_merge_no_shift, _merge_no_normalise, _merge_lse_no_log,
                                    _merge_swapped], ids=lambda f: f.__name__)
def test_merge_mutants_are_caught(monkeypatch, mutant):
    monkeypatch.setattr(S, "merge_pair", mutant)
    caught = False
    with np.errstate(all="ignore"):
        try:
            for case in _cases("merge_cases") + _cases("split_cases"):
                if "q" in case:
                    test_golden_split(case)
                else:
                    test_golden_merge(case)
            test_merge_of_splits_is_unsplit_attention(True, True, 7)
        except AssertionError:
            caught = True
    assert caught, f"{mutant.__name__} was not caught"


def test_range_mutant_is_caught(monkeypatch):
    """A range that leaks one key past its end double-counts keys in the merge."""
    orig = S.head_forward_range

    def leaky(q, k, v, scale, causal, kv_len_b, kbeg, kend):
        return orig(q, k, v, scale, causal, kv_len_b, kbeg, min(kend + 1, k.shape[0]))
    monkeypatch.setattr(S, "head_forward_range", leaky)
    with pytest.raises(AssertionError):
        test_merge_of_splits_is_unsplit_attention(False, False, 7)
