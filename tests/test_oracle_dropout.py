"""The dropout oracle against facts other than itself: the ROCm random-number library's
own Philox4x32-10 engine (the generator, and the element -> byte mapping written out
through it), statistics of the mask, p = 0, an identity V that exposes P * Z, finite
differences of the backward pass, unbiasedness over seeds, and planted mistakes that
those pins catch."""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle
from oracle import dropout as DR

_HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def rocrand_block(tmp_path_factory):
    """Philox4x32-10 block through rocRAND's host-callable engine, built here with g++."""
    out = str(tmp_path_factory.mktemp("philox") / "libphilox_ref.so")
    subprocess.run(["g++", "-O1", "-fPIC", "-shared", "-D__HIP_PLATFORM_AMD__",
                    "-I/opt/rocm/include", os.path.join(_HERE, "philox4x32_rocrand.cpp"),
                    "-o", out], check=True, capture_output=True)
    lib = ctypes.CDLL(out)
    lib.philox4x32_rocrand.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int]

    def block(ctr, key):
        c = np.asarray(ctr, dtype=np.uint32).reshape(-1, 4).copy()
        k = np.asarray(key, dtype=np.uint32).reshape(-1, 2).copy()
        o = np.zeros_like(c)
        lib.philox4x32_rocrand(c.ctypes.data, k.ctypes.data, o.ctypes.data, len(c))
        return o
    return block


def test_philox_matches_rocrand(rocrand_block):
    rng = np.random.default_rng(1)
    n = 400
    ctr = rng.integers(0, 2**32, size=(n, 4), dtype=np.uint64)
    ctr[:, 1] >>= 2                       # the engine's offset is 4 (c0 + 2^32 c1) < 2^64
    key = rng.integers(0, 2**32, size=(n, 2), dtype=np.uint64)
    edge = np.array([[0, 0, 0, 0], [2**32 - 1, 2**30 - 1, 2**32 - 1, 2**32 - 1],
                     [1, 0, 0, 0], [0, 0, 1, 0]], dtype=np.uint64)
    ctr = np.concatenate([ctr, edge])
    key = np.concatenate([key, np.array([[0, 0], [2**32 - 1, 2**32 - 1], [0, 1], [1, 0]],
                                        dtype=np.uint64)])
    mine = np.stack(DR.philox4x32(ctr[:, 0], ctr[:, 1], ctr[:, 2], ctr[:, 3], key[:, 0],
                                  key[:, 1]), axis=-1)
    assert np.array_equal(mine, rocrand_block(ctr, key))


def _byte(rocrand_block, i, j, bh, seed, offset):
    """The byte of element (i, j), spelled out one element at a time."""
    g, u = j // 32, j % 32
    blk = 2 * g + (u // 8) % 2
    pos = 8 * (u // 16) + u % 8
    words = rocrand_block([i, blk, bh, offset], [seed % 2**32, seed // 2**32])[0]
    return int(words[pos // 4]) >> (8 * (pos % 4)) & 0xFF


def test_byte_mapping_through_rocrand(rocrand_block):
    seed, offset, bh = 0xDEADBEEF12345678, 99, 5
    b = DR.random_bytes(40, 200, bh, seed, offset)
    rng = np.random.default_rng(2)
    for _ in range(80):
        i, j = int(rng.integers(0, 40)), int(rng.integers(0, 200))
        assert b[i, j] == _byte(rocrand_block, i, j, bh, seed, offset)


def test_key_range():
    for seed, offset in ((-1, 0), (1 << 64, 0), (0, 1 << 32), (0, -1)):
        with pytest.raises(ValueError):
            DR.random_bytes(2, 2, 0, seed, offset)


@pytest.mark.parametrize("p", [0.1, 0.25, 0.5])
def test_mask_statistics(p):
    t = DR.dropout_threshold(p)
    z = np.concatenate([DR.keep_mask(300, bh, p, 7, 0).ravel() for bh in range(4)])
    keep = (256 - t) / 256
    sigma = np.sqrt(keep * (1 - keep) / z.size)
    assert abs(z.mean() - keep) < 5 * sigma
    b = DR.random_bytes(256, 256, 0, 11, 3).ravel()
    counts = np.bincount(b, minlength=256)
    chi2 = float(((counts - b.size / 256) ** 2 / (b.size / 256)).sum())
    assert chi2 < 400  # 255 degrees of freedom; far above any plausible fluctuation


def _inputs(N, d, seed):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((1, 2, N, d)) for _ in range(4)]


def test_p_zero_is_plain_attention():
    q, k, v, do = _inputs(20, 4, 3)
    o, l = oracle.attention_forward_dropout(q, k, v, 0.5, True, None, p=0.0, seed=1)
    ro, rl = oracle.attention_forward(q, k, v, 0.5, True)
    assert np.allclose(o, ro, atol=1e-14, rtol=0) and np.allclose(l, rl, atol=1e-14, rtol=0)
    g = oracle.attention_backward_dropout(q, k, v, do, 0.5, True, None, p=0.0, seed=1)
    rg = oracle.attention_backward(q, k, v, do, 0.5, True)
    for a, b in zip(g, rg):
        assert np.allclose(a, b, atol=1e-13, rtol=0)


@pytest.mark.parametrize("causal", [False, True])
def test_identity_v_exposes_masked_probabilities(causal):
    """With V = I (N = d) the output is P * Z / keep, P from the plain definition."""
    N, p, seed, offset = 48, 0.3, 1234, 9
    rng = np.random.default_rng(4)
    q, k = rng.standard_normal((2, 1, 2, N, N))
    v = np.broadcast_to(np.eye(N), (1, 2, N, N)).copy()
    o, lse = oracle.attention_forward_dropout(q, k, v, 0.3, causal, None, p, seed, offset)
    po, plse = oracle.attention_forward(q, k, v, 0.3, causal)   # = P (V = I)
    t = DR.dropout_threshold(p)
    for h in range(2):
        z = DR.random_bytes(N, N, h, seed, offset) >= t
        assert np.allclose(o[0, h], po[0, h] * z * 256 / (256 - t), atol=1e-14, rtol=0)
    assert np.allclose(lse, plse, atol=1e-14, rtol=0)


def test_finite_differences():
    N, d = 9, 3
    q, k, v, do = _inputs(N, d, 5)
    kw = dict(causal=True, kv_len=None, p=0.4, seed=77, offset=1)
    grads = oracle.attention_backward_dropout(q, k, v, do, 0.8, **kw)
    h = 1e-6
    for which in range(3):
        xs = [q, k, v]
        fd = np.zeros_like(xs[which])
        for idx in np.ndindex(*xs[which].shape):
            xp = [x.copy() for x in xs]
            xm = [x.copy() for x in xs]
            xp[which][idx] += h
            xm[which][idx] -= h
            lp = (oracle.attention_forward_dropout(*xp, 0.8, **kw)[0] * do).sum()
            lm = (oracle.attention_forward_dropout(*xm, 0.8, **kw)[0] * do).sum()
            fd[idx] = (lp - lm) / (2 * h)
        assert np.abs(grads[which] - fd).max() < 1e-7, "QKV"[which]


def test_unbiased_over_seeds():
    """The mean over many generator keys of the dropped output approaches the plain one."""
    q, k, v, _ = _inputs(16, 4, 6)
    ro, _ = oracle.attention_forward(q, k, v, 0.5, False)
    acc = np.zeros_like(ro)
    n = 600
    for s in range(n):
        acc += oracle.attention_forward_dropout(q, k, v, 0.5, False, None, 0.25, s, 0)[0]
    assert np.abs(acc / n - ro).max() < 0.1


# ---- planted mistakes ------------------------------------------------------------------

def _bwd_variant(q, k, v, dout, scale, causal, kv_len_b, z, ks, dp_scale=True, dv_mask=True,
                 d_mask=True):
    a = oracle.allowed_mask(q.shape[0], k.shape[0], causal, kv_len_b)
    s = np.where(a, scale * (q @ k.T), -np.inf)
    e = np.exp(s - s.max(axis=1)[:, None])
    p = e / e.sum(axis=1)[:, None]
    pd = p * z * ks if dv_mask else p
    dv = pd.T @ dout
    dp = (dout @ v.T) * (z * ks if dp_scale else z)
    dsum = (p * dp).sum(axis=1) if d_mask else (p * (dout @ v.T)).sum(axis=1)
    ds = p * (dp - dsum[:, None])
    return scale * (ds @ k), scale * (ds.T @ q), dv


@pytest.mark.parametrize("kind", ["dp_scale", "dv_mask", "d_mask"])
def test_backward_mutants_are_caught(monkeypatch, kind):
    def mutant(q, k, v, dout, scale, causal, kv_len_b, z, ks):
        return _bwd_variant(q, k, v, dout, scale, causal, kv_len_b, z, ks, **{kind: False})
    monkeypatch.setattr(DR, "head_backward_dropout", mutant)
    with pytest.raises(AssertionError):
        test_finite_differences()


def test_transposed_mask_is_caught(monkeypatch, rocrand_block):
    orig = DR.random_bytes
    monkeypatch.setattr(DR, "random_bytes", lambda n_q, n_k, bh, s, o: orig(n_k, n_q, bh, s, o).T)
    # the identity-V pin builds its own mask through the same function, so check against
    # bytes computed through rocRAND directly
    b = DR.random_bytes(40, 40, 1, 5, 6)
    assert any(b[i, j] != _byte(rocrand_block, i, j, 1, 5, 6) for i, j in ((3, 17), (3, 9),
                                                                          (30, 2)))


# ---- the quantisation of p --------------------------------------------------------------

_GOLDEN = os.path.join(_HERE, "golden", "dropout_threshold_cases.json")


def _golden_cases():
    import json
    return json.load(open(_GOLDEN))["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: repr(c["p"]))
def test_threshold_golden(case):
    """Hand-derived thresholds and keep scales (tests/golden/dropout_threshold_cases.json)."""
    from fractions import Fraction
    assert DR.dropout_threshold(case["p"]) == case["t"]
    num, den = case["keep_scale"]
    assert DR.keep_scale(case["p"]) == float(Fraction(num, den))


def _nearest_threshold(p):
    """Brute force over every byte threshold: the t whose keep probability (256 - t)/256
    is nearest to 1 - p (the larger t on a tie), p taken as float32."""
    from fractions import Fraction
    p = Fraction(float(np.float32(p)))
    best = None
    for t in range(256):
        err = abs(Fraction(256 - t, 256) - (1 - p))
        if best is None or err < best[0] or err == best[0]:
            best = (err, t)
    return best[1]


def test_threshold_is_the_nearest_keep_probability():
    """Over a grid of p and every float32 around each halfway point k + 1/2 of 256 p, the
    oracle's t is the threshold whose keep probability is nearest 1 - p, within half a
    grid step; the keep scale is the inverse of the keep probability (their product is 1
    up to the float64 rounding of the scale)."""
    from fractions import Fraction
    ps = list(np.linspace(0.0, 0.999, 1999))
    for k in range(0, 256):
        mid = np.float32((k + 0.5) / 256)
        ps += [float(mid), float(np.nextafter(mid, np.float32(0))),
               float(np.nextafter(mid, np.float32(1)))]
    ps = [p for p in ps if 0.0 <= float(np.float32(p)) < 1.0]
    for p in ps:
        t = DR.dropout_threshold(p)
        assert t == _nearest_threshold(p), p
        keep = Fraction(256 - t, 256)
        if t < 255:   # the cap at 255 is the only place the error may exceed half a step
            assert abs(keep - (1 - Fraction(float(np.float32(p))))) <= Fraction(1, 512), p
        # the keep scale is the inverse keep probability, correctly rounded to float64
        assert DR.keep_scale(p) == float(1 / keep), p
        assert abs(Fraction(DR.keep_scale(p)) * keep - 1) <= Fraction(1, 2**52), p


_THRESHOLD_MUTANTS = {
    "round_255p": (lambda p: min(255, int(np.floor(255.0 * float(np.float32(p)) + 0.5))),
                   DR.keep_scale),
    "floor_256p": (lambda p: min(255, int(np.floor(256.0 * float(np.float32(p))))),
                   DR.keep_scale),
    "inverse_1_minus_p": (DR.dropout_threshold, lambda p: 1.0 / (1.0 - p)),
}


@pytest.mark.parametrize("name", sorted(_THRESHOLD_MUTANTS))
def test_threshold_mutants_are_caught(monkeypatch, name):
    """A plausible other reading of the quantisation fails one of the pins above."""
    thr, ks = _THRESHOLD_MUTANTS[name]
    monkeypatch.setattr(DR, "dropout_threshold", thr)
    monkeypatch.setattr(DR, "keep_scale", ks)
    failed = False
    for case in _golden_cases():
        try:
            test_threshold_golden(case)
        except AssertionError:
            failed = True
    try:
        test_threshold_is_the_nearest_keep_probability()
    except AssertionError:
        failed = True
    assert failed, name
