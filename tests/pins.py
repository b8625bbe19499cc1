"""Checks that pin the oracle to facts other than itself.

Each check takes the forward and backward functions under test (signature of
oracle.attention_forward / attention_backward on [B,H,N,d] float64 arrays) and raises
AssertionError when a fact fails. The real oracle must pass every check; the mutation
tests plant plausible mistakes in the oracle and require that some check fails.

Facts used (none of them is the oracle's own formula retyped):
- closed forms: Q = 0 gives uniform rows; causal row 0 sees only key 0; N = 1;
  constant V; V = identity turns O into P itself;
- invariants: rows of P sum to 1; shifting every key by c changes nothing but LSE
  (the safe-softmax shift identity); gradient sums; masked keys are inert;
- independent library routines: torch's scaled_dot_product_attention in float64 and
  torch.autograd through it, scipy's logsumexp;
- brute force: scalar loops on tiny inputs;
- finite differences of L = sum(dO * O);
- hand-derived exact cases stored in tests/golden/.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import scipy.special
import torch
import torch.nn.functional as F

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

MASK_MODES = [(False, None), (True, None), (False, "pad"), (True, "pad")]


def _rng(seed):
    return np.random.default_rng(seed)


def _inputs(rng, B, H, N, d, scale_q=1.0):
    q = rng.standard_normal((B, H, N, d)) * scale_q
    k = rng.standard_normal((B, H, N, d))
    v = rng.standard_normal((B, H, N, d))
    do = rng.standard_normal((B, H, N, d))
    return q, k, v, do


def _kv(rng, B, N, mode):
    if mode != "pad":
        return None
    return rng.integers(1, N + 1, size=B).astype(np.int32)


def _visible(N, causal, kvb):
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    a = np.ones((N, N), bool)
    if causal:
        a &= j <= i
    if kvb is not None:
        a &= j < kvb
    return a


def _close(a, b, tol, what):
    err = float(np.max(np.abs(np.asarray(a) - np.asarray(b)), initial=0.0))
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


# ---- independent library routines ---------------------------------------------------

def check_torch_sdpa(fwd, bwd, seed=1):
    """O matches torch SDPA (float64, CPU); gradients match torch.autograd through it;
    LSE matches scipy.special.logsumexp over the masked scores."""
    rng = _rng(seed)
    for B, H, N, d in [(2, 2, 7, 5), (1, 3, 16, 8), (2, 1, 33, 4)]:
        for causal, mode in MASK_MODES:
            q, k, v, do = _inputs(rng, B, H, N, d)
            kv = _kv(rng, B, N, mode)
            scale = 0.37
            o, lse = fwd(q, k, v, scale, causal, kv)
            dq, dk, dv = bwd(q, k, v, do, scale, causal, kv)
            mask = np.stack([_visible(N, causal, None if kv is None else kv[b])
                             for b in range(B)])[:, None]  # [B,1,N,N]
            tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
            to = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.tensor(mask),
                                                scale=scale)
            (to * torch.tensor(do)).sum().backward()
            _close(o, to.detach().numpy(), 1e-12, "O vs torch sdpa")
            _close(dq, tq.grad.numpy(), 1e-10, "dQ vs autograd")
            _close(dk, tk.grad.numpy(), 1e-10, "dK vs autograd")
            _close(dv, tv.grad.numpy(), 1e-10, "dV vs autograd")
            s = scale * torch.matmul(torch.tensor(q), torch.tensor(k).transpose(-1, -2)).numpy()
            s = np.where(mask, s, -np.inf)
            _close(lse, scipy.special.logsumexp(s, axis=-1), 1e-12, "LSE vs scipy logsumexp")


# ---- closed forms ---------------------------------------------------------------------

def check_identity_v_gives_p(fwd, bwd, seed=2):
    """With d = N and V = I, O is P itself: rows sum to 1, entries >= 0, masked entries
    are exactly 0, and P = exp(S - LSE) on the visible entries."""
    rng = _rng(seed)
    for causal, mode in MASK_MODES:
        B, H, N = 2, 2, 9
        q = rng.standard_normal((B, H, N, N))
        k = rng.standard_normal((B, H, N, N))
        v = np.broadcast_to(np.eye(N), (B, H, N, N)).copy()
        kv = _kv(rng, B, N, mode)
        scale = 0.5
        o, lse = fwd(q, k, v, scale, causal, kv)
        _close(o.sum(-1), 1.0, 1e-14, "rows of P sum to 1")
        assert (o >= 0).all(), "P has a negative entry"
        for b in range(B):
            vis = _visible(N, causal, None if kv is None else kv[b])
            assert np.all(o[b][:, ~vis] == 0.0), "a masked entry of P is not 0"
            s = scale * np.einsum("hid,hjd->hij", q[b], k[b])
            p = np.exp(s - lse[b][..., None])
            _close(np.where(vis, p, 0.0), o[b], 1e-13, "P = exp(S - LSE)")


def check_zero_q(fwd, bwd, seed=3):
    """Q = 0: uniform weights over the visible keys. O_i is their mean, LSE_i = ln(count),
    dK = 0, dV_j = sum over rows i that see j of dO_i / count_i."""
    rng = _rng(seed)
    for causal, mode in MASK_MODES:
        B, H, N, d = 2, 2, 11, 3
        _, k, v, do = _inputs(rng, B, H, N, d)
        q = np.zeros_like(k)
        kv = _kv(rng, B, N, mode)
        o, lse = fwd(q, k, v, 0.9, causal, kv)
        dq, dk, dv = bwd(q, k, v, do, 0.9, causal, kv)
        for b in range(B):
            vis = _visible(N, causal, None if kv is None else kv[b]).astype(float)
            cnt = vis.sum(1)
            for h in range(H):
                _close(o[b, h], (vis @ v[b, h]) / cnt[:, None], 1e-13, "Q=0: O is the mean")
                _close(lse[b, h], np.log(cnt), 1e-14, "Q=0: LSE = ln(count)")
                _close(dk[b, h], 0.0, 1e-14, "Q=0: dK = 0")
                _close(dv[b, h], vis.T @ (do[b, h] / cnt[:, None]), 1e-13, "Q=0: dV")


def check_causal_row0_and_n1(fwd, bwd, seed=4):
    """Causal row 0 sees only key 0: O_0 = V_0, LSE_0 = scale q_0.k_0, dQ_0 = 0.
    N = 1 (any mask): O = V, LSE = scale q.k, dV = dO, dQ = dK = 0."""
    rng = _rng(seed)
    q, k, v, do = _inputs(rng, 2, 3, 6, 4)
    o, lse = fwd(q, k, v, 0.7, True, None)
    dq, dk, dv = bwd(q, k, v, do, 0.7, True, None)
    _close(o[:, :, 0], v[:, :, 0], 1e-15, "causal O_0 = V_0")
    _close(lse[:, :, 0], 0.7 * (q[:, :, 0] * k[:, :, 0]).sum(-1), 1e-14, "causal LSE_0")
    _close(dq[:, :, 0], 0.0, 1e-14, "causal dQ_0 = 0")
    for causal, mode in MASK_MODES:
        q, k, v, do = _inputs(rng, 2, 2, 1, 5)
        kv = None if mode is None else np.ones(2, np.int32)
        o, lse = fwd(q, k, v, 0.3, causal, kv)
        dq, dk, dv = bwd(q, k, v, do, 0.3, causal, kv)
        _close(o, v, 1e-15, "N=1: O = V")
        _close(lse, 0.3 * (q * k).sum(-1), 1e-15, "N=1: LSE")
        _close(dv, do, 1e-15, "N=1: dV = dO")
        _close(dq, 0.0, 1e-15, "N=1: dQ = 0")
        _close(dk, 0.0, 1e-15, "N=1: dK = 0")


def check_constant_v(fwd, bwd, seed=5):
    """Every V row equal to c: O = c and dQ = dK = 0 (dP is constant along each row)."""
    rng = _rng(seed)
    for causal, mode in MASK_MODES:
        q, k, _, do = _inputs(rng, 2, 2, 10, 4)
        c = rng.standard_normal(4)
        v = np.broadcast_to(c, q.shape).copy()
        kv = _kv(rng, 2, 10, mode)
        o, _ = fwd(q, k, v, 0.6, causal, kv)
        dq, dk, _ = bwd(q, k, v, do, 0.6, causal, kv)
        _close(o, np.broadcast_to(c, o.shape), 1e-14, "constant V: O = c")
        _close(dq, 0.0, 1e-13, "constant V: dQ = 0")
        _close(dk, 0.0, 1e-13, "constant V: dK = 0")


# ---- invariants -----------------------------------------------------------------------

def check_key_shift(fwd, bwd, seed=6):
    """k_j -> k_j + c for every key: O, dQ, dK, dV unchanged; LSE_i shifts by scale q_i.c
    (the safe-softmax shift identity; dQ is unchanged because rows of dS sum to 0)."""
    rng = _rng(seed)
    for causal, mode in MASK_MODES:
        q, k, v, do = _inputs(rng, 2, 2, 12, 5)
        kv = _kv(rng, 2, 12, mode)
        c = rng.standard_normal(5) * 3
        o1, l1 = fwd(q, k, v, 0.45, causal, kv)
        g1 = bwd(q, k, v, do, 0.45, causal, kv)
        o2, l2 = fwd(q, k + c, v, 0.45, causal, kv)
        g2 = bwd(q, k + c, v, do, 0.45, causal, kv)
        _close(o1, o2, 1e-12, "shift: O")
        _close(l2 - l1, 0.45 * (q @ c), 1e-12, "shift: LSE")
        for a, b_, nm in zip(g1, g2, ("dQ", "dK", "dV")):
            _close(a, b_, 1e-11, f"shift: {nm}")


def check_gradient_sums(fwd, bwd, seed=7):
    """sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i per head (rows of P sum to 1)."""
    rng = _rng(seed)
    for causal, mode in MASK_MODES:
        q, k, v, do = _inputs(rng, 2, 3, 13, 6)
        kv = _kv(rng, 2, 13, mode)
        dq, dk, dv = bwd(q, k, v, do, 0.4, causal, kv)
        _close(dk.sum(2), 0.0, 1e-12, "sum_j dK_j = 0")
        _close(dv.sum(2), do.sum(2), 1e-12, "sum_j dV_j = sum_i dO_i")


def check_masked_keys_inert(fwd, bwd, seed=8):
    """Padded keys: dK_j = dV_j = 0 for j >= kv_len, and perturbing padded K/V rows
    changes nothing. Causal: perturbing K_j, V_j for j > i leaves O_i and dQ_i alone."""
    rng = _rng(seed)
    B, H, N, d = 3, 2, 12, 4
    q, k, v, do = _inputs(rng, B, H, N, d)
    kv = np.array([5, 12, 1], np.int32)
    for causal in (False, True):
        o, lse = fwd(q, k, v, 0.5, causal, kv)
        dq, dk, dv = bwd(q, k, v, do, 0.5, causal, kv)
        k2, v2 = k.copy(), v.copy()
        for b in range(B):
            assert np.all(dk[b, :, kv[b]:] == 0.0) and np.all(dv[b, :, kv[b]:] == 0.0), \
                "padded key has a nonzero gradient"
            k2[b, :, kv[b]:] += 100.0
            v2[b, :, kv[b]:] -= 50.0
        o2, lse2 = fwd(q, k2, v2, 0.5, causal, kv)
        dq2, _, _ = bwd(q, k2, v2, do, 0.5, causal, kv)
        _close(o, o2, 1e-13, "padded K/V perturbed: O")
        _close(lse, lse2, 1e-13, "padded K/V perturbed: LSE")
        _close(dq, dq2, 1e-12, "padded K/V perturbed: dQ")
    o, _ = fwd(q, k, v, 0.5, True, None)
    dq, _, _ = bwd(q, k, v, do, 0.5, True, None)
    for i in (0, 4, 10):
        k2, v2 = k.copy(), v.copy()
        k2[:, :, i + 1:] = rng.standard_normal(k2[:, :, i + 1:].shape) * 10
        v2[:, :, i + 1:] = rng.standard_normal(v2[:, :, i + 1:].shape) * 10
        o2, _ = fwd(q, k2, v2, 0.5, True, None)
        dq2, _, _ = bwd(q, k2, v2, do, 0.5, True, None)
        _close(o[:, :, :i + 1], o2[:, :, :i + 1], 1e-13, "causal: future keys inert (O)")
        _close(dq[:, :, :i + 1], dq2[:, :, :i + 1], 1e-12, "causal: future keys inert (dQ)")


def check_large_scores(fwd, bwd, seed=9):
    """Scores of order +-1e3 (e^x overflows float64 without the max shift): O stays a
    convex combination of V rows and matches torch SDPA; LSE is finite and >= max score."""
    rng = _rng(seed)
    q, k, v, do = _inputs(rng, 1, 2, 16, 4)
    q = q * 300.0
    o, lse = fwd(q, k, v, 1.0, False, None)
    assert np.isfinite(o).all() and np.isfinite(lse).all(), "overflow with large scores"
    s = np.einsum("bhid,bhjd->bhij", q, k)
    assert (lse >= s.max(-1) - 1e-9).all(), "LSE below the row maximum"
    to = F.scaled_dot_product_attention(torch.tensor(q), torch.tensor(k), torch.tensor(v),
                                        scale=1.0)
    _close(o, to.numpy(), 1e-9, "large scores: O vs torch sdpa")
    dq, dk, dv = bwd(q, k, v, do, 1.0, False, None)
    assert np.isfinite(dq).all() and np.isfinite(dk).all() and np.isfinite(dv).all()


# ---- brute force and finite differences ------------------------------------------------

def brute_forward(q, k, v, scale, causal, kv):
    """Scalar loops straight from the definition (tiny inputs only)."""
    B, H, N, d = q.shape
    o = np.zeros((B, H, N, v.shape[3]))
    lse = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            for i in range(N):
                w = []
                for j in range(N):
                    if (causal and j > i) or (kv is not None and j >= kv[b]):
                        continue
                    w.append((j, scale * sum(q[b, h, i, t] * k[b, h, j, t] for t in range(d))))
                mx = max(s for _, s in w)
                z = sum(math.exp(s - mx) for _, s in w)
                lse[b, h, i] = mx + math.log(z)
                for j, s in w:
                    o[b, h, i] += math.exp(s - mx) / z * v[b, h, j]
    return o, lse


def check_brute_force(fwd, bwd, seed=10):
    rng = _rng(seed)
    for causal, mode in MASK_MODES:
        q, k, v, _ = _inputs(rng, 2, 2, 9, 3)
        kv = _kv(rng, 2, 9, mode)
        o, lse = fwd(q, k, v, 0.8, causal, kv)
        ob, lb = brute_forward(q, k, v, 0.8, causal, kv)
        _close(o, ob, 1e-13, "O vs brute force")
        _close(lse, lb, 1e-13, "LSE vs brute force")


def check_finite_differences(fwd, bwd, seed=11, h=1e-6):
    """Central differences of L = sum(dO * O) against dQ, dK, dV."""
    rng = _rng(seed)
    for N, d in [(1, 1), (2, 3), (5, 4), (8, 1), (8, 4)]:
        for causal, mode in MASK_MODES:
            q, k, v, do = _inputs(rng, 1, 1, N, d)
            kv = _kv(rng, 1, N, mode)
            grads = bwd(q, k, v, do, 0.6, causal, kv)
            for which, g in enumerate(grads):
                base = [q, k, v]
                fd = np.zeros_like(g)
                for idx in np.ndindex(g.shape):
                    xs_p = [a.copy() for a in base]
                    xs_m = [a.copy() for a in base]
                    xs_p[which][idx] += h
                    xs_m[which][idx] -= h
                    lp = float((fwd(*xs_p, 0.6, causal, kv)[0] * do).sum())
                    lm = float((fwd(*xs_m, 0.6, causal, kv)[0] * do).sum())
                    fd[idx] = (lp - lm) / (2 * h)
                tol = 1e-7 * max(1.0, float(np.abs(g).max()))
                _close(g, fd, tol, f"finite differences ({'QKV'[which]}, N={N}, d={d}, "
                                   f"causal={causal}, pad={mode})")


# ---- hand-derived exact cases -------------------------------------------------------------

def golden_cases():
    with open(os.path.join(GOLDEN, "closed_form_cases.json")) as f:
        return json.load(f)["cases"]


def _ev(x):
    """Evaluate a fixture entry: a number or an expression in +-*/ and ln()."""
    if isinstance(x, list):
        return [_ev(e) for e in x]
    if isinstance(x, str):
        return float(eval(x, {"__builtins__": {}}, {"ln": math.log}))  # noqa: S307
    return float(x)


def check_golden(fwd, bwd):
    for case in golden_cases():
        q, k, v = (np.array(_ev(case[n]), dtype=np.float64)[None, None] for n in "qkv")
        kv = None if case.get("kv_len") is None else np.array(case["kv_len"], np.int32)
        o, lse = fwd(q, k, v, case["scale"], case["causal"], kv)
        _close(o[0, 0], np.array(_ev(case["O"])), 1e-14, f"golden {case['name']}: O")
        _close(lse[0, 0], np.array(_ev(case["LSE"])), 1e-14, f"golden {case['name']}: LSE")
        if "dO" in case:
            do = np.array(_ev(case["dO"]))[None, None]
            dq, dk, dv = bwd(q, k, v, do, case["scale"], case["causal"], kv)
            for nm, g in (("dQ", dq), ("dK", dk), ("dV", dv)):
                _close(g[0, 0], np.array(_ev(case[nm])), 1e-14, f"golden {case['name']}: {nm}")


ALL_CHECKS = [
    check_torch_sdpa,
    check_identity_v_gives_p,
    check_zero_q,
    check_causal_row0_and_n1,
    check_constant_v,
    check_key_shift,
    check_gradient_sums,
    check_masked_keys_inert,
    check_large_scores,
    check_brute_force,
    check_finite_differences,
    check_golden,
]
