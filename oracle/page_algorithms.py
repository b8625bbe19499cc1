"""The softmax and attention recurrences the pages derive, as plain float64 scalar loops.

TEST INFRASTRUCTURE ONLY (see the package header). These cross-check the definition in
``attention``: each must reproduce it to rounding (~1e-12) on tiny inputs. Each is
written from the page's notation and order of steps, not from its listings.

Masked scores are -inf. Where a recurrence would evaluate e^{(-inf) - (-inf)} (a state
that has seen only masked entries), the weight is taken as 0: such a state holds
nothing yet, and a masked entry contributes exactly zero (the reading that the Triton
listings of the review imply by loading -inf for out-of-range keys).
"""
from __future__ import annotations

import math

import numpy as np

NEG_INF = -math.inf


def _w(a: float, b: float) -> float:
    """e^{a-b}, with weight 0 when a is -inf (a state or score that holds nothing)."""
    if a == NEG_INF:
        return 0.0
    return math.exp(a - b)


# ---- "[Review] From Online Softmax to Flash Attention": (safe) softmax -------------

def softmax_three_pass(x) -> list:
    """Algorithm 3-pass safe softmax.

    Pass 1 builds the running maximum m_i = max(m_{i-1}, x_i) from m_0 = -inf.
    Pass 2 builds the denominator d_i = d_{i-1} + e^{x_i - m_N} from d_0 = 0.
    Pass 3 emits a_i = e^{x_i - m_N} / d_N.
    """
    n = len(x)
    m = NEG_INF
    for i in range(n):
        m = max(m, x[i])
    d = 0.0
    for i in range(n):
        d = d + _w(x[i], m)
    return [_w(x[i], m) / d for i in range(n)]


def softmax_online_two_pass(x) -> list:
    """Algorithm 2-pass online softmax (section Online Softmax).

    Pass 1 carries (m_i, d'_i) with d'_i = d'_{i-1} e^{m_{i-1} - m_i} + e^{x_i - m_i}:
    the denominator no longer waits for the global maximum m_N.
    Pass 2 emits a_i = e^{x_i - m_N} / d'_N.
    """
    n = len(x)
    m_prev, d_prev = NEG_INF, 0.0
    for i in range(n):
        m_i = max(m_prev, x[i])
        d_prev = d_prev * _w(m_prev, m_i) + _w(x[i], m_i)
        m_prev = m_i
    return [_w(x[i], m_prev) / d_prev for i in range(n)]


# ---- same review, section FlashAttention: one query row k of the attention --------

def _scores(q_row, K, scale, allowed_row):
    """x_i = scale * Q[k,:] K^T[:, i], or -inf where key i is not visible."""
    out = []
    for i in range(len(K)):
        if allowed_row is not None and not allowed_row[i]:
            out.append(NEG_INF)
        else:
            out.append(scale * float(sum(float(a) * float(b) for a, b in zip(q_row, K[i]))))
    return out


def attention_row_two_pass(q_row, K, V, scale=1.0, allowed_row=None):
    """Two passes over the keys of one query row (section FlashAttention, first form).

    Pass 1: the online (m, d') recurrence over x_i = Q[k,:] K^T[:, i].
    Pass 2: a_i = e^{x_i - m_N} / d'_N (the garbled numerator on the page is read as
    e^{x_i - m_N}, as in the 3-pass algorithm) and o_i = o_{i-1} + a_i V[i, :].
    Returns (O[k,:], LSE) with LSE = m_N + ln d'_N.
    """
    x = _scores(q_row, K, scale, allowed_row)
    n, dv = len(K), len(V[0])
    m, d = NEG_INF, 0.0
    for i in range(n):
        m_i = max(m, x[i])
        d = d * _w(m, m_i) + _w(x[i], m_i)
        m = m_i
    o = [0.0] * dv
    for i in range(n):
        a = _w(x[i], m) / d
        for c in range(dv):
            o[c] = o[c] + a * float(V[i][c])
    return o, m + math.log(d)


def attention_row_one_pass(q_row, K, V, scale=1.0, allowed_row=None):
    """One pass (Algorithm FlashAttention): the state (x_i, m_i, d'_i, o'_i) per key.

    o'_i = o'_{i-1} d'_{i-1} e^{m_{i-1} - m_i} / d'_i + e^{x_i - m_i} / d'_i V[i, :],
    so o'_N equals the normalised output without a second pass.
    """
    x = _scores(q_row, K, scale, allowed_row)
    n, dv = len(K), len(V[0])
    m, d = NEG_INF, 0.0
    o = [0.0] * dv
    for i in range(n):
        m_i = max(m, x[i])
        carry = d * _w(m, m_i)
        d_i = carry + _w(x[i], m_i)
        if d_i == 0.0:  # only masked keys so far: the state is still empty
            m = m_i
            continue
        p = _w(x[i], m_i) / d_i
        for c in range(dv):
            o[c] = o[c] * carry / d_i + p * float(V[i][c])
        m, d = m_i, d_i
    return o, m + math.log(d)


def attention_row_tiled(q_row, K, V, b, scale=1.0, allowed_row=None):
    """Algorithm FlashAttention (Tiling): the one-pass recurrence over key tiles of width b.

    Tile t covers keys [t*b, (t+1)*b) (the last tile is ragged: keys past the end do
    not exist, which is the same as scoring them -inf). Per tile: the local maximum,
    m_t = max(m_{t-1}, local max), d'_t = d'_{t-1} e^{m_{t-1} - m_t} + sum_j e^{x_t[j] - m_t},
    o'_t = o'_{t-1} d'_{t-1} e^{m_{t-1} - m_t} / d'_t + sum_j e^{x_t[j] - m_t} / d'_t V[t*b + j, :].
    """
    x = _scores(q_row, K, scale, allowed_row)
    n, dv = len(K), len(V[0])
    m, d = NEG_INF, 0.0
    o = [0.0] * dv
    for t0 in range(0, n, b):
        tile = range(t0, min(n, t0 + b))
        m_loc = max(x[j] for j in tile)
        m_t = max(m, m_loc)
        carry = d * _w(m, m_t)
        d_t = carry + sum(_w(x[j], m_t) for j in tile)
        if d_t == 0.0:
            m = m_t
            continue
        new_o = [o[c] * carry / d_t for c in range(dv)]
        for j in tile:
            p = _w(x[j], m_t) / d_t
            for c in range(dv):
                new_o[c] += p * float(V[j][c])
        o, m, d = new_o, m_t, d_t
    return o, m + math.log(d)


def flashatt_spec(q, k, v):
    """The review's one-dimensional spec: z_i = sum_j softmax(q_i k_1, ..., q_i k_T)_j v_j.

    q has N0 entries, k and v have T. This is attention with head_dim 1, scale 1 and no
    mask. Written from the formula, with the row maximum subtracted (safe softmax).
    """
    z = []
    for qi in q:
        x = [float(qi) * float(kj) for kj in k]
        a = softmax_three_pass(x)
        z.append(sum(aj * float(vj) for aj, vj in zip(a, v)))
    return z


# ---- "FlashAttention: Fast and Memory-Efficient Exact Attention with IO-Awareness",
# ---- Method: incremental softmax tracking and the Br x Bc block update --------------

def merge_stats(m1, l1, m2, l2):
    """Statistics of a vector split into x1 and x2 (incremental softmax tracking).

    m(x) = max(m(x1), m(x2)); l(x) = e^{m(x1) - m(x)} l(x1) + e^{m(x2) - m(x)} l(x2).
    """
    m = max(m1, m2)
    return m, _w(m1, m) * l1 + _w(m2, m) * l2


def attention_blocks(Q, K, V, Br, Bc, scale=1.0, allowed=None):
    """The block form of the Method section, for one head.

    For each query block i (Br rows) the state is O_i = 0, l_i = 0, m_i = -inf. For each
    key/value block j (Bc rows): S_ij = scale * Q_i K_j^T (masked entries -inf);
    m~ = rowmax(S_ij); P~ = exp(S_ij - m~); l~ = rowsum(P~); m_new = max(m_i, m~);
    l_new = e^{m_i - m_new} l_i + e^{m~ - m_new} l~;
    O_i <- diag(l_new)^-1 (diag(l_i) e^{m_i - m_new} O_i + e^{m~ - m_new} P~ V_j).
    A block row with every entry masked has m~ = -inf and contributes nothing.
    Returns (O [N,d], LSE [N]) with LSE = m + ln l.
    """
    Q, K, V = (np.asarray(a, dtype=np.float64) for a in (Q, K, V))
    n, nk, dv = Q.shape[0], K.shape[0], V.shape[1]
    O = np.zeros((n, dv))
    lse = np.zeros(n)
    for i0 in range(0, n, Br):
        rows = range(i0, min(n, i0 + Br))
        Oi = np.zeros((len(rows), dv))
        li = [0.0] * len(rows)
        mi = [NEG_INF] * len(rows)
        for j0 in range(0, nk, Bc):
            cols = range(j0, min(nk, j0 + Bc))
            S = scale * (Q[i0:i0 + len(rows)] @ K[j0:j0 + len(cols)].T)
            for r, row in enumerate(rows):
                for c, col in enumerate(cols):
                    if allowed is not None and not allowed[row][col]:
                        S[r, c] = NEG_INF
            for r in range(len(rows)):
                m_t = max(S[r, c] for c in range(len(cols)))
                pt = [_w(S[r, c], m_t) for c in range(len(cols))]
                l_t = sum(pt)
                m_new = max(mi[r], m_t)
                a_old, a_new = _w(mi[r], m_new), _w(m_t, m_new)
                l_new = a_old * li[r] + a_new * l_t
                if l_new == 0.0:
                    mi[r] = m_new
                    continue
                pv = np.array(pt) @ V[j0:j0 + len(cols)]
                Oi[r] = (li[r] * a_old * Oi[r] + a_new * pv) / l_new
                mi[r], li[r] = m_new, l_new
        O[i0:i0 + len(rows)] = Oi
        lse[i0:i0 + len(rows)] = [mi[r] + math.log(li[r]) for r in range(len(rows))]
    return O, lse


# ---- "Fewer matrix multiplications, same results" (flash-attention issue thread):
# ---- the deferred P V variant ------------------------------------------------------

def attention_deferred_pv(Q, K, V, block, scale=1.0, allowed=None):
    """The thread's variant, for one head: per query block, the numerator blocks f_j of
    the whole key row are kept and only one product with V is formed at the end.

    For query block i and key blocks j = 0, 1, ...: S_ij = scale * Q_i K_j^T (masked
    entries -inf); m_loc = rowmax(S_ij); f_j = exp(S_ij - m_loc); l_loc = rowsum(f_j).
    For j = 0 the state is (m, l) = (m_loc, l_loc). Otherwise m_new = max(m, m_loc),
    l_new = e^{m - m_new} l + e^{m_loc - m_new} l_loc, every earlier block f_k (k < j)
    is multiplied by e^{m - m_new}, f_j by e^{m_loc - m_new}, and (m, l) <- (m_new,
    l_new). At the end O_i = (f / l) V with f = [f_0 ... f_last]. The thread writes the
    blocks as square (query block = key block) and adds a small constant to l_loc; here
    the key blocks are `block` wide, the last one ragged, and nothing is added.
    Returns (O [N,d], LSE [N]) with LSE = m + ln l.
    """
    Q, K, V = (np.asarray(a, dtype=np.float64) for a in (Q, K, V))
    n, nk, dv = Q.shape[0], K.shape[0], V.shape[1]
    O = np.zeros((n, dv))
    lse = np.zeros(n)
    for i0 in range(0, n, block):
        rows = list(range(i0, min(n, i0 + block)))
        f_blocks = []
        m = [NEG_INF] * len(rows)
        l = [0.0] * len(rows)
        for jb, j0 in enumerate(range(0, nk, block)):
            cols = list(range(j0, min(nk, j0 + block)))
            S = scale * (Q[rows[0]:rows[-1] + 1] @ K[j0:cols[-1] + 1].T)
            for r, row in enumerate(rows):
                for c, col in enumerate(cols):
                    if allowed is not None and not allowed[row][col]:
                        S[r, c] = NEG_INF
            f = np.zeros_like(S)
            for r in range(len(rows)):
                m_loc = max(S[r, c] for c in range(len(cols)))
                f[r] = [_w(S[r, c], m_loc) for c in range(len(cols))]
                l_loc = float(sum(f[r]))
                if jb == 0:
                    m[r], l[r] = m_loc, l_loc
                    continue
                m_new = max(m[r], m_loc)
                a_old, a_loc = _w(m[r], m_new), _w(m_loc, m_new)
                for fk in f_blocks:
                    fk[r] *= a_old
                f[r] *= a_loc
                m[r], l[r] = m_new, a_old * l[r] + a_loc * l_loc
            f_blocks.append(f)
        F = np.concatenate(f_blocks, axis=1)
        O[rows[0]:rows[-1] + 1] = (F / np.array(l)[:, None]) @ V
        lse[rows[0]:rows[-1] + 1] = [m[r] + math.log(l[r]) for r in range(len(rows))]
    return O, lse
