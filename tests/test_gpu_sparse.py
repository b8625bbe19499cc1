"""Block-sparse parity on the GPU: fa_fwd_sparse / fa_bwd_sparse (HIP, through the C ABI)
against the fp64 oracle's block-masked attention on the same seeded inputs."""
import numpy as np
import pytest
import torch

import io_aware_softmax_tiled_amd as fa
import oracle
import workloads
from tests import gpu_util as U

pytestmark = pytest.mark.gpu
BLK = 128


@pytest.fixture(autouse=True)
def _gpu():
    U.require_gpu()


def _mask(N, density, seed, empty_row=None):
    nb = -(-N // BLK)
    rng = np.random.default_rng(seed)
    m = (rng.random((nb, nb)) < density).astype(np.uint8)
    if empty_row is not None and empty_row < nb:
        m[empty_row] = 0
    return m


def _run(inp, m, dev=None, backward=True):
    dev = dev or U.to_dev(inp)
    bm = torch.from_numpy(m).cuda()
    o, lse = fa.fa_fwd_sparse(dev["q"], dev["k"], dev["v"], bm, causal=inp["causal"],
                              scale=inp["scale"], kv_len=dev["kv_len"])
    grads = None
    if backward:
        grads = fa.fa_bwd_sparse(dev["q"], dev["k"], dev["v"], o, dev["dout"], lse, bm,
                                 causal=inp["causal"], scale=inp["scale"], kv_len=dev["kv_len"])
    torch.cuda.synchronize()
    return o, lse, grads


def _check_fwd(o, lse, ref_o, ref_l, dtype, sel=lambda t: t):
    lg = sel(lse).double().cpu().numpy()
    empty = np.isneginf(ref_l)
    assert np.array_equal(np.isneginf(lg), empty), "-inf pattern of lse differs"
    og = sel(o).double().cpu().numpy()
    assert np.all(og[empty] == 0.0), "rows that see no key must have O = 0"
    U.compare("O", torch.from_numpy(og), ref_o, dtype)
    U.compare("LSE", torch.from_numpy(lg[~empty]), ref_l[~empty], dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [64, 130, 300, 513])
@pytest.mark.parametrize("causal,pad", [(False, False), (True, False), (False, True),
                                       (True, True)])
def test_sparse_small(dtype, d, N, causal, pad):
    kv = (1, N) if pad else None
    w, inp = workloads.custom(2, 2, N, d, dtype, causal, kv_range=kv, seed=500 + N + d)
    m = _mask(N, 0.6, N + d, empty_row=1)
    U.say(f"[sparse] N={N} d={d} {dtype} causal={causal} pad={pad} mask={m.tolist()}")
    o, lse, (dq, dk, dv) = _run(inp, m)
    q, k, v, do = (U.f64(inp, n) for n in ("q", "k", "v", "dout"))
    kvn = U.kv_np(inp)
    ref_o, ref_l = oracle.attention_forward_sparse(q, k, v, inp["scale"], causal, kvn, m, BLK)
    _check_fwd(o, lse, ref_o, ref_l, dtype)
    rq, rk, rv = oracle.attention_backward_sparse(q, k, v, do, inp["scale"], causal, kvn, m, BLK)
    U.compare("dQ", dq, rq, dtype)
    U.compare("dK", dk, rk, dtype)
    U.compare("dV", dv, rv, dtype)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_sparse_wide_grid(d, causal):
    """B*H*ceil(N/128) = 768 dK/dV workgroups (head_dim 64: the one-wave dK/dV kernel)."""
    N = 300
    w, inp = workloads.custom(8, 32, N, d, "bf16", causal, kv_range=(1, N), seed=550 + d)
    m = _mask(N, 0.6, 551 + d, empty_row=1)
    U.say(f"[sparse] wide grid N={N} d={d} causal={causal} mask={m.tolist()}")
    o, lse, (dq, dk, dv) = _run(inp, m)
    q, k, v, do = (U.f64(inp, n) for n in ("q", "k", "v", "dout"))
    kvn = U.kv_np(inp)
    ref_o, ref_l = oracle.attention_forward_sparse(q, k, v, inp["scale"], causal, kvn, m, BLK)
    _check_fwd(o, lse, ref_o, ref_l, "bf16")
    rq, rk, rv = oracle.attention_backward_sparse(q, k, v, do, inp["scale"], causal, kvn, m, BLK)
    U.compare("dQ", dq, rq, "bf16")
    U.compare("dK", dk, rk, "bf16")
    U.compare("dV", dv, rv, "bf16")


@pytest.mark.parametrize("d", [64, 128])
def test_all_ones_mask_matches_dense(d):
    w, inp = workloads.custom(2, 3, 300, d, "bf16", True, kv_range=(100, 300), seed=77)
    dev = U.to_dev(inp)
    m = np.ones((3, 3), np.uint8)
    o, lse, (dq, dk, dv) = _run(inp, m, dev)
    o_d, lse_d, dq_d, dk_d, dv_d = U.gpu_bwd(inp, dev)
    for a, b in ((o, o_d), (lse, lse_d), (dq, dq_d), (dk, dk_d), (dv, dv_d)):
        assert (a - b).abs().max().item() <= 1e-5


def test_all_zero_mask():
    w, inp = workloads.custom(1, 2, 200, 64, "bf16", False, seed=78)
    o, lse, (dq, dk, dv) = _run(inp, np.zeros((2, 2), np.uint8))
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))
    assert torch.all(dq == 0) and torch.all(dk == 0) and torch.all(dv == 0)


def test_sparse_full_size():
    """B=2, H=16, N=4096, d=128, causal, Q x4 with half of the lower block triangle on
    (and the diagonal blocks always on): two sampled heads against the oracle."""
    w = workloads.WORKLOADS[4]
    inp = workloads.draw(w)
    nb = w.N // BLK
    rng = np.random.default_rng(9)
    m = np.tril((rng.random((nb, nb)) < 0.5).astype(np.uint8))
    np.fill_diagonal(m, 1)
    U.say(f"[sparse] full size {w.name}, {int(m.sum())} of {nb * (nb + 1) // 2} blocks on")
    o, lse, (dq, dk, dv) = _run(inp, m)
    for t in (o, lse, dq, dk, dv):
        assert torch.isfinite(t).all()
    q, k, v, do = (U.f64(inp, n) for n in ("q", "k", "v", "dout"))
    for b, h in U.sample_heads(w.B, w.H, 2):
        ro, rl = oracle.head_forward_sparse(q[b, h], k[b, h], v[b, h], w.scale, True, None, m)
        U.compare(f"O ({b},{h})", o[b, h], ro, "bf16")
        U.compare(f"LSE ({b},{h})", lse[b, h], rl, "bf16")
        rq, rk, rv = oracle.head_backward_sparse(q[b, h], k[b, h], v[b, h], do[b, h], w.scale,
                                                 True, None, m)
        U.compare(f"dQ ({b},{h})", dq[b, h], rq, "bf16")
        U.compare(f"dK ({b},{h})", dk[b, h], rk, "bf16")
        U.compare(f"dV ({b},{h})", dv[b, h], rv, "bf16")
