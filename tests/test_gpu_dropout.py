"""Dropout parity on the GPU: fa_fwd_dropout / fa_bwd_dropout (HIP, through the C ABI)
against the fp64 oracle's attention with dropout, whose mask comes from the oracle's own
Philox4x32-10. Besides the tolerance tests on random inputs, three tests read the mask
the kernels used back out of O, dV and dQ with one-hot inputs and compare it bit for bit
with the oracle's mask."""
import numpy as np
import pytest
import torch

import io_aware_softmax_tiled_amd as fa
import oracle
import workloads
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    U.require_gpu()


def _run(inp, p, seed, offset, dev=None, backward=True):
    dev = dev or U.to_dev(inp)
    kw = dict(p=p, seed=seed, offset=offset, causal=inp["causal"], scale=inp["scale"],
              kv_len=dev["kv_len"])
    o, lse = fa.fa_fwd_dropout(dev["q"], dev["k"], dev["v"], **kw)
    grads = None
    if backward:
        grads = fa.fa_bwd_dropout(dev["q"], dev["k"], dev["v"], o, dev["dout"], lse, **kw)
    torch.cuda.synchronize()
    return o, lse, grads


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [64, 130, 300, 513])
@pytest.mark.parametrize("causal,pad", [(False, False), (True, False), (False, True),
                                       (True, True)])
def test_dropout_small(dtype, d, N, causal, pad):
    kv = (1, N) if pad else None
    w, inp = workloads.custom(2, 2, N, d, dtype, causal, kv_range=kv, seed=700 + N + d)
    p, seed, offset = 0.17, 1234 + N, 5
    U.say(f"[dropout] N={N} d={d} {dtype} causal={causal} pad={pad} p={p} seed={seed}")
    o, lse, (dq, dk, dv) = _run(inp, p, seed, offset)
    q, k, v, do = (U.f64(inp, n) for n in ("q", "k", "v", "dout"))
    kvn = U.kv_np(inp)
    ref_o, ref_l = oracle.attention_forward_dropout(q, k, v, inp["scale"], causal, kvn, p,
                                                    seed, offset)
    U.compare("O", o, ref_o, dtype)
    U.compare("LSE", lse, ref_l, dtype)
    rq, rk, rv = oracle.attention_backward_dropout(q, k, v, do, inp["scale"], causal, kvn, p,
                                                   seed, offset)
    U.compare("dQ", dq, rq, dtype)
    U.compare("dK", dk, rk, dtype)
    U.compare("dV", dv, rv, dtype)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_dropout_wide_grid(d, causal):
    """B*H*ceil(N/128) = 768 dK/dV workgroups (head_dim 64: the one-wave dK/dV kernel)."""
    N = 300
    w, inp = workloads.custom(8, 32, N, d, "bf16", causal, kv_range=(1, N), seed=750 + d)
    p, seed, offset = 0.17, 4321 + d, 9
    U.say(f"[dropout] wide grid N={N} d={d} causal={causal} p={p} seed={seed}")
    o, lse, (dq, dk, dv) = _run(inp, p, seed, offset)
    q, k, v, do = (U.f64(inp, n) for n in ("q", "k", "v", "dout"))
    kvn = U.kv_np(inp)
    ref_o, ref_l = oracle.attention_forward_dropout(q, k, v, inp["scale"], causal, kvn, p,
                                                    seed, offset)
    U.compare("O", o, ref_o, "bf16")
    U.compare("LSE", lse, ref_l, "bf16")
    rq, rk, rv = oracle.attention_backward_dropout(q, k, v, do, inp["scale"], causal, kvn, p,
                                                   seed, offset)
    U.compare("dQ", dq, rq, "bf16")
    U.compare("dK", dk, rk, "bf16")
    U.compare("dV", dv, rv, "bf16")


def _onehot(N, d, chunk):
    """[N, d]: row j is e_(j - chunk*d) for keys j of chunk `chunk`, 0 elsewhere."""
    m = np.zeros((N, d))
    lo, hi = chunk * d, min(N, (chunk + 1) * d)
    m[np.arange(lo, hi), np.arange(hi - lo)] = 1.0
    return m


def _masks(B, H, N, p, seed, offset):
    return np.array([[oracle.keep_mask(N, b * H + h, p, seed, offset) for h in range(H)]
                     for b in range(B)])


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("p", [0.1, 0.5, 0.9])
def test_forward_mask_bit_exact(causal, p):
    """Q = 0 makes P uniform over the visible keys, and V one-hot on one chunk of d keys
    copies P * Z * keep_scale of those keys into O: O > 0 exactly where Z = 1."""
    B, H, N, d = 2, 3, 300, 128
    seed, offset = 99, 3
    z = _masks(B, H, N, p, seed, offset)
    vis = oracle.allowed_mask(N, N, causal, None)
    q = torch.zeros(B, H, N, d, dtype=torch.bfloat16, device="cuda")
    k = torch.randn(B, H, N, d, device="cuda").to(torch.bfloat16)
    for c in range(-(-N // d)):
        v = torch.from_numpy(np.broadcast_to(_onehot(N, d, c), (B, H, N, d)).copy())
        v = v.to(torch.bfloat16).cuda()
        o, _ = fa.fa_fwd_dropout(q, k, v, p=p, seed=seed, offset=offset, causal=causal)
        torch.cuda.synchronize()
        lo, hi = c * d, min(N, (c + 1) * d)
        got = o[..., : hi - lo].cpu().numpy() > 0
        want = z[..., lo:hi] & vis[None, None, :, lo:hi]
        assert np.array_equal(got, want), f"mask differs in key chunk {c}"


@pytest.mark.parametrize("causal", [False, True])
def test_backward_masks_bit_exact(causal):
    """dV (the dK/dV kernel): with Q = 0 and dO one-hot on a chunk of queries,
    dV[j, i - chunk*d] = P_ij Z_ij keep_scale, nonzero exactly where Z_ij = 1.
    dQ (the dQ kernel): with Q = 0, K one-hot on a chunk of keys, V[:, 0] = 1 and
    dO[:, 0] = 1, dQ[i, j - chunk*d] = scale P_ij (Z_ij keep_scale - D_i): the kernel's
    value against that formula with the oracle's Z, closer than half of the gap that
    flipping any one Z_ij would open."""
    B, H, N, d, p = 1, 2, 260, 128, 0.3
    seed, offset = 2024, 11
    scale = 1.0 / np.sqrt(d)
    z = _masks(B, H, N, p, seed, offset)
    t = oracle.dropout_threshold(p)
    ks = 256.0 / (256 - t)
    vis = oracle.allowed_mask(N, N, causal, None)
    P = vis / vis.sum(axis=1, keepdims=True)
    q = torch.zeros(B, H, N, d, dtype=torch.float16, device="cuda")
    kr = torch.randn(B, H, N, d, device="cuda").to(torch.float16)
    vr = torch.randn(B, H, N, d, device="cuda").to(torch.float16)
    chunks = range(-(-N // d))
    for c in chunks:   # dV
        do = torch.from_numpy(np.broadcast_to(_onehot(N, d, c), (B, H, N, d)).copy())
        do = do.to(torch.float16).cuda()
        o, lse = fa.fa_fwd_dropout(q, kr, vr, p=p, seed=seed, offset=offset, causal=causal)
        _, _, dv = fa.fa_bwd_dropout(q, kr, vr, o, do, lse, p=p, seed=seed, offset=offset,
                                     causal=causal)
        torch.cuda.synchronize()
        lo, hi = c * d, min(N, (c + 1) * d)
        got = dv[..., : hi - lo].cpu().numpy() > 0            # [B,H,key j, query i - lo]
        want = np.swapaxes(z[..., lo:hi, :] & vis[None, None, lo:hi, :], -1, -2)
        assert np.array_equal(got, want), f"dV mask differs in query chunk {c}"
    v1 = torch.zeros(B, H, N, d, dtype=torch.float16, device="cuda")
    v1[..., 0] = 1.0
    for c in chunks:   # dQ
        k = torch.from_numpy(np.broadcast_to(_onehot(N, d, c), (B, H, N, d)).copy())
        k = k.to(torch.float16).cuda()
        o, lse = fa.fa_fwd_dropout(q, k, v1, p=p, seed=seed, offset=offset, causal=causal)
        dq, _, _ = fa.fa_bwd_dropout(q, k, v1, o, v1, lse, p=p, seed=seed, offset=offset,
                                     causal=causal)
        torch.cuda.synchronize()
        lo, hi = c * d, min(N, (c + 1) * d)
        for b in range(B):
            for h in range(H):
                zz = z[b, h] & vis
                D = (P * zz * ks).sum(axis=1)
                want = scale * P * (zz * ks - D[:, None])
                gap = scale * P * ks                            # change from one flip
                got = dq[b, h, :, : hi - lo].double().cpu().numpy()
                err = np.abs(got - want[:, lo:hi])
                sel = vis[:, lo:hi]
                assert np.all(err[sel] < 0.5 * gap[:, lo:hi][sel]), \
                    f"dQ mask differs in key chunk {c}, head ({b},{h})"
                assert np.all(got[~sel] == 0.0)


@pytest.mark.parametrize("d", [64, 128])
def test_p_zero_matches_dense(d):
    w, inp = workloads.custom(2, 3, 300, d, "bf16", True, kv_range=(100, 300), seed=79)
    dev = U.to_dev(inp)
    o, lse, (dq, dk, dv) = _run(inp, 0.0, 5, 0, dev)
    o_d, lse_d, dq_d, dk_d, dv_d = U.gpu_bwd(inp, dev)
    for a, b in ((o, o_d), (lse, lse_d), (dq, dq_d), (dk, dk_d), (dv, dv_d)):
        assert (a - b).abs().max().item() <= 1e-5


def test_deterministic_and_keyed():
    """Same key: bit-identical results; another seed or offset: another mask."""
    w, inp = workloads.custom(2, 2, 256, 128, "bf16", False, seed=80)
    dev = U.to_dev(inp)
    a = _run(inp, 0.25, 7, 1, dev)
    b = _run(inp, 0.25, 7, 1, dev)
    for x, y in zip((a[0], a[1]) + a[2], (b[0], b[1]) + b[2]):
        assert torch.equal(x, y)
    for seed, offset in ((8, 1), (7, 2)):
        c = _run(inp, 0.25, seed, offset, dev, backward=False)
        assert not torch.equal(a[0], c[0])
        assert torch.equal(a[1], c[1])          # lse is that of the undropped scores


def test_dropout_full_size():
    """B=2, H=16, N=4096, d=128, causal, Q x4, p = 0.1: two sampled heads against the
    oracle."""
    w = workloads.WORKLOADS[4]
    inp = workloads.draw(w)
    p, seed, offset = 0.1, 31337, 0
    U.say(f"[dropout] full size {w.name} p={p}")
    o, lse, (dq, dk, dv) = _run(inp, p, seed, offset)
    for t in (o, lse, dq, dk, dv):
        assert torch.isfinite(t).all()
    q, k, v, do = (U.f64(inp, n) for n in ("q", "k", "v", "dout"))
    t = oracle.dropout_threshold(p)
    for b, h in U.sample_heads(w.B, w.H, 2):
        z = oracle.keep_mask(w.N, b * w.H + h, p, seed, offset)
        ks = 256.0 / (256 - t)
        ro, rl = oracle.head_forward_dropout(q[b, h], k[b, h], v[b, h], w.scale, True, None,
                                             z, ks)
        U.compare(f"O ({b},{h})", o[b, h], ro, "bf16")
        U.compare(f"LSE ({b},{h})", lse[b, h], rl, "bf16")
        rq, rk, rv = oracle.head_backward_dropout(q[b, h], k[b, h], v[b, h], do[b, h],
                                                  w.scale, True, None, z, ks)
        U.compare(f"dQ ({b},{h})", dq[b, h], rq, "bf16")
        U.compare(f"dK ({b},{h})", dk[b, h], rk, "bf16")
        U.compare(f"dV ({b},{h})", dv[b, h], rv, "bf16")
