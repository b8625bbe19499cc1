"""Split-KV parity on the GPU: fa_fwd_partial and fa_merge (HIP, through the C ABI)
against the fp64 oracle's partial attention and merge, on the same seeded inputs."""
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


def _gpu_partial(inp, split_len, dev=None):
    dev = dev or U.to_dev(inp)
    o_p, l_p = fa.fa_fwd_partial(dev["q"], dev["k"], dev["v"], split_len=split_len,
                                 causal=inp["causal"], scale=inp["scale"], kv_len=dev["kv_len"])
    torch.cuda.synchronize()
    return o_p, l_p


def _oracle_partial(inp, split_len):
    q, k, v = (U.f64(inp, n) for n in "qkv")
    return oracle.attention_forward_split(q, k, v, inp["scale"], inp["causal"], U.kv_np(inp),
                                          split_len)


def _compare_partials(o_p, l_p, ref_o, ref_l, dtype):
    """Empty partials must be exactly (0, -inf); the rest within the tolerance."""
    lg = l_p.double().cpu().numpy()
    og = o_p.double().cpu().numpy()
    empty = np.isneginf(ref_l)
    assert np.array_equal(np.isneginf(lg), empty), "-inf pattern of lse_part differs"
    assert np.all(og[empty] == 0.0), "empty partial rows must be exactly 0"
    full = ~empty
    U.compare("O_part", torch.from_numpy(og[full]), ref_o[full], dtype)
    U.compare("LSE_part", torch.from_numpy(lg[full]), ref_l[full], dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N,split_len", [(64, 64), (130, 64), (300, 128), (257, 192)])
@pytest.mark.parametrize("causal,pad", [(False, False), (True, False), (False, True),
                                       (True, True)])
def test_partials_and_merge_small(dtype, d, N, split_len, causal, pad):
    kv = (1, N) if pad else None
    w, inp = workloads.custom(2, 2, N, d, dtype, causal, kv_range=kv, seed=300 + N + d)
    U.say(f"[split] N={N} d={d} {dtype} causal={causal} pad={pad} split_len={split_len}")
    dev = U.to_dev(inp)
    o_p, l_p = _gpu_partial(inp, split_len, dev)
    ref_op, ref_lp = _oracle_partial(inp, split_len)
    assert o_p.shape[0] == fa.fa_split_count(N, split_len) == ref_op.shape[0]
    _compare_partials(o_p, l_p, ref_op, ref_lp, dtype)
    o, lse = fa.fa_merge(o_p, l_p)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.attention_forward(*(U.f64(inp, n) for n in "qkv"), inp["scale"],
                                            inp["causal"], U.kv_np(inp))
    U.compare("merged O", o, ref_o, dtype)
    U.compare("merged LSE", lse, ref_l, dtype)


def test_merge_kernel_alone():
    """fa_merge on random float32 partials (with empty splits and all-empty rows) against
    the oracle's merge in float64, to float32 rounding."""
    rng = np.random.default_rng(41)
    P, B, H, N, d = 5, 2, 3, 77, 128
    o_p = rng.standard_normal((P, B, H, N, d)).astype(np.float32)
    l_p = (8.0 * rng.standard_normal((P, B, H, N))).astype(np.float32)
    hole = rng.random((P, B, H, N)) < 0.3
    l_p[hole] = -np.inf
    o_p[hole] = 0.0
    l_p[:, 0, 0, 5] = -np.inf      # a row with no visible key anywhere
    o_p[:, 0, 0, 5] = 0.0
    l_p[:, 1, 2, 9] = 500.0        # large but equal LSE: weights 1/P each
    ref_o, ref_l = oracle.merge_partials(o_p.astype(np.float64), l_p.astype(np.float64))
    o, lse = fa.fa_merge(torch.from_numpy(o_p).cuda(), torch.from_numpy(l_p).cuda())
    torch.cuda.synchronize()
    lg = lse.double().cpu().numpy()
    assert np.array_equal(np.isneginf(lg), np.isneginf(ref_l))
    assert np.all(o.cpu().numpy()[0, 0, 5] == 0.0)
    fin = ~np.isneginf(ref_l)
    U.compare("merge O", o, ref_o, "f32")
    U.compare("merge LSE", torch.from_numpy(lg[fin]), ref_l[fin], "f32")
    for P1 in (1, 2):   # one split is a copy; two splits, the pairwise rule
        o1, l1 = fa.fa_merge(torch.from_numpy(o_p[:P1].copy()).cuda(),
                             torch.from_numpy(l_p[:P1].copy()).cuda())
        r1o, r1l = oracle.merge_partials(o_p[:P1].astype(np.float64), l_p[:P1].astype(np.float64))
        U.compare(f"merge O (P={P1})", o1, r1o, "f32")
        f1 = ~np.isneginf(r1l)
        U.compare(f"merge LSE (P={P1})", torch.from_numpy(l1.double().cpu().numpy()[f1]),
                  r1l[f1], "f32")


@pytest.mark.parametrize("split_len", [1024, 4096])
def test_split_full_size(split_len):
    """B=2, H=16, N=4096, d=128, causal, Q x4 (the benchmarked shape): partials of two
    sampled heads against the oracle, and the merge of all heads against the unsplit
    kernel and, for the sampled heads, the oracle."""
    w = workloads.WORKLOADS[4]
    inp = workloads.draw(w)
    U.say(f"[split] full size {w.name} split_len={split_len}")
    dev = U.to_dev(inp)
    o_p, l_p = _gpu_partial(inp, split_len, dev)
    o, lse = fa.fa_merge(o_p, l_p)
    o_ref_gpu, lse_ref_gpu = U.gpu_fwd(inp, dev)
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    # merged vs unsplit on the GPU: same result up to rounding order
    assert (o - o_ref_gpu).abs().max().item() < 2e-3
    assert (lse - lse_ref_gpu).abs().max().item() < 2e-3
    heads = U.sample_heads(w.B, w.H, 2)
    q, k, v = (U.f64(inp, n) for n in "qkv")
    for b, h in heads:
        ref_o, ref_l = oracle.head_forward(q[b, h], k[b, h], v[b, h], w.scale, w.causal)
        U.compare(f"merged O ({b},{h})", o[b, h], ref_o, "bf16")
        U.compare(f"merged LSE ({b},{h})", lse[b, h], ref_l, "bf16")
        for p, (kb, ke) in enumerate(oracle.split_ranges(w.N, split_len)):
            rp_o, rp_l = oracle.head_forward_range(q[b, h], k[b, h], v[b, h], w.scale,
                                                   w.causal, None, kb, ke)
            _compare_partials(o_p[p, b, h], l_p[p, b, h], rp_o, rp_l, "bf16")


@pytest.mark.parametrize("B,H,N,d,causal", [(1, 2, 2048, 128, True), (1, 2, 4096, 64, False)])
def test_split_hint_path_matches_oracle(B, H, N, d, causal):
    """The split fa_split_hint recommends, run as fa_fwd_partial + fa_merge, gives the
    oracle's O and LSE (the hint is nonzero on both shapes: few query blocks)."""
    h = fa.fa_split_hint(B, H, N, d, causal=causal)
    assert h > 0
    w, inp = workloads.custom(B, H, N, d, "bf16", causal, seed=900 + d, with_dout=False)
    U.say(f"[split] hint B={B} H={H} N={N} d={d} causal={causal} split_len={h}")
    o_p, l_p = _gpu_partial(inp, h)
    o, lse = fa.fa_merge(o_p, l_p)
    torch.cuda.synchronize()
    ref = U.oracle_fwd(inp, workers=1)
    ro = np.stack([[ref[(b, hh)][0] for hh in range(H)] for b in range(B)])
    rl = np.stack([[ref[(b, hh)][1] for hh in range(H)] for b in range(B)])
    U.compare("O", o, ro, "bf16")
    U.compare("LSE", lse, rl, "bf16")


@pytest.mark.parametrize("B,H,N,d,causal", [(1, 2, 2048, 128, True), (1, 2, 4096, 64, False),
                                            (1, 3, 300, 128, True)])
def test_fwd_auto(B, H, N, d, causal):
    """fa_fwd_auto: the hinted split through its workspace matches the oracle; where no split
    pays (N = 300) it is fa_fwd, bit for bit."""
    w, inp = workloads.custom(B, H, N, d, "bf16", causal, seed=950 + N + d, with_dout=False)
    U.say(f"[split] auto B={B} H={H} N={N} d={d} causal={causal} "
          f"workspace={fa.fa_fwd_workspace_size(B, H, N, d, causal=causal)}")
    dev = U.to_dev(inp)
    o, lse = fa.fa_fwd_auto(dev["q"], dev["k"], dev["v"], causal=causal, scale=inp["scale"])
    torch.cuda.synchronize()
    if fa.fa_split_hint(B, H, N, d, causal=causal) == 0:
        o2, l2 = fa.fa_fwd(dev["q"], dev["k"], dev["v"], causal=causal, scale=inp["scale"])
        torch.cuda.synchronize()
        assert torch.equal(o, o2) and torch.equal(lse, l2)
    ref = U.oracle_fwd(inp, workers=1)
    ro = np.stack([[ref[(b, hh)][0] for hh in range(H)] for b in range(B)])
    rl = np.stack([[ref[(b, hh)][1] for hh in range(H)] for b in range(B)])
    U.compare("O", o, ro, "bf16")
    U.compare("LSE", lse, rl, "bf16")
