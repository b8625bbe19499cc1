"""Deferred-P.V forward parity on the GPU: fa_fwd_deferred (HIP, through the C ABI)
against the fp64 oracle's definition of attention, on the same seeded inputs, and
against the single-pass forward."""
import numpy as np
import pytest
import torch

import io_aware_softmax_tiled_amd as fa
import oracle
import workloads
from oracle import page_algorithms as pa
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    U.require_gpu()


def _run(inp, dev=None):
    dev = dev or U.to_dev(inp)
    o, lse = fa.fa_fwd_deferred(dev["q"], dev["k"], dev["v"], causal=inp["causal"],
                                scale=inp["scale"], kv_len=dev["kv_len"])
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 64, 130, 300, 512])
@pytest.mark.parametrize("causal,pad", [(False, False), (True, False), (False, True),
                                       (True, True)])
def test_deferred_small(dtype, d, N, causal, pad):
    kv = (1, N) if pad else None
    w, inp = workloads.custom(2, 3, N, d, dtype, causal, kv_range=kv, seed=900 + N + d,
                              with_dout=False)
    U.say(f"[deferred] N={N} d={d} {dtype} causal={causal} pad={pad}")
    dev = U.to_dev(inp)
    o, lse = _run(inp, dev)
    ref_o, ref_l = oracle.attention_forward(*(U.f64(inp, n) for n in "qkv"), inp["scale"],
                                            causal, U.kv_np(inp))
    U.compare("O", o, ref_o, dtype)
    U.compare("LSE", lse, ref_l, dtype)
    o1, l1 = U.gpu_fwd(inp, dev)
    assert (o - o1).abs().max().item() < 2e-3
    assert (lse - l1).abs().max().item() < 2e-3


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_deferred_rising_scores(d, causal):
    """Scores rise by more than 2^16 in the exponent from one 32-key sub-block to the
    next, so every sub-block raises the reference maximum and every earlier numerator
    block is rescaled (left unscaled, they would outweigh the true maximum)."""
    N, B, H = 512, 1, 2
    scale = 1.0 / np.sqrt(d)
    step = 17.0 / (scale * np.log2(np.e) * 32)         # per key, in units of k[:, 0]
    rng = np.random.default_rng(12)
    q = np.zeros((B, H, N, d))
    q[..., 0] = 1.0
    q[..., 1:] = 0.05 * rng.standard_normal((B, H, N, d - 1))
    k = 0.05 * rng.standard_normal((B, H, N, d))
    k[..., 0] = step * np.arange(N)
    v = rng.standard_normal((B, H, N, d))
    t = {n: torch.from_numpy(x).to(torch.bfloat16) for n, x in (("q", q), ("k", k), ("v", v))}
    o, lse = fa.fa_fwd_deferred(t["q"].cuda(), t["k"].cuda(), t["v"].cuda(), causal=causal,
                                scale=scale)
    torch.cuda.synchronize()
    q64, k64, v64 = (workloads.as_f64(t[n]) for n in "qkv")
    ref_o, ref_l = oracle.attention_forward(q64, k64, v64, scale, causal)
    U.compare("O", o, ref_o, "bf16")
    U.compare("LSE", lse, ref_l, "bf16")
    # the issue thread's own algorithm agrees with the definition on these inputs
    pa_o, pa_l = pa.attention_deferred_pv(
        q64[0, 0, :96], k64[0, 0, :96], v64[0, 0, :96], 32, scale,
        oracle.allowed_mask(96, 96, causal, None))
    r_o, r_l = oracle.head_forward(q64[0, 0, :96], k64[0, 0, :96], v64[0, 0, :96], scale,
                                   causal)
    assert np.abs(pa_o - r_o).max() < 1e-9 and np.abs(pa_l - r_l).max() < 1e-9


def test_deferred_bert_large_keypad():
    """B=8, H=16, N=512, d=64, key padding U{256..512}: three sampled heads against the
    oracle, all heads against the single-pass forward."""
    w = workloads.WORKLOADS[3]
    inp = workloads.draw(w, with_dout=False)
    U.say(f"[deferred] full size {w.name}")
    dev = U.to_dev(inp)
    o, lse = _run(inp, dev)
    o1, l1 = U.gpu_fwd(inp, dev)
    assert (o - o1).abs().max().item() < 2e-3 and (lse - l1).abs().max().item() < 2e-3
    heads = U.sample_heads(w.B, w.H, 3)
    ref = U.oracle_fwd(inp, heads=heads)
    for b, h in heads:
        U.compare(f"O ({b},{h})", o[b, h], ref[(b, h)][0], "bf16")
        U.compare(f"LSE ({b},{h})", lse[b, h], ref[(b, h)][1], "bf16")


def test_deferred_limit():
    w, inp = workloads.custom(1, 1, 513, 64, "bf16", False, seed=1, with_dout=False)
    with pytest.raises(fa.FaError):
        _run(inp)
