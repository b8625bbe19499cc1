"""Forward parity on the GPU: fa_fwd (HIP, through the C ABI) against the fp64 oracle on
the same seeded inputs, element by element, plus GPU-side invariants."""
import numpy as np
import pytest
import torch

import io_aware_softmax_tiled_amd as fa
import workloads
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    U.require_gpu()


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_fwd_workload(cfg):
    """The five workloads at full size, every head compared element by element."""
    w = workloads.WORKLOADS[cfg]
    U.say(f"[fwd] workload {cfg} {w.name}")
    inp = workloads.draw(w, with_dout=False)
    o, lse = U.gpu_fwd(inp)
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    ref = U.oracle_fwd(inp, heads=heads)
    rep = {}
    ro = np.stack([ref[h][0] for h in heads])
    rl = np.stack([ref[h][1] for h in heads])
    idx_b = torch.tensor([h[0] for h in heads])
    idx_h = torch.tensor([h[1] for h in heads])
    oc, lc = o.cpu(), lse.cpu()
    U.compare("O", oc[idx_b, idx_h], ro, w.dtype, rep)
    U.compare("LSE", lc[idx_b, idx_h], rl, w.dtype, rep)
    assert torch.isfinite(oc).all() and torch.isfinite(lc).all()
    U.say(f"  errors {rep}")


SHAPES = [1, 7, 64, 65, 129, 257]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", SHAPES)
@pytest.mark.parametrize("causal,pad", [(False, False), (True, False), (False, True),
                                       (True, True)])
def test_fwd_small(dtype, d, N, causal, pad):
    """Ragged and tiny shapes spanning several tiles, every mask mode and dtype."""
    kv = (1, N) if pad else None
    w, inp = workloads.custom(2, 3, N, d, dtype, causal, kv_range=kv, seed=N + d,
                              with_dout=False)
    U.say(f"[fwd] small N={N} d={d} {dtype} causal={causal} pad={pad}")
    o, lse = U.gpu_fwd(inp)
    ref = U.oracle_fwd(inp, workers=1)
    ro = np.stack([[ref[(b, h)][0] for h in range(3)] for b in range(2)])
    rl = np.stack([[ref[(b, h)][1] for h in range(3)] for b in range(2)])
    U.compare("O", o, ro, dtype)
    U.compare("LSE", lse, rl, dtype)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal,pad", [(False, False), (True, False), (True, True)])
def test_fwd_f32_many_subblocks_per_wave(d, causal, pad):
    """fp32 at N = 1500 with Q x4: each wave of the key-split workgroup takes several
    32-key sub-blocks (raising its reference maximum between them) and the waves' partial
    states, with different maxima, are combined at the end."""
    N = 1500
    w, inp = workloads.custom(1, 2, N, d, "f32", causal, kv_range=(N // 2, N) if pad else None,
                              q_mult=4.0, seed=60 + d, with_dout=False)
    U.say(f"[fwd] f32 N={N} d={d} causal={causal} pad={pad}")
    o, lse = U.gpu_fwd(inp)
    ref = U.oracle_fwd(inp, workers=1)
    ro = np.stack([ref[(0, h)][0] for h in range(2)])[None]
    rl = np.stack([ref[(0, h)][1] for h in range(2)])[None]
    U.compare("O", o, ro, "f32")
    U.compare("LSE", lse, rl, "f32")


def test_fwd_peaky_rows_and_many_tiles():
    """Q scaled x4 (peaky rows that exercise the rescale) over 1000 keys, bf16, d=128."""
    w, inp = workloads.custom(1, 4, 1000, 128, "bf16", True, q_mult=4.0, seed=7,
                              with_dout=False)
    o, lse = U.gpu_fwd(inp)
    ref = U.oracle_fwd(inp)
    ro = np.stack([ref[(0, h)][0] for h in range(4)])[None]
    rl = np.stack([ref[(0, h)][1] for h in range(4)])[None]
    U.compare("O", o, ro, "bf16")
    U.compare("LSE", lse, rl, "bf16")


def test_fwd_large_scores_no_overflow():
    """Scores near +-1e3 (Q x 64 at d=64, bf16): exponents stay finite."""
    w, inp = workloads.custom(1, 2, 300, 64, "bf16", False, q_mult=64.0, seed=3,
                              with_dout=False)
    o, lse = U.gpu_fwd(inp)
    ref = U.oracle_fwd(inp)
    U.compare("O", o, np.stack([ref[(0, h)][0] for h in range(2)])[None], "bf16")
    # LSE is of order 1e2..1e3 here: the same absolute bar as every other output
    U.compare("LSE", lse, np.stack([ref[(0, h)][1] for h in range(2)])[None], "bf16")


def test_padded_keys_are_inert():
    """Changing K/V rows at or past kv_len[b] leaves O and LSE bit-identical."""
    w, inp = workloads.custom(3, 2, 200, 64, "bf16", False, kv_range=(1, 200), seed=11,
                              with_dout=False)
    dev = U.to_dev(inp)
    o1, l1 = U.gpu_fwd(inp, dev)
    k2, v2 = dev["k"].clone(), dev["v"].clone()
    for b, n in enumerate(inp["kv_len"].tolist()):
        k2[b, :, n:] = 37.0
        v2[b, :, n:] = -1000.0
    dev2 = dict(dev, k=k2, v=v2)
    o2, l2 = U.gpu_fwd(inp, dev2)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_causal_future_keys_are_inert():
    """Under the causal mask, changing K_j, V_j for j > i leaves rows 0..i bit-identical."""
    w, inp = workloads.custom(1, 2, 300, 128, "bf16", True, seed=12, with_dout=False)
    dev = U.to_dev(inp)
    o1, l1 = U.gpu_fwd(inp, dev)
    for i in (0, 63, 64, 127, 200):
        k2, v2 = dev["k"].clone(), dev["v"].clone()
        k2[:, :, i + 1:] = 5.0
        v2[:, :, i + 1:] = 99.0
        o2, l2 = U.gpu_fwd(inp, dict(dev, k=k2, v=v2))
        assert torch.equal(o1[:, :, :i + 1], o2[:, :, :i + 1]), i
        assert torch.equal(l1[:, :, :i + 1], l2[:, :, :i + 1]), i


def test_causal_row0_is_v0_and_zero_q_is_prefix_mean():
    w, inp = workloads.custom(1, 2, 130, 64, "bf16", True, seed=13, with_dout=False)
    o, lse = U.gpu_fwd(inp)
    assert torch.equal(o[:, :, 0].cpu(), inp["v"][:, :, 0].float())
    inp0 = dict(inp, q=torch.zeros_like(inp["q"]))
    o0, l0 = U.gpu_fwd(inp0)
    v = inp["v"].double()
    prefix = torch.cumsum(v, dim=2) / torch.arange(1, 131, dtype=torch.float64)[:, None]
    assert (o0.cpu().double() - prefix).abs().max() < 2e-3
    assert (l0.cpu().double() - torch.log(torch.arange(1, 131, dtype=torch.float64))).abs().max() < 1e-5


def test_fwd_deterministic():
    w, inp = workloads.custom(2, 4, 777, 128, "bf16", True, kv_range=(100, 777), seed=14,
                              with_dout=False)
    dev = U.to_dev(inp)
    o1, l1 = U.gpu_fwd(inp, dev)
    o2, l2 = U.gpu_fwd(inp, dev)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_fwd_on_side_stream():
    """The kernel runs on the caller's current stream."""
    w, inp = workloads.custom(1, 2, 256, 64, "f16", False, seed=15, with_dout=False)
    dev = U.to_dev(inp)
    ref_o, ref_l = U.gpu_fwd(inp, dev)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        o, l = fa.fa_fwd(dev["q"], dev["k"], dev["v"], scale=inp["scale"])
    s.synchronize()
    assert torch.equal(o, ref_o) and torch.equal(l, ref_l)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal,pad", [(False, False), (True, False), (False, True),
                                       (True, True)])
def test_fwd_wide_grid(d, causal, pad):
    """Enough heads that the 256-row (8-wave) workgroups are used, with a ragged N."""
    N = 300
    w, inp = workloads.custom(8, 32, N, d, "bf16", causal, kv_range=(1, N) if pad else None,
                              seed=31 + d, with_dout=False)
    U.say(f"[fwd] wide grid N={N} d={d} causal={causal} pad={pad}")
    o, lse = U.gpu_fwd(inp)
    heads = [(b, h) for b in range(8) for h in range(32)]
    ref = U.oracle_fwd(inp)
    ro = np.stack([np.stack([ref[(b, h)][0] for h in range(32)]) for b in range(8)])
    rl = np.stack([np.stack([ref[(b, h)][1] for h in range(32)]) for b in range(8)])
    U.compare("O", o, ro, "bf16")
    U.compare("LSE", lse, rl, "bf16")
