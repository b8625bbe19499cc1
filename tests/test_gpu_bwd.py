"""Backward parity on the GPU: fa_bwd (HIP, through the C ABI) against the fp64 oracle's
gradients on the same seeded inputs, element by element, plus GPU-side invariants."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    U.require_gpu()


def _stack(ref, heads, i):
    return np.stack([ref[h][i] for h in heads])


def _sel(t, heads):
    idx_b = torch.tensor([h[0] for h in heads])
    idx_h = torch.tensor([h[1] for h in heads])
    return t.cpu()[idx_b, idx_h]


@pytest.mark.parametrize("cfg", [3, 4])
def test_bwd_workload(cfg):
    """Workloads with a backward pass at full size, every head compared."""
    w = workloads.WORKLOADS[cfg]
    U.say(f"[bwd] workload {cfg} {w.name}")
    inp = workloads.draw(w)
    o, lse, dq, dk, dv = U.gpu_bwd(inp)
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    ref = U.oracle_bwd(inp, heads=heads)
    rep = {}
    for name, t, i in (("dQ", dq, 0), ("dK", dk, 1), ("dV", dv, 2)):
        U.compare(name, _sel(t, heads), _stack(ref, heads, i), w.dtype, rep)
    for t in (dq, dk, dv):
        assert torch.isfinite(t).all()
    U.say(f"  errors {rep}")


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 7, 65, 129, 257])
@pytest.mark.parametrize("causal,pad", [(False, False), (True, False), (False, True),
                                       (True, True)])
def test_bwd_small(dtype, d, N, causal, pad):
    kv = (1, N) if pad else None
    w, inp = workloads.custom(2, 2, N, d, dtype, causal, kv_range=kv, seed=100 + N + d)
    U.say(f"[bwd] small N={N} d={d} {dtype} causal={causal} pad={pad}")
    o, lse, dq, dk, dv = U.gpu_bwd(inp)
    heads = [(b, h) for b in range(2) for h in range(2)]
    ref = U.oracle_bwd(inp, workers=1)
    for name, t, i in (("dQ", dq, 0), ("dK", dk, 1), ("dV", dv, 2)):
        U.compare(name, _sel(t, heads), _stack(ref, heads, i), dtype)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal,pad", [(False, False), (True, False), (False, True),
                                       (True, True)])
def test_bwd_wide_grid(d, causal, pad):
    """B*H*ceil(N/128) = 768 dK/dV workgroups, three per compute unit: head_dim 64 runs
    the one-wave dK/dV kernel here (smaller grids run the two-wave one); every head."""
    N = 300
    w, inp = workloads.custom(8, 32, N, d, "bf16", causal, kv_range=(1, N) if pad else None,
                              seed=41 + d)
    U.say(f"[bwd] wide grid N={N} d={d} causal={causal} pad={pad}")
    o, lse, dq, dk, dv = U.gpu_bwd(inp)
    heads = [(b, h) for b in range(8) for h in range(32)]
    ref = U.oracle_bwd(inp, heads=heads)
    for name, t, i in (("dQ", dq, 0), ("dK", dk, 1), ("dV", dv, 2)):
        U.compare(name, _sel(t, heads), _stack(ref, heads, i), "bf16")


@pytest.mark.parametrize("N", [447, 511, 575, 703])
def test_causal_padded_mid_sizes(N):
    """Causal with key padding at head_dim 128 over two or three 256-row query blocks: the
    forward's per-wave tail steps begin at every tile offset modulo the three LDS buffers,
    some waves' rows run past N, and the 8-wave row groups are paired per SIMD in the
    forward and dQ kernels. O, LSE and all three gradients against the oracle."""
    w, inp = workloads.custom(2, 2, N, 128, "bf16", True, kv_range=(N // 3, N), seed=300 + N)
    U.say(f"[bwd] causal padded mid-size N={N} kv_len={inp['kv_len'].tolist()}")
    o, lse, dq, dk, dv = U.gpu_bwd(inp)
    heads = [(b, h) for b in range(2) for h in range(2)]
    ref_f = U.oracle_fwd(inp, workers=1)
    U.compare("O", _sel(o, heads), _stack(ref_f, heads, 0), "bf16")
    U.compare("LSE", _sel(lse, heads), _stack(ref_f, heads, 1), "bf16")
    ref = U.oracle_bwd(inp, workers=1)
    for name, t, i in (("dQ", dq, 0), ("dK", dk, 1), ("dV", dv, 2)):
        U.compare(name, _sel(t, heads), _stack(ref, heads, i), "bf16")


def test_bwd_peaky_long():
    """Q x4 (peaky softmax) over 1100 keys, causal, d=128: the config-4 regime at a size
    the oracle checks in full."""
    w, inp = workloads.custom(1, 3, 1100, 128, "bf16", True, q_mult=4.0, seed=21)
    o, lse, dq, dk, dv = U.gpu_bwd(inp)
    heads = [(0, h) for h in range(3)]
    ref = U.oracle_bwd(inp)
    for name, t, i in (("dQ", dq, 0), ("dK", dk, 1), ("dV", dv, 2)):
        U.compare(name, _sel(t, heads), _stack(ref, heads, i), "bf16")


def test_bwd_padded_keys_get_zero_gradient():
    w, inp = workloads.custom(3, 2, 300, 64, "bf16", False, kv_range=(1, 300), seed=22)
    o, lse, dq, dk, dv = U.gpu_bwd(inp)
    for b, n in enumerate(inp["kv_len"].tolist()):
        assert torch.count_nonzero(dk[b, :, n:]) == 0
        assert torch.count_nonzero(dv[b, :, n:]) == 0


def test_bwd_gradient_sums():
    """sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i (rows of P sum to 1), to fp16 rounding."""
    w, inp = workloads.custom(2, 2, 513, 128, "bf16", True, seed=23)
    o, lse, dq, dk, dv = U.gpu_bwd(inp)
    do = inp["dout"].double()
    assert (dk.double().sum(2).cpu()).abs().max() < 5e-2
    assert (dv.double().sum(2).cpu() - do.sum(2)).abs().max() < 5e-2


def test_bwd_deterministic():
    """Every gradient is written once (no atomics): runs are bit-identical."""
    w, inp = workloads.custom(2, 2, 640, 64, "bf16", True, kv_range=(300, 640), seed=24)
    dev = U.to_dev(inp)
    r1 = U.gpu_bwd(inp, dev)
    r2 = U.gpu_bwd(inp, dev)
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)


def test_bwd_stages_match_fa_bwd():
    """fa_bwd_stage 0, 1, 2 give fa_bwd's results bit for bit, also with stages 1 and 2
    on two streams, and so do stages 3, 1 (dQ forming and writing D, then dK/dV)."""
    import io_aware_softmax_tiled_amd as fa
    w, inp = workloads.custom(2, 3, 700, 128, "bf16", True, kv_range=(350, 700), seed=25)
    dev = U.to_dev(inp)
    o, lse, dq, dk, dv = U.gpu_bwd(inp, dev)
    ws = torch.empty(fa.fa_bwd_workspace_size(2, 3, 700, 128), dtype=torch.uint8,
                     device="cuda")
    outs = [torch.full_like(dq, float("nan")) for _ in range(3)]
    kw = dict(causal=True, scale=inp["scale"], kv_len=dev["kv_len"])
    for st in range(3):
        fa.fa_bwd_stage(st, dev["q"], dev["k"], dev["v"], o, dev["dout"], lse, *outs, ws, **kw)
    torch.cuda.synchronize()
    for a, b in zip(outs, (dq, dk, dv)):
        assert torch.equal(a, b)
    outs2 = [torch.full_like(dq, float("nan")) for _ in range(3)]
    side = torch.cuda.Stream()
    fa.fa_bwd_stage(0, dev["q"], dev["k"], dev["v"], o, dev["dout"], lse, *outs2, ws, **kw)
    side.wait_stream(torch.cuda.current_stream())
    fa.fa_bwd_stage(1, dev["q"], dev["k"], dev["v"], o, dev["dout"], lse, *outs2, ws, **kw)
    fa.fa_bwd_stage(2, dev["q"], dev["k"], dev["v"], o, dev["dout"], lse, *outs2, ws,
                    stream=side, **kw)
    torch.cuda.synchronize()
    for a, b in zip(outs2, (dq, dk, dv)):
        assert torch.equal(a, b)
    # stage 3 (dQ writing D) then stage 1 is what fa_bwd runs; D from either stage is the
    # same bits
    outs3 = [torch.full_like(dq, float("nan")) for _ in range(3)]
    ws.fill_(255)
    for st in (3, 1):
        fa.fa_bwd_stage(st, dev["q"], dev["k"], dev["v"], o, dev["dout"], lse, *outs3, ws, **kw)
    torch.cuda.synchronize()
    for a, b in zip(outs3, (dq, dk, dv)):
        assert torch.equal(a, b)


@pytest.mark.parametrize("B,H", [(1, 1), (1, 3), (3, 5), (2, 6), (1, 9)])
def test_head_counts_not_multiple_of_8(B, H):
    """B*H below or off a multiple of 8 (workgroups then spread with heads varying
    fastest instead of one head per XCD): forward and backward against the oracle."""
    w, inp = workloads.custom(B, H, 700, 128, "bf16", True, seed=60 + B * H)
    U.say(f"[bwd] B={B} H={H} N=700 d=128 causal")
    o, lse, dq, dk, dv = U.gpu_bwd(inp)
    q, k, v, do = (U.f64(inp, n) for n in ("q", "k", "v", "dout"))
    ro, rl = oracle.attention_forward(q, k, v, inp["scale"], True)
    rq, rk, rv = oracle.attention_backward(q, k, v, do, inp["scale"], True)
    for name, got, ref in (("O", o, ro), ("LSE", lse, rl), ("dQ", dq, rq), ("dK", dk, rk),
                           ("dV", dv, rv)):
        U.compare(name, got, ref, "bf16")


@pytest.mark.parametrize("dtype,mult", [("bf16", 2.0 ** -20), ("bf16", 2.0 ** 12),
                                        ("bf16", 2.0 ** -60), ("f16", 2.0 ** -10)])
def test_bwd_gradient_magnitude(dtype, mult):
    """dO scaled by a power of two (exact in the input dtype): the gradients scale by the
    same factor, so grad / mult must meet the usual tolerance against the oracle's
    gradients of the same inputs divided by mult. Small dO would otherwise leave the
    fp16 range of the matrix-core operands (dS, dO) and large dO would overflow dS;
    peaky rows (Q x 4) over 1000 keys, causal, head_dim 128."""
    w, inp = workloads.custom(1, 4, 1000, 128, dtype, True, q_mult=4.0, seed=9)
    inp["dout"] = (inp["dout"].double() * mult).to(workloads.DTYPES[dtype])
    U.say(f"[bwd] gradient magnitude {dtype} x {mult:g}")
    o, lse, dq, dk, dv = U.gpu_bwd(inp)
    ref = U.oracle_bwd(inp)
    heads = [(0, h) for h in range(4)]
    rep = {}
    for name, t, i in (("dQ", dq, 0), ("dK", dk, 1), ("dV", dv, 2)):
        U.compare(name, _sel(t, heads).double() / mult, _stack(ref, heads, i) / mult, dtype, rep)
    U.say(f"  errors (relative to the gradient scale) {rep}")


@pytest.mark.parametrize("B,H,N,d,causal,kv,q_mult", [
    (1, 1, 256, 64, False, None, 1.0),        # the fp32 workload's shape, with a backward pass
    (2, 2, 1000, 128, True, None, 1.0),       # causal, several tiles
    (2, 3, 517, 64, False, (100, 517), 1.0),  # key padding, ragged
    (2, 2, 1000, 128, True, None, 4.0),       # peaky rows (scores of order 20)
])
def test_bwd_f32(B, H, N, d, causal, kv, q_mult):
    """fp32 backward (fp32 matrix cores throughout) against the oracle at 1e-5 max-abs.
    With peaky rows the scores reach |s| ~ 20 and fp32 rounding of s alone perturbs P by
    ~2^-24 * |s| / scale relative, so the bar there is 1e-5 times the gradient's
    magnitude (max(1, max|ref|)), the same relative accuracy."""
    w, inp = workloads.custom(B, H, N, d, "f32", causal, kv_range=kv, q_mult=q_mult, seed=N)
    U.say(f"[bwd] f32 B={B} H={H} N={N} d={d} causal={causal} kv={kv} q x{q_mult}")
    o, lse, dq, dk, dv = U.gpu_bwd(inp)
    ref = U.oracle_bwd(inp)
    heads = [(b, h) for b in range(B) for h in range(H)]
    rep = {}
    for name, t, i in (("dQ", dq, 0), ("dK", dk, 1), ("dV", dv, 2)):
        r = _stack(ref, heads, i)
        mag = max(1.0, float(np.abs(r).max())) if q_mult != 1.0 else 1.0
        U.compare(name, _sel(t, heads).double() / mag, r / mag, "f32", rep)
    U.say(f"  errors {rep}")


def test_bwd_f32_stages_match_fa_bwd():
    """fp32: stages 0, 1, 2 give fa_bwd's results bit for bit."""
    import io_aware_softmax_tiled_amd as fa
    w, inp = workloads.custom(1, 2, 300, 128, "f32", True, seed=4)
    dev = U.to_dev(inp)
    o, lse = fa.fa_fwd(dev["q"], dev["k"], dev["v"], causal=True, scale=inp["scale"])
    ref = fa.fa_bwd(dev["q"], dev["k"], dev["v"], o, dev["dout"], lse, causal=True,
                    scale=inp["scale"])
    outs = [torch.empty_like(ref[0]) for _ in range(3)]
    ws = torch.empty(fa.fa_bwd_workspace_size(1, 2, 300, 128), dtype=torch.uint8, device="cuda")
    for stage in (0, 1, 2):
        fa.fa_bwd_stage(stage, dev["q"], dev["k"], dev["v"], o, dev["dout"], lse, *outs, ws,
                        causal=True, scale=inp["scale"])
    torch.cuda.synchronize()
    for a, b in zip(outs, ref):
        assert torch.equal(a, b)
