"""Parity at the longest sequence the library accepts (N = 2^22, one head, causal),
where the oracle can only afford blocks of query rows: O, LSE and dQ on the first, a
middle and the last 16 rows; dK and dV on the last 16 keys (under the causal mask only
the last rows see them, so the last row block holds their whole gradient); and the
column sum of dV, which equals the column sum of dO at any size."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

N_MAX = 1 << 22
ROWS = 16


@pytest.fixture(autouse=True)
def _gpu():
    U.require_gpu()


@pytest.mark.parametrize("d", [64, 128])
def test_max_sequence_length(d):
    w, inp = workloads.custom(1, 1, N_MAX, d, "bf16", True, seed=4242)
    U.say(f"[max] N={N_MAX} d={d} bf16 causal: forward and backward")
    o, lse, dq, dk, dv = U.gpu_bwd(inp)
    for t in (o, lse, dq, dk, dv):
        assert torch.isfinite(t).all()
    q, k, v, do = (U.f64(inp, n)[0, 0] for n in ("q", "k", "v", "dout"))
    del inp
    for r0 in (0, N_MAX // 2 + 7, N_MAX - ROWS):
        r1 = r0 + ROWS
        U.say(f"[max] oracle rows {r0}..{r1 - 1}")
        ro, rl, rdq, rdk, rdv = oracle.head_row_block(q, k, v, do, w.scale, True, None, r0, r1)
        U.compare(f"O rows {r0}+", o[0, 0, r0:r1], ro, "bf16")
        U.compare(f"LSE rows {r0}+", lse[0, 0, r0:r1], rl, "bf16")
        U.compare(f"dQ rows {r0}+", dq[0, 0, r0:r1], rdq, "bf16")
    U.compare("dK last keys", dk[0, 0, N_MAX - ROWS:], rdk[N_MAX - ROWS:], "bf16")
    U.compare("dV last keys", dv[0, 0, N_MAX - ROWS:], rdv[N_MAX - ROWS:], "bf16")
    # sum_j dV_j = sum_i dO_i (rows of P sum to 1); the kernel's P is rounded to fp16,
    # so the two differ by at most about 2^-11 of sum_i |dO_i| per column
    sv = dv[0, 0].double().sum(dim=0).cpu().numpy()
    so = do.sum(axis=0)
    bound = 1e-3 * np.abs(do).sum(axis=0)
    assert np.all(np.abs(sv - so) <= bound), float(np.max(np.abs(sv - so) / bound))


SPARSE_MAX_N = 1 << 18


@pytest.mark.parametrize("d", [64, 128])
def test_max_sparse_length(d):
    """Block-sparse at its limit (N = 2^18, one head, causal, 5% of the lower block
    triangle plus the diagonal): O, LSE, dQ on three 16-row blocks and dK, dV on the last
    16 keys against the oracle's row blocks, and sum_j dV_j = sum_i dO_i."""
    import io_aware_softmax_tiled_amd as fa
    N, blk = SPARSE_MAX_N, 128
    w, inp = workloads.custom(1, 1, N, d, "bf16", True, seed=4343)
    nb = N // blk
    rng = np.random.default_rng(17)
    m = np.tril((rng.random((nb, nb)) < 0.05).astype(np.uint8))
    np.fill_diagonal(m, 1)
    U.say(f"[max] sparse N={N} d={d} ({int(m.sum())} blocks on)")
    dev = U.to_dev(inp)
    bm = torch.from_numpy(m).cuda()
    o, lse = fa.fa_fwd_sparse(dev["q"], dev["k"], dev["v"], bm, causal=True, scale=w.scale)
    dq, dk, dv = fa.fa_bwd_sparse(dev["q"], dev["k"], dev["v"], o, dev["dout"], lse, bm,
                                  causal=True, scale=w.scale)
    torch.cuda.synchronize()
    q, k, v, do = (U.f64(inp, n)[0, 0] for n in ("q", "k", "v", "dout"))
    del inp, dev
    for r0 in (0, N // 2 + 7, N - ROWS):
        r1 = r0 + ROWS
        ro, rl, rdq, rdk, rdv = oracle.head_row_block_sparse(q, k, v, do, w.scale, True, None,
                                                             m, r0, r1, blk)
        U.compare(f"O rows {r0}+", o[0, 0, r0:r1], ro, "bf16")
        U.compare(f"LSE rows {r0}+", lse[0, 0, r0:r1], rl, "bf16")
        U.compare(f"dQ rows {r0}+", dq[0, 0, r0:r1], rdq, "bf16")
    U.compare("dK last keys", dk[0, 0, N - ROWS:], rdk[N - ROWS:], "bf16")
    U.compare("dV last keys", dv[0, 0, N - ROWS:], rdv[N - ROWS:], "bf16")
    sv = dv[0, 0].double().sum(dim=0).cpu().numpy()
    so = do.sum(axis=0)
    assert np.all(np.abs(sv - so) <= 1e-3 * np.abs(do).sum(axis=0))


def test_max_split_length():
    """Split-KV at N = 2^22 (one head, d = 128, causal, four key ranges of 2^20): the
    merge equals the unsplit forward, and the oracle's row blocks agree with it."""
    import io_aware_softmax_tiled_amd as fa
    w, inp = workloads.custom(1, 1, N_MAX, 128, "bf16", True, seed=4444, with_dout=False)
    U.say(f"[max] split-KV N={N_MAX} d=128, split_len 2^20")
    dev = U.to_dev(inp)
    o_p, l_p = fa.fa_fwd_partial(dev["q"], dev["k"], dev["v"], split_len=1 << 20, causal=True,
                                 scale=w.scale)
    o, lse = fa.fa_merge(o_p, l_p)
    del o_p, l_p
    o1, l1 = fa.fa_fwd(dev["q"], dev["k"], dev["v"], causal=True, scale=w.scale)
    torch.cuda.synchronize()
    assert (o - o1).abs().max().item() < 2e-3 and (lse - l1).abs().max().item() < 2e-3
    del o1, l1
    q, k, v = (U.f64(inp, n)[0, 0] for n in "qkv")
    z = np.broadcast_to(np.zeros(128), (N_MAX, 128))   # dO unused here
    for r0 in (0, (1 << 20) - 8, N_MAX - ROWS):   # the second block straddles a range end
        r1 = r0 + ROWS
        ro, rl, *_ = oracle.head_row_block(q, k, v, z, w.scale, True, None, r0, r1)
        U.compare(f"merged O rows {r0}+", o[0, 0, r0:r1], ro, "bf16")
        U.compare(f"merged LSE rows {r0}+", lse[0, 0, r0:r1], rl, "bf16")
