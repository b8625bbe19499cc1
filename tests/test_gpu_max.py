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
