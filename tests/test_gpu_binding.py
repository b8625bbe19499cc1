"""The binding refuses mismatched caller-supplied buffers for GPU inputs too: each case
raises before any kernel is launched."""
import pytest
import torch

import io_aware_softmax_tiled_amd as fa
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    U.require_gpu()


def _qkv():
    q = torch.zeros((1, 2, 64, 64), dtype=torch.bfloat16, device="cuda")
    return q, q.clone(), q.clone()


@pytest.mark.parametrize("kw", [
    dict(out=torch.empty((1, 2, 64, 32))),
    dict(out="dev_wrong_shape"),
    dict(out="dev_bf16"),
    dict(lse="dev_wrong_lse"),
])
def test_fwd_rejects_bad_outputs(kw):
    q, k, v = _qkv()
    bad = {"dev_wrong_shape": torch.empty((1, 2, 63, 64), device="cuda"),
           "dev_bf16": torch.empty((1, 2, 64, 64), dtype=torch.bfloat16, device="cuda"),
           "dev_wrong_lse": torch.empty((1, 2, 65), device="cuda")}
    kw = {n: bad.get(x, x) if isinstance(x, str) else x for n, x in kw.items()}
    with pytest.raises(ValueError):
        fa.fa_fwd(q, k, v, **kw)


def test_bwd_and_stage_reject_bad_buffers():
    q, k, v = _qkv()
    o, lse = fa.fa_fwd(q, k, v)
    with pytest.raises(ValueError, match="lse"):
        fa.fa_bwd(q, k, v, o, q, lse[..., :-1])
    with pytest.raises(ValueError, match="o must"):
        fa.fa_bwd(q, k, v, o.cpu(), q, lse)
    dq = torch.empty((1, 2, 64, 64), device="cuda")
    ws = torch.empty(fa.fa_bwd_workspace_size(1, 2, 64, 64), dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError, match="dk"):
        fa.fa_bwd_stage(3, q, k, v, o, q, lse, dq, dq.half(), dq.clone(), ws)
    with pytest.raises(ValueError, match="workspace"):
        fa.fa_bwd_stage(3, q, k, v, o, q, lse, dq, dq.clone(), dq.clone(), ws[:-1])
    torch.cuda.synchronize()
