"""fa_bwd_noalloc (the backward pass with the library's static per-GPU scratch instead
of a caller workspace) against fa_bwd, through the C ABI: two calls in a row, the second
on a smaller input, each bit-identical to fa_bwd on the same inputs (so within the
oracle tolerance wherever fa_bwd is), plus the host-side rejection of sizes beyond the
scratch."""
import ctypes

import pytest
import torch

import io_aware_softmax_tiled_amd as fa
import workloads
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    U.require_gpu()


def _noalloc_c(lib, dev, o, lse, dq, dk, dv, inp, dtype_code):
    B, H, N, d = (int(x) for x in dev["q"].shape)
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    st = lib.fa_bwd_noalloc(p(dev["q"]), p(dev["k"]), p(dev["v"]), p(o), p(dev["dout"]), p(lse),
                            p(dq), p(dk), p(dv), B, H, N, d, inp["scale"], int(inp["causal"]),
                            dtype_code, p(dev["kv_len"]),
                            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, fa.fa_last_error()


@pytest.mark.parametrize("second", [False, True])
def test_noalloc_matches_fa_bwd_twice(second):
    lib = fa.load_library()
    cases = [dict(B=2, H=4, N=1000, d=128, dtype="bf16", causal=True, kv=None, q_mult=4.0),
             dict(B=1, H=2, N=300, d=64, dtype="f16", causal=False, kv=(100, 300), q_mult=1.0)]
    for c in (cases if second else cases[:1]):
        w, inp = workloads.custom(c["B"], c["H"], c["N"], c["d"], c["dtype"], c["causal"],
                                  kv_range=c["kv"], q_mult=c["q_mult"], seed=c["N"])
        U.say(f"[noalloc] B={c['B']} H={c['H']} N={c['N']} d={c['d']} {c['dtype']}")
        dev = U.to_dev(inp)
        o, lse = fa.fa_fwd(dev["q"], dev["k"], dev["v"], causal=inp["causal"],
                           scale=inp["scale"], kv_len=dev["kv_len"])
        ref = fa.fa_bwd(dev["q"], dev["k"], dev["v"], o, dev["dout"], lse,
                        causal=inp["causal"], scale=inp["scale"], kv_len=dev["kv_len"])
        got = [torch.full_like(ref[0], float("nan")) for _ in range(3)]
        _noalloc_c(lib, dev, o, lse, *got, inp, workloads.DTYPE_CODES[c["dtype"]])
        torch.cuda.synchronize()
        for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
            assert torch.equal(g, r), name
        # the Python wrapper marshals the same call
        got2 = [torch.empty_like(ref[0]) for _ in range(3)]
        fa.fa_bwd_noalloc(dev["q"], dev["k"], dev["v"], o, dev["dout"], lse, *got2,
                          causal=inp["causal"], scale=inp["scale"], kv_len=dev["kv_len"])
        torch.cuda.synchronize()
        for g, r in zip(got2, ref):
            assert torch.equal(g, r)


def test_noalloc_rejects_oversized_problem_without_launching():
    lib = fa.load_library()
    q = torch.zeros((1, 1, 64, 64), dtype=torch.bfloat16, device="cuda")
    B, H, N, d = 64, 32, 8192, 64
    st = lib.fa_bwd_noalloc(*([ctypes.c_void_p(q.data_ptr())] * 9), B, H, N, d, 0.125, 0, 1,
                            None, None)
    assert st == 3 and "static scratch" in fa.fa_last_error()
