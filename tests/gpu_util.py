"""Helpers for the GPU parity tests: run the HIP path through the binding, run the oracle
on the same seeded inputs, and compare element by element in float64."""
from __future__ import annotations

import json
import os
import sys

import numpy as np
import pytest
import torch

import io_aware_softmax_tiled_amd as fa
import oracle
import workloads

# max-abs (and mean-abs) tolerances: 1e-5 for fp32 inputs; 2e-2 and 2e-3 for 16-bit inputs
TOL = {"f32": (1e-5, None), "bf16": (2e-2, 2e-3), "f16": (2e-2, 2e-3)}


def require_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU test needs a ROCm GPU (torch.cuda.is_available() is False)")
    fa.load_library()


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(inp):
    dev = {}
    for key in ("q", "k", "v", "dout"):
        dev[key] = None if inp[key] is None else inp[key].cuda()
    dev["kv_len"] = None if inp["kv_len"] is None else inp["kv_len"].cuda()
    return dev


def f64(inp, key):
    return workloads.as_f64(inp[key])


def kv_np(inp):
    return None if inp["kv_len"] is None else inp["kv_len"].numpy()


def gpu_fwd(inp, dev=None):
    dev = dev or to_dev(inp)
    o, lse = fa.fa_fwd(dev["q"], dev["k"], dev["v"], causal=inp["causal"],
                       scale=inp["scale"], kv_len=dev["kv_len"])
    torch.cuda.synchronize()
    return o, lse


def gpu_bwd(inp, dev=None):
    dev = dev or to_dev(inp)
    o, lse = fa.fa_fwd(dev["q"], dev["k"], dev["v"], causal=inp["causal"],
                       scale=inp["scale"], kv_len=dev["kv_len"])
    dq, dk, dv = fa.fa_bwd(dev["q"], dev["k"], dev["v"], o, dev["dout"], lse,
                           causal=inp["causal"], scale=inp["scale"], kv_len=dev["kv_len"])
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


def oracle_fwd(inp, heads=None, workers=None):
    q, k, v = f64(inp, "q"), f64(inp, "k"), f64(inp, "v")
    return oracle.attention_forward_heads(q, k, v, inp["scale"], inp["causal"], kv_np(inp),
                                          heads=heads, workers=workers)


def oracle_bwd(inp, heads=None, workers=None):
    q, k, v, do = f64(inp, "q"), f64(inp, "k"), f64(inp, "v"), f64(inp, "dout")
    return oracle.attention_backward_heads(q, k, v, do, inp["scale"], inp["causal"],
                                           kv_np(inp), heads=heads, workers=workers)


def compare(name, got, ref, dtype, report=None):
    """got: torch tensor (any device), ref: float64 numpy; asserts the tolerance."""
    g = got.detach().double().cpu().numpy()
    assert g.shape == ref.shape, (name, g.shape, ref.shape)
    assert np.isfinite(g).all(), f"{name}: non-finite values"
    diff = np.abs(g - ref)
    mx, mean = float(diff.max(initial=0.0)), float(diff.mean()) if diff.size else 0.0
    tmax, tmean = TOL[dtype]
    if report is not None:
        report[name] = (mx, mean)
    path = os.environ.get("FA_PARITY_REPORT")
    if path:  # one JSON line per comparison, for the record of achieved errors
        with open(path, "a") as f:
            f.write(json.dumps({"test": os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0],
                                "output": name, "dtype": dtype, "max_abs": mx,
                                "mean_abs": mean}) + "\n")
    assert mx <= tmax, f"{name}: max-abs error {mx:.3e} > {tmax:.1e} (mean {mean:.2e})"
    if tmean is not None:
        assert mean <= tmean, f"{name}: mean-abs error {mean:.3e} > {tmean:.1e}"
    return mx, mean


def sample_heads(B, H, n, seed=0):
    """n distinct (b, h) heads, always including the first and the last."""
    allh = [(b, h) for b in range(B) for h in range(H)]
    if n >= len(allh):
        return allh
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(1, len(allh) - 1), size=n - 2, replace=False)
    return [allh[0]] + [allh[i] for i in sorted(mid)] + [allh[-1]]
