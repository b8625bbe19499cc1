"""The C ABI library on the CPU: it loads, exports every symbol include/fa.h declares,
and rejects invalid arguments on the host with the documented codes before touching the
GPU. No call here launches a kernel (no GPU is needed)."""
import ctypes
import os
import re
import subprocess

import pytest

import io_aware_softmax_tiled_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

FA_OK, FA_EINVAL, FA_EUNSUPPORTED, FA_EWORKSPACE, FA_EHIP = 0, 1, 2, 3, 4
P = 0x7f0000001000  # a 4 KiB-aligned fake device address: never dereferenced on error


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"FA_API\s+[\w\s\*]+?\b(fa_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.lib_path()):
        pytest.fail("libfa_mi355x.so is not built (python -m io_aware_softmax_tiled_amd.build)")
    return fa.load_library()


def test_header_declares_the_api():
    assert declared_symbols() == ["fa_bwd", "fa_bwd_dropout", "fa_bwd_noalloc", "fa_bwd_sparse",
                                  "fa_bwd_stage",
                                  "fa_bwd_workspace_size", "fa_dropout_threshold",
                                  "fa_fwd", "fa_fwd_auto", "fa_fwd_deferred", "fa_fwd_dropout", "fa_fwd_partial",
                                  "fa_fwd_sparse", "fa_fwd_workspace_size",
                                  "fa_last_error", "fa_merge", "fa_split_count", "fa_split_hint",
                                  "fa_status_str", "fa_version"]


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", fa.lib_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT\s+(\w+)", out))
    for name in declared_symbols():
        assert name in exported, f"{name} not exported"
        assert hasattr(lib, name)
    # nothing else with the public prefix leaks out
    assert {s for s in exported if s.startswith("fa_")} == set(declared_symbols())


def test_status_strings_and_version(lib):
    for code in range(5):
        assert fa.fa_status_str(code).startswith("FA_")
    assert fa.fa_status_str(99) == "unknown status"
    assert fa.fa_version() == 100
    assert fa.fa_last_error() == ""


def _fwd(lib, q=P, k=P + 0x100000, v=P + 0x200000, o=P + 0x300000, lse=P + 0x400000,
         B=1, H=1, N=64, d=64, scale=0.125, causal=0, dtype=1, kv=None):
    return lib.fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, kv, None)


def _bwd(lib, B=1, H=1, N=64, d=64, scale=0.125, dtype=1, ws=P + 0x900000, ws_bytes=None,
         **over):
    ptrs = dict(q=P, k=P + 0x100000, v=P + 0x200000, o=P + 0x300000, dout=P + 0x400000,
                lse=P + 0x500000, dq=P + 0x600000, dk=P + 0x700000, dv=P + 0x800000)
    ptrs.update(over)
    if ws_bytes is None:
        ws_bytes = lib.fa_bwd_workspace_size(B, H, N, d)
    return lib.fa_bwd(ptrs["q"], ptrs["k"], ptrs["v"], ptrs["o"], ptrs["dout"], ptrs["lse"],
                      ptrs["dq"], ptrs["dk"], ptrs["dv"], B, H, N, d, scale, 0, dtype, None,
                      ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), FA_EINVAL),
    (dict(lse=None), FA_EINVAL),
    (dict(d=96), FA_EUNSUPPORTED),
    (dict(d=32), FA_EUNSUPPORTED),
    (dict(dtype=7), FA_EUNSUPPORTED),
    (dict(N=-1), FA_EINVAL),
    (dict(B=-2), FA_EINVAL),
    (dict(scale=0.0), FA_EINVAL),
    (dict(scale=-1.0), FA_EINVAL),
    (dict(scale=float("inf")), FA_EINVAL),
    (dict(scale=float("nan")), FA_EINVAL),
    (dict(N=(1 << 22) + 1), FA_EINVAL),
    (dict(q=P + 8), FA_EINVAL),            # misaligned
    (dict(o=P + 4), FA_EINVAL),
    (dict(lse=P + 0x400002), FA_EINVAL),
    (dict(kv=P + 0x500002), FA_EINVAL),
    (dict(o=P), FA_EINVAL),                # output overlaps q
    (dict(lse=P + 0x300000 + 64), FA_EINVAL),  # lse inside o
])
def test_fwd_rejects_before_launch(lib, kw, code):
    assert _fwd(lib, **kw) == code
    assert fa.fa_last_error() != ""


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(N=0), dict(N=0, q=None)])
def test_fwd_empty_is_noop(lib, kw):
    assert _fwd(lib, **kw) == FA_OK


def test_workspace_size(lib):
    # D (one float per row) then the largest |dO| of each 32-row group, each region
    # rounded up to 256 bytes
    rnd = lambda x: (x + 255) // 256 * 256
    assert fa.fa_bwd_workspace_size(2, 3, 100, 64) == rnd(2 * 3 * 100 * 4) + rnd(2 * 3 * 4 * 4)
    assert fa.fa_bwd_workspace_size(0, 3, 100, 64) == 0
    assert fa.fa_bwd_workspace_size(8, 16, 512, 64) % 256 == 0


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=0, d=80), FA_EUNSUPPORTED),  # fp32 backward exists, head_dim 80 does not
    (dict(d=80), FA_EUNSUPPORTED),
    (dict(dq=None), FA_EINVAL),
    (dict(ws=None), FA_EWORKSPACE),
    (dict(ws_bytes=16), FA_EWORKSPACE),
    (dict(ws=P + 0x900000 + 16), FA_EINVAL),   # workspace not 256-aligned
    (dict(dk=P + 0x100000), FA_EINVAL),        # dk overlaps k
    (dict(dv=P + 0x600000), FA_EINVAL),        # dv overlaps dq
    (dict(lse=P + 0x500002), FA_EINVAL),
    (dict(scale=0.0), FA_EINVAL),
])
def test_bwd_rejects_before_launch(lib, kw, code):
    assert _bwd(lib, **kw) == code
    assert fa.fa_last_error() != ""


def test_bwd_empty_is_noop(lib):
    assert _bwd(lib, N=0) == FA_OK
    assert _bwd(lib, B=0, ws=None, ws_bytes=0) == FA_OK


def test_python_binding_requires_gpu_tensors():
    import torch
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.fa_fwd(q, q, q)


# ---- split-KV partials and merge -----------------------------------------------------

def test_split_count(lib):
    assert fa.fa_split_count(4096, 1024) == 4
    assert fa.fa_split_count(4097, 1024) == 5
    assert fa.fa_split_count(64, 4096) == 1
    assert fa.fa_split_count(0, 64) == 0
    assert fa.fa_split_count(100, 0) == -1
    assert fa.fa_split_count(100, 96) == -1      # not a multiple of 64
    assert fa.fa_split_count(100, -64) == -1


def _part(lib, q=P, k=P + 0x100000, v=P + 0x200000, o=P + 0x300000, lse=P + 0x700000,
          B=1, H=1, N=256, d=64, scale=0.125, causal=0, dtype=1, kv=None, split_len=64):
    return lib.fa_fwd_partial(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, kv,
                              split_len, None)


@pytest.mark.parametrize("kw,code", [
    (dict(split_len=0), FA_EINVAL),
    (dict(split_len=96), FA_EINVAL),
    (dict(split_len=-64), FA_EINVAL),
    (dict(dtype=0), FA_EUNSUPPORTED),      # no fp32 partials
    (dict(d=32), FA_EUNSUPPORTED),
    (dict(o=None), FA_EINVAL),
    (dict(o=P + 8), FA_EINVAL),
    (dict(lse=P + 0x700002), FA_EINVAL),
    (dict(o=P + 0x200000), FA_EINVAL),     # o_part overlaps v
    (dict(lse=P + 0x300000 + 4096), FA_EINVAL),  # lse_part inside o_part (4 splits)
    (dict(scale=float("nan")), FA_EINVAL),
])
def test_partial_rejects_before_launch(lib, kw, code):
    assert _part(lib, **kw) == code
    assert fa.fa_last_error() != ""


def test_partial_empty_is_noop(lib):
    assert _part(lib, N=0) == FA_OK
    assert _part(lib, B=0, q=None) == FA_OK


def _merge(lib, op=P, lp=P + 0x400000, o=P + 0x500000, lse=P + 0x600000, n=4, B=1, H=1,
           N=256, d=64):
    return lib.fa_merge(op, lp, o, lse, n, B, H, N, d, None)


@pytest.mark.parametrize("kw,code", [
    (dict(n=0), FA_EINVAL),
    (dict(n=65537), FA_EINVAL),
    (dict(d=96), FA_EUNSUPPORTED),
    (dict(N=-1), FA_EINVAL),
    (dict(op=None), FA_EINVAL),
    (dict(o=P + 8), FA_EINVAL),
    (dict(lse=P + 0x600002), FA_EINVAL),
    (dict(o=P + 0x1000), FA_EINVAL),       # o overlaps o_part
    (dict(lse=P + 0x500000 + 64), FA_EINVAL),  # lse inside o
])
def test_merge_rejects_before_launch(lib, kw, code):
    assert _merge(lib, **kw) == code
    assert fa.fa_last_error() != ""


def test_merge_empty_is_noop(lib):
    assert _merge(lib, N=0) == FA_OK


# ---- block-sparse --------------------------------------------------------------------

def _sfwd(lib, mask=P + 0x800000, N=256, dtype=1, **kw):
    args = dict(q=P, k=P + 0x100000, v=P + 0x200000, o=P + 0x300000, lse=P + 0x700000)
    args.update(kw)
    return lib.fa_fwd_sparse(args["q"], args["k"], args["v"], args["o"], args["lse"], 1, 1, N,
                             64, 0.125, 0, dtype, None, mask, None)


@pytest.mark.parametrize("kw,code", [
    (dict(mask=None), FA_EINVAL),
    (dict(dtype=0), FA_EUNSUPPORTED),
    (dict(N=(1 << 18) + 1), FA_EINVAL),
    (dict(mask=P + 0x300000 + 8), FA_EINVAL),   # o overlaps the mask
    (dict(q=None), FA_EINVAL),
])
def test_sparse_fwd_rejects_before_launch(lib, kw, code):
    assert _sfwd(lib, **kw) == code
    assert fa.fa_last_error() != ""


def test_sparse_bwd_rejects_before_launch(lib):
    args = [P, P + 0x100000, P + 0x200000, P + 0x300000, P + 0x400000, P + 0x500000,
            P + 0x600000, P + 0x700000, P + 0x800000, 1, 1, 256, 64, 0.125, 0, 1, None]
    ws = lib.fa_bwd_workspace_size(1, 1, 256, 64)
    assert lib.fa_bwd_sparse(*args, None, P + 0xa00000, ws, None) == FA_EINVAL
    assert lib.fa_bwd_sparse(*args[:15], 0, None, P + 0x900000, P + 0xa00000, ws,
                             None) == FA_EUNSUPPORTED
    assert lib.fa_bwd_sparse(*args, P + 0x900000, None, 0, None) == FA_EWORKSPACE
    assert lib.fa_bwd_sparse(*args, P + 0x600000 + 16, P + 0xa00000, ws, None) == FA_EINVAL


def test_sparse_empty_is_noop(lib):
    assert _sfwd(lib, N=0, mask=None) == FA_OK


def test_bwd_stage_rejects_before_launch(lib):
    args = [P, P + 0x100000, P + 0x200000, P + 0x300000, P + 0x400000, P + 0x500000,
            P + 0x600000, P + 0x700000, P + 0x800000, 1, 1, 64, 64, 0.125, 0, 1, None]
    ws = lib.fa_bwd_workspace_size(1, 1, 64, 64)
    for bad in (-1, 4, 7):
        assert lib.fa_bwd_stage(bad, *args, P + 0x900000, ws, None) == FA_EINVAL
    assert lib.fa_bwd_stage(1, *args, None, 0, None) == FA_EWORKSPACE
    args[15] = 0   # f32 (has a backward pass) with head_dim 80 (has none)
    args[12] = 80
    assert lib.fa_bwd_stage(0, *args, P + 0x900000, ws, None) == FA_EUNSUPPORTED


# ---- dropout -------------------------------------------------------------------------

def _dfwd(lib, p=0.1, N=256, dtype=1, q=P, seed=1, offset=0):
    return lib.fa_fwd_dropout(q, P + 0x100000, P + 0x200000, P + 0x300000, P + 0x700000, 1,
                              1, N, 64, 0.125, 0, dtype, None, p, seed, offset, None)


@pytest.mark.parametrize("kw,code", [
    (dict(p=-0.01), FA_EINVAL),
    (dict(p=1.0), FA_EINVAL),
    (dict(p=float("nan")), FA_EINVAL),
    (dict(p=float("inf")), FA_EINVAL),
    (dict(dtype=0), FA_EUNSUPPORTED),
    (dict(q=None), FA_EINVAL),
])
def test_dropout_fwd_rejects_before_launch(lib, kw, code):
    assert _dfwd(lib, **kw) == code
    assert fa.fa_last_error() != ""


def test_dropout_empty_is_noop(lib):
    assert _dfwd(lib, N=0, seed=(1 << 64) - 1, offset=(1 << 32) - 1) == FA_OK


def test_dropout_bwd_rejects_before_launch(lib):
    args = [P, P + 0x100000, P + 0x200000, P + 0x300000, P + 0x400000, P + 0x500000,
            P + 0x600000, P + 0x700000, P + 0x800000, 1, 1, 256, 64, 0.125, 0, 1, None]
    ws = lib.fa_bwd_workspace_size(1, 1, 256, 64)
    assert lib.fa_bwd_dropout(*args, 1.5, 1, 0, P + 0xa00000, ws, None) == FA_EINVAL
    assert lib.fa_bwd_dropout(*args, 0.1, 1, 0, None, 0, None) == FA_EWORKSPACE
    assert lib.fa_bwd_dropout(*args[:15], 0, None, 0.1, 1, 0, P + 0xa00000, ws,
                              None) == FA_EUNSUPPORTED
    assert lib.fa_bwd_dropout(*args[:15], 1, None, 0.1, 1, 0, P + 0x600000 + 16, ws,
                              None) == FA_EINVAL   # workspace overlaps dq


def test_dropout_binding_checks_key():
    import torch
    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    for seed, offset in ((-1, 0), (1 << 64, 0), (0, 1 << 32), (0, -1)):
        with pytest.raises(ValueError):
            fa.fa_fwd_dropout(q, q, q, p=0.1, seed=seed, offset=offset)


# ---- deferred P V --------------------------------------------------------------------

@pytest.mark.parametrize("N,dtype,q,code", [
    (513, 1, P, FA_EINVAL),
    (256, 0, P, FA_EUNSUPPORTED),
    (256, 1, None, FA_EINVAL),
    (0, 1, P, FA_OK),
])
def test_deferred_rejects_before_launch(lib, N, dtype, q, code):
    st = lib.fa_fwd_deferred(q, P + 0x100000, P + 0x200000, P + 0x300000, P + 0x700000, 1, 1,
                             N, 64, 0.125, 0, dtype, None, None)
    assert st == code


def test_dropout_threshold_matches_the_oracle(lib):
    """The library's byte threshold (what the kernels receive) equals the oracle's on a
    grid of p and on the float32 values around every halfway point 256 p = k + 1/2, and
    rejects p outside [0, 1)."""
    import numpy as np
    import oracle
    ps = [float(x) for x in np.linspace(0.0, 0.9999, 4001)]
    for k in range(256):
        mid = np.float32((k + 0.5) / 256)
        ps += [float(mid), float(np.nextafter(mid, np.float32(0))),
               float(np.nextafter(mid, np.float32(1)))]
    ps = [p for p in ps if float(np.float32(p)) < 1.0]
    for p in ps:
        assert fa.fa_dropout_threshold(p) == oracle.dropout_threshold(p), p
    for bad in (-1e-9, 1.0, 2.0, float("nan"), float("inf")):
        assert fa.fa_dropout_threshold(bad) == -1


def test_noalloc_rejects_sizes_beyond_its_scratch(lib):
    """fa_bwd_noalloc refuses, on the host, sizes whose scratch exceeds the static array
    (no GPU is touched), and validates like fa_bwd."""
    B, H, N, d = 64, 32, 8192, 64        # 16.8 M rows: beyond the 32 MiB scratch
    assert fa.fa_bwd_workspace_size(B, H, N, d) > fa.FA_NOALLOC_SCRATCH_BYTES
    st = lib.fa_bwd_noalloc(P, P + 0x100000, P + 0x200000, P + 0x300000, P + 0x400000,
                            P + 0x500000, P + 0x600000, P + 0x700000, P + 0x800000, B, H, N, d,
                            0.125, 0, 1, None, None)
    assert st == FA_EWORKSPACE and "static scratch" in fa.fa_last_error()
    st = lib.fa_bwd_noalloc(P, P + 0x100000, P + 0x200000, P + 0x300000, P + 0x400000,
                            P + 0x500000, P + 0x600000, P + 0x700000, P + 0x800000, 1, 1, 64, 96,
                            0.125, 0, 1, None, None)
    assert st == FA_EUNSUPPORTED
    assert lib.fa_bwd_noalloc(None, None, None, None, None, None, None, None, None, 0, 1, 64, 64,
                              0.125, 0, 1, None, None) == FA_OK
