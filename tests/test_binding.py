"""The Python binding's argument checks, on the CPU: every caller-supplied buffer is
compared with what the kernels will read or write through its pointer (shape, dtype,
device, contiguity) before anything reaches the library, and inputs that are not GPU
tensors are refused. No kernel runs here."""
import pytest
import torch

import io_aware_softmax_tiled_amd as fa

CPU = torch.device("cpu")


def test_short_names_are_the_entry_points():
    assert fa.fwd is fa.fa_fwd and fa.bwd is fa.fa_bwd
    assert "fwd" in fa.__all__ and "bwd" in fa.__all__


def test_expect_accepts_a_matching_buffer():
    t = torch.empty((2, 3, 5, 64), dtype=torch.float32)
    assert fa._expect(t, "out", (2, 3, 5, 64), torch.float32, CPU) is t


@pytest.mark.parametrize("make,msg", [
    (lambda: torch.empty((2, 3, 5, 63)), "shape"),
    (lambda: torch.empty((2, 3, 5)), "shape"),
    (lambda: torch.empty((2, 3, 5, 64), dtype=torch.float64), "float32"),
    (lambda: torch.empty((2, 3, 5, 64), dtype=torch.bfloat16), "float32"),
    (lambda: torch.empty((2, 3, 64, 5)).transpose(2, 3), "contiguous"),
    (lambda: torch.empty((2, 3, 5, 64), device="meta"), "on cpu"),
    (lambda: [[0.0]], "torch.Tensor"),
])
def test_expect_rejects_mismatches(make, msg):
    with pytest.raises((ValueError, TypeError), match=msg):
        fa._expect(make(), "out", (2, 3, 5, 64), torch.float32, CPU)


def test_workspace_size_and_placement(monkeypatch):
    monkeypatch.setattr(fa, "fa_bwd_workspace_size", lambda B, H, N, d: 4 * B * H * N)
    ok = torch.empty(4 * 2 * 3 * 5, dtype=torch.uint8)
    assert fa._workspace(ok, 2, 3, 5, 64, CPU) is ok
    with pytest.raises(ValueError, match="needs 120 bytes"):
        fa._workspace(torch.empty(119, dtype=torch.uint8), 2, 3, 5, 64, CPU)
    with pytest.raises(ValueError, match="contiguous"):
        fa._workspace(torch.empty(240, dtype=torch.uint8)[::2], 2, 3, 5, 64, CPU)
    assert fa._workspace(None, 2, 3, 5, 64, CPU).numel() == 120


def test_grad_inputs_checked():
    q = torch.empty((1, 2, 8, 64), dtype=torch.bfloat16)
    o = torch.empty((1, 2, 8, 64))
    lse = torch.empty((1, 2, 8))
    fa._grad_inputs(q, o, q.clone(), lse)
    with pytest.raises(ValueError, match="lse"):
        fa._grad_inputs(q, o, q.clone(), torch.empty((1, 2, 9)))
    with pytest.raises(ValueError, match="o must"):
        fa._grad_inputs(q, o.to(torch.bfloat16), q.clone(), lse)
    with pytest.raises(ValueError, match="dout"):
        fa._grad_inputs(q, o, q.float(), lse)


@pytest.mark.parametrize("call", ["fwd", "bwd", "fwd_partial", "fwd_sparse", "fwd_dropout",
                                  "fwd_deferred"])
def test_cpu_inputs_are_refused_before_the_library(call):
    q = torch.zeros((1, 1, 8, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensors"):
        if call == "fwd":
            fa.fa_fwd(q, q, q)
        elif call == "bwd":
            fa.fa_bwd(q, q, q, q.float(), q, torch.zeros((1, 1, 8)))
        elif call == "fwd_partial":
            fa.fa_fwd_partial(q, q, q, split_len=64)
        elif call == "fwd_sparse":
            fa.fa_fwd_sparse(q, q, q, torch.ones((1, 1), dtype=torch.uint8))
        elif call == "fwd_dropout":
            fa.fa_fwd_dropout(q, q, q, p=0.1, seed=1)
        else:
            fa.fa_fwd_deferred(q, q, q)


# (B, H, N, d, causal) -> split_len on a 256-compute-unit device (the CPU run assumes
# 256 when no device is visible; the MI355X has 256)
SPLIT_HINTS = [
    ((1, 4, 8192, 128, False), 4096),   # 128 query-block workgroups: two splits
    ((1, 4, 8192, 128, True), 2048),    # causal, 128 workgroups: four splits
    ((1, 8, 4096, 128, True), 1024),    # four splits of 1024 keys
    ((1, 16, 2048, 128, False), 0),     # two splits would hold 1024 keys: below 2048
    ((1, 8, 4096, 128, False), 2048),   # two splits of 2048 keys
    ((1, 2, 2048, 128, True), 1024),    # causal: four would be 512 keys, two hold 1024
    ((1, 4, 16384, 64, True), 4096),    # 256 causal workgroups: four splits
    ((1, 4, 16384, 64, False), 0),      # 256 workgroups without the mask: unsplit
    ((1, 8, 8192, 128, False), 0),      # one workgroup per compute unit: unsplit
    ((1, 16, 8192, 128, True), 0),      # 512 causal workgroups: unsplit
    ((2, 16, 4096, 128, True), 0),      # the benchmarked shape: unsplit
    ((4, 12, 1024, 64, True), 0),       # N < 2048: unsplit
]


@pytest.mark.parametrize("shape,expect", SPLIT_HINTS)
def test_split_hint_rule(shape, expect):
    B, H, N, d, causal = shape
    h = fa.fa_split_hint(B, H, N, d, causal=causal)
    assert h == expect
    if h:
        assert h % 64 == 0 and h >= (1024 if causal else 2048)
        assert fa.fa_split_count(N, h) in (2, 4)


def test_split_hint_f32_and_rejections():
    assert fa.fa_split_hint(1, 4, 8192, 128, dtype=torch.float32) == 0
    with pytest.raises(fa.FaError, match="head_dim 96"):
        fa.fa_split_hint(1, 4, 8192, 96)
    assert fa.fa_split_hint(0, 4, 8192, 128) == 0  # empty problem: nothing to split
    with pytest.raises(fa.FaError):
        fa.fa_split_hint(-1, 4, 8192, 128)


def test_fwd_workspace_size_follows_the_split():
    """The split's partials: n_splits * B*H*N*d floats (256-byte aligned) + n_splits *
    B*H*N floats; 0 where no split pays or the arguments are invalid."""
    B, H, N, d = 1, 4, 8192, 128
    for causal, P in ((False, 2), (True, 4)):
        rows = B * H * N
        assert fa.fa_fwd_workspace_size(B, H, N, d, causal=causal) == \
            (P * rows * d * 4 + 255) // 256 * 256 + P * rows * 4
    assert fa.fa_fwd_workspace_size(2, 16, 4096, 128, causal=True) == 0
    assert fa.fa_fwd_workspace_size(1, 4, 8192, 128, dtype=torch.float32) == 0
    assert fa.fa_fwd_workspace_size(1, 4, 8192, 96) == 0
