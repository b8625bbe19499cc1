"""Seeded synthetic inputs for exact attention, shared by the tests, the bench and the oracle checks.

This module only draws random numbers and casts them; it holds none of the attention
arithmetic. Both the GPU path and the CPU oracle receive bit-identical tensors from it:
the oracle sees the cast values upcast exactly to float64, the GPU the same bits.

Layout follows the [batch, heads, seq, head_dim] convention of the causal PyTorch
listing in "Fewer matrix multiplications, same results" (Dao-AILab/flash-attention
issue #941). Shapes borrow GPT-2-small and BERT-large attention, the workloads of the
results section of the FlashAttention paper summary (arXiv 2205.14135); the values are
i.i.d. standard normal because no dataset is used.

Draw order for every workload (one CPU generator, seed 0 unless stated): Q, K, V,
then dO when the backward pass is exercised, then the per-sequence key lengths when
key padding is used. Q is multiplied by a power of two (exact) where a workload asks
for peaky softmax rows. Casting to bf16/f16 rounds to nearest even.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
# dtype codes of the C ABI (include/fa.h)
DTYPE_CODES = {"f32": 0, "bf16": 1, "f16": 2}


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str
    B: int
    H: int
    N: int
    d: int
    causal: bool
    passes: tuple = ("fwd",)
    kv_range: tuple | None = None  # inclusive [lo, hi] for per-sequence key lengths
    q_mult: float = 1.0
    seed: int = 0
    note: str = field(default="", compare=False)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def has_bwd(self) -> bool:
        return "bwd" in self.passes

    def fwd_flops(self) -> float:
        """Nominal forward FLOPs: 4*B*H*N^2*d, halved when causal."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2 if self.causal else f

    def bwd_flops(self) -> float:
        """Nominal backward FLOPs: 2.5x the forward count."""
        return 2.5 * self.fwd_flops()


# The five workloads the build is measured and parity-checked on.
WORKLOADS = {
    1: Workload("f32_b1h1_n256_d64", "f32", 1, 1, 256, 64, False,
                note="forward only, fp32, non-causal, scale 1/8"),
    2: Workload("gpt2s_b4h12_n1024_d64_causal", "bf16", 4, 12, 1024, 64, True,
                note="forward only, GPT-2-small-shaped causal self-attention"),
    3: Workload("bertl_b8h16_n512_d64_keypad", "bf16", 8, 16, 512, 64, False,
                passes=("fwd", "bwd"), kv_range=(256, 512),
                note="forward+backward, BERT-large-shaped, per-sequence key padding"),
    4: Workload("b2h16_n4096_d128_causal_q4", "bf16", 2, 16, 4096, 128, True,
                passes=("fwd", "bwd"), q_mult=4.0,
                note="forward+backward, causal, Q scaled x4 for peaky rows"),
    5: Workload("b1h16_n16384_d64_causal", "bf16", 1, 16, 16384, 64, True,
                note="forward only, long-context causal"),
}


def draw(w: Workload, with_dout: bool | None = None) -> dict:
    """Draw the seeded inputs of workload ``w`` as CPU tensors.

    Returns a dict with q, k, v (dtype of the workload, shape [B,H,N,d]),
    dout (same, when the backward pass is drawn), kv_len (int32 [B] or None),
    scale, causal.
    """
    if with_dout is None:
        with_dout = w.has_bwd
    g = torch.Generator("cpu").manual_seed(w.seed)
    shape = (w.B, w.H, w.N, w.d)
    q = torch.randn(shape, dtype=torch.float32, generator=g)
    k = torch.randn(shape, dtype=torch.float32, generator=g)
    v = torch.randn(shape, dtype=torch.float32, generator=g)
    dout = torch.randn(shape, dtype=torch.float32, generator=g) if with_dout else None
    kv_len = None
    if w.kv_range is not None:
        lo, hi = w.kv_range
        kv_len = torch.randint(lo, hi + 1, (w.B,), generator=g).to(torch.int32)
    if w.q_mult != 1.0:
        q = q * w.q_mult
    dt = DTYPES[w.dtype]
    out = {
        "q": q.to(dt).contiguous(),
        "k": k.to(dt).contiguous(),
        "v": v.to(dt).contiguous(),
        "dout": dout.to(dt).contiguous() if dout is not None else None,
        "kv_len": kv_len,
        "scale": w.scale,
        "causal": w.causal,
    }
    return out


def custom(B, H, N, d, dtype="bf16", causal=False, kv_range=None, q_mult=1.0,
           seed=0, with_dout=True, name="custom") -> tuple:
    """A workload of arbitrary shape with the same draw recipe; returns (workload, inputs)."""
    w = Workload(name, dtype, B, H, N, d, causal,
                 passes=("fwd", "bwd") if with_dout else ("fwd",),
                 kv_range=kv_range, q_mult=q_mult, seed=seed)
    return w, draw(w, with_dout=with_dout)


def as_f64(t):
    """Exact upcast of a drawn tensor to a float64 numpy array (None passes through)."""
    if t is None:
        return None
    return t.to(torch.float64).numpy()
