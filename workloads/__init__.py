"""Seeded synthetic inputs for the attention forward (prefill and decode).

This module only draws random numbers and names shapes. It holds none of the
method's arithmetic, so both the CPU oracle's tests and the GPU path can take
their inputs from it without sharing any computation.

Recipe (the pages fix only "i.i.d. N(0,1) from seed"; the generator is our
reading): one ``torch.Generator('cpu')`` seeded with ``seed``.  Prefill draws
``randn(B, H, N, d)`` in float32 for q, then k, then v, and rounds each to the
storage dtype (round to nearest even).  Decode draws q ``(B, H, 1, d)``, then
the K cache, then the V cache ``(B, H, max_len, d)`` the same way, then the
per-sequence lengths ``randint(1, max_len + 1, (B,))``; a batch of one takes
the full ``max_len`` without a draw.

Shapes follow the workloads the pages describe: a GPT-2-sized prompt (12 heads
of 64), dense d=128 prefill at 4K/8K/16K tokens (the B200 comparison on
page 1), a ragged decode batch over a 4096-row cache (page 3, "What can it
do"), and a long video-generation-like sequence.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import torch

DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class PrefillCase:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str
    causal: bool
    scale: float

    @property
    def flop(self) -> float:
        """Algorithmic flop: 4*B*H*N*N*d, exactly halved when causal."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2 if self.causal else f


@dataclass(frozen=True)
class DecodeCase:
    name: str
    B: int
    H: int
    max_len: int
    d: int
    dtype: str
    scale: float


def prefill_inputs(B, H, N, d, dtype="f16", seed=0):
    """q, k, v as CPU tensors of the storage dtype, shape (B, H, N, d)."""
    g = torch.Generator("cpu").manual_seed(seed)
    tdt = DTYPES[dtype]
    q = torch.randn(B, H, N, d, generator=g, dtype=torch.float32).to(tdt)
    k = torch.randn(B, H, N, d, generator=g, dtype=torch.float32).to(tdt)
    v = torch.randn(B, H, N, d, generator=g, dtype=torch.float32).to(tdt)
    return q, k, v


def decode_inputs(B, H, max_len, d, dtype="f16", seed=0, seq_lens=None):
    """q (B,H,1,d), k_cache, v_cache (B,H,max_len,d), seq_lens int32 (B,), all CPU.

    ``seq_lens`` may be given explicitly (edge-case tests); otherwise it is drawn
    after the three tensors, uniform in [1, max_len], and fixed at max_len when B == 1.
    """
    g = torch.Generator("cpu").manual_seed(seed)
    tdt = DTYPES[dtype]
    q = torch.randn(B, H, 1, d, generator=g, dtype=torch.float32).to(tdt)
    kc = torch.randn(B, H, max_len, d, generator=g, dtype=torch.float32).to(tdt)
    vc = torch.randn(B, H, max_len, d, generator=g, dtype=torch.float32).to(tdt)
    if seq_lens is None:
        if B == 1:
            lens = torch.full((1,), max_len, dtype=torch.int64)
        else:
            lens = torch.randint(1, max_len + 1, (B,), generator=g)
    else:
        lens = torch.as_tensor(seq_lens, dtype=torch.int64)
    return q, kc, vc, lens.to(torch.int32)


def prefill_inputs_gqa(B, Hq, Hkv, N, d, dtype="f16", seed=0):
    """Grouped heads: q (B, Hq, N, d), k and v (B, Hkv, N, d), drawn q, k, v in order."""
    g = torch.Generator("cpu").manual_seed(seed)
    tdt = DTYPES[dtype]
    q = torch.randn(B, Hq, N, d, generator=g, dtype=torch.float32).to(tdt)
    k = torch.randn(B, Hkv, N, d, generator=g, dtype=torch.float32).to(tdt)
    v = torch.randn(B, Hkv, N, d, generator=g, dtype=torch.float32).to(tdt)
    return q, k, v


def decode_inputs_gqa(B, Hq, Hkv, max_len, d, dtype="f16", seed=0, seq_lens=None):
    """Grouped heads: q (B, Hq, 1, d), caches (B, Hkv, max_len, d), lengths as in decode_inputs."""
    g = torch.Generator("cpu").manual_seed(seed)
    tdt = DTYPES[dtype]
    q = torch.randn(B, Hq, 1, d, generator=g, dtype=torch.float32).to(tdt)
    kc = torch.randn(B, Hkv, max_len, d, generator=g, dtype=torch.float32).to(tdt)
    vc = torch.randn(B, Hkv, max_len, d, generator=g, dtype=torch.float32).to(tdt)
    if seq_lens is None:
        if B == 1:
            lens = torch.full((1,), max_len, dtype=torch.int64)
        else:
            lens = torch.randint(1, max_len + 1, (B,), generator=g)
    else:
        lens = torch.as_tensor(seq_lens, dtype=torch.int64)
    return q, kc, vc, lens.to(torch.int32)


def prefill_rows_sample(N, count, seed=0, include_edges=True):
    """Row indices for sampled parity at full size: edges plus a seeded spread."""
    g = torch.Generator("cpu").manual_seed(10_000 + seed)
    rows = set(torch.randint(0, N, (count,), generator=g).tolist())
    if include_edges:
        rows.update({0, 1, min(63, N - 1), min(64, N - 1), N // 2, N - 2 if N > 1 else 0, N - 1})
    return sorted(r for r in rows if 0 <= r < N)


# The workloads, named by what they are.
SMALL_F16 = [
    PrefillCase("prefill_b1_h1_n128_d64_f16_full", 1, 1, 128, 64, "f16", False, 0.125),
    PrefillCase("prefill_b1_h1_n128_d64_f16_causal", 1, 1, 128, 64, "f16", True, 0.125),
]
GPT2_F16 = [
    PrefillCase("prefill_gpt2_b1_h12_n2048_d64_f16_full", 1, 12, 2048, 64, "f16", False, 0.125),
    PrefillCase("prefill_gpt2_b1_h12_n2048_d64_f16_causal", 1, 12, 2048, 64, "f16", True, 0.125),
]
GPT2_SWEEP = [
    PrefillCase(f"prefill_gpt2_b{B}_h12_n{N}_d64_f16_{'causal' if c else 'full'}", B, 12, N, 64, "f16", c, 0.125)
    for B in (1, 4) for N in (128, 512, 1024, 4096) for c in (False, True)
]
DENSE_D128 = [
    PrefillCase(f"prefill_dense_b{B}_h16_n{N}_d128_bf16_full", B, 16, N, 128, "bf16", False, 1 / math.sqrt(128))
    for (B, N) in ((4, 4096), (2, 8192), (1, 16384))
]
HEADLINE = DENSE_D128[2]  # B=1, H=16, N=16384, d=128, bf16, non-causal
LONG = [
    PrefillCase("prefill_long_b1_h24_n32768_d128_bf16_full", 1, 24, 32768, 128, "bf16", False, 1 / math.sqrt(128)),
    PrefillCase("prefill_long_b1_h24_n16384_d128_bf16_causal", 1, 24, 16384, 128, "bf16", True, 1 / math.sqrt(128)),
]
DECODE = [
    DecodeCase("decode_b1_h12_len4096_d64_f16", 1, 12, 4096, 64, "f16", 0.125),
    DecodeCase("decode_b8_h12_len4096_d64_f16_ragged", 8, 12, 4096, 64, "f16", 0.125),
]


# Grouped-head decode shaped like a Llama-3-8B layer (32 query heads over 8 K/V heads
# of 128): a ragged batch of 8 over a 4096-row cache.
DECODE_GQA = [
    DecodeCase("decode_gqa_b8_hq32_hkv8_len4096_d128_bf16_ragged", 8, 32, 4096, 128, "bf16", 1 / math.sqrt(128)),
]
DECODE_GQA_HKV = {DECODE_GQA[0].name: 8}


def decode_bytes(H, d, seq_lens, elem_bytes=2, Hkv=None):
    """Algorithmic decode bytes: K and V rows actually read (once per K/V head), plus
    q in and out (once per query head)."""
    B = len(seq_lens)
    Hkv = H if Hkv is None else Hkv
    return sum(2 * Hkv * int(L) * d * elem_bytes for L in seq_lens) + 2 * B * H * d * elem_bytes
