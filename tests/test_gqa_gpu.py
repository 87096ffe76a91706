"""Grouped K/V heads (grouped-query and multi-query attention) on the GPU, through the
C-ABI library: parity with the fp64 oracle, and bit-identity with multi-head
attention on K/V whose heads are repeated for their groups (the kernels do the same
arithmetic per query head either way)."""

import numpy as np
import pytest
import torch

import exact_attention_prefill_amd as ea
import oracle
import workloads as W
from parity import TOL, check, f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

PREFILL_CASES = [
    # B, Hq, Hkv, N, d, dtype
    (2, 8, 2, 200, 64, "f16"),
    (1, 6, 3, 333, 128, "bf16"),
    (1, 4, 1, 129, 128, "f16"),
    (2, 12, 4, 65, 64, "bf16"),
    (1, 10, 5, 64, 128, "bf16"),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", PREFILL_CASES, ids=lambda c: "b{}_hq{}_hkv{}_n{}_d{}_{}".format(*c))
def test_prefill_gqa_parity(case, causal):
    B, Hq, Hkv, N, d, dtype = case
    q, k, v = W.prefill_inputs_gqa(B, Hq, Hkv, N, d, dtype, seed=N + Hq)
    out = ea.prefill(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, scale=1 / np.sqrt(d))
    torch.cuda.synchronize()
    ref = oracle.prefill(f64(q), f64(k), f64(v), causal, 1 / np.sqrt(d))
    check(f64(out), ref, dtype, f"prefill gqa {case} causal={causal}")


@pytest.mark.parametrize("d", [64, 128])
def test_prefill_gqa_equals_repeated_heads(d):
    B, Hq, Hkv, N = 2, 8, 2, 300
    q, k, v = (t.to(DEV) for t in W.prefill_inputs_gqa(B, Hq, Hkv, N, d, "bf16", seed=d))
    kr = k.repeat_interleave(Hq // Hkv, dim=1).contiguous()
    vr = v.repeat_interleave(Hq // Hkv, dim=1).contiguous()
    for causal in (False, True):
        a = ea.prefill(q, k, v, causal=causal, scale=0.09)
        b = ea.prefill(q, kr, vr, causal=causal, scale=0.09)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), causal


@pytest.mark.parametrize("causal", [False, True])
def test_prefill_gqa_eight_wave_form_sampled(causal):
    """32 query heads over 8 K/V heads at 8300 tokens: enough 256-row blocks, and long
    enough workgroups (causal too), for the eight-wave form, with a ragged last block."""
    B, Hq, Hkv, N, d = 1, 32, 8, 8300, 128
    scale = 1 / np.sqrt(d)
    q, k, v = W.prefill_inputs_gqa(B, Hq, Hkv, N, d, "bf16", seed=5)
    out = ea.prefill(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, scale=scale)
    torch.cuda.synchronize()
    rows = W.prefill_rows_sample(N, 40, seed=5)
    for h in (0, 3, 4, 31):
        ref = oracle.prefill_rows(f64(q[0:1]), f64(k[0:1]), f64(v[0:1]), causal, scale, 0, h, rows)
        check(f64(out[0, h, rows]), ref, "bf16", f"gqa eight-wave h={h}")
    assert torch.isfinite(out).all()


# Group sizes g = Hq / Hkv: 3..32 run on the matrix cores (one wave per K/V head);
# 2 and larger groups on the vector ALUs with the largest divisor of g up to 8 heads
# per wave (33 -> 3, 34 -> 2, 37 -> 1, 40 -> 8, 42 -> 7).
DECODE_GROUPS = [2, 3, 4, 5, 6, 7, 8, 11, 16, 31, 32, 33, 34, 37, 40, 42]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("g", DECODE_GROUPS)
def test_decode_gqa_parity(g, d, dtype):
    B, Hkv, max_len = 3, 2, 700
    lens = [700, 1, 333]
    q, kc, vc, lens = W.decode_inputs_gqa(B, g * Hkv, Hkv, max_len, d, dtype, seed=g, seq_lens=lens)
    scale = 1 / np.sqrt(d)
    out = ea.decode(q.to(DEV), kc.to(DEV), vc.to(DEV), lens.to(DEV), scale=scale)
    torch.cuda.synchronize()
    ref = oracle.decode(f64(q), f64(kc), f64(vc), lens.numpy(), scale)
    check(f64(out), ref, dtype, f"decode gqa g={g} d={d} {dtype}")


@pytest.mark.parametrize("g", [1, 2, 3, 4, 8, 16, 32, 40])
def test_decode_gqa_equals_repeated_heads(g):
    """Grouped decode equals multi-head decode on K/V whose heads are repeated for their
    groups.  Groups of 3..32 heads run on the matrix cores and multi-head decode on the
    vector ALUs, so the two agree within the gate of each other (and of the oracle);
    groups of one or two heads, and groups larger than 32 (vector ALUs, heads shared
    by a wave), do the same arithmetic per head and agree bit for bit."""
    B, Hkv, max_len, d = 4, 2, 1000, 128
    q, kc, vc, lens = (t.to(DEV) for t in W.decode_inputs_gqa(B, g * Hkv, Hkv, max_len, d, "bf16", seed=40 + g))
    kr = kc.repeat_interleave(g, dim=1).contiguous()
    vr = vc.repeat_interleave(g, dim=1).contiguous()
    # The same chunk for both (the automatic split differs: a grouped wave serves
    # several heads), so the partials and their merge cover the same rows.
    chunk = 128
    ws = torch.empty(ea.decode_workspace_bytes(B, g * Hkv, -(-max_len // chunk), d), dtype=torch.uint8, device=DEV)
    a = ea.decode(q, kc, vc, lens, scale=0.088, chunk=chunk, workspace=ws).clone()
    b = ea.decode(q, kr, vr, lens, scale=0.088, chunk=chunk, workspace=ws)
    torch.cuda.synchronize()
    if g < 3 or g > 32:
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    else:
        ref = oracle.decode(f64(q), f64(kc), f64(vc), lens.cpu().numpy(), 0.088)
        check(f64(a), ref, "bf16", f"grouped g={g}")
        check(f64(b), ref, "bf16", f"repeated g={g}")
        assert np.max(np.abs(f64(a) - f64(b))) <= TOL["bf16"]


def test_decode_gqa_chunks():
    B, Hq, Hkv, max_len, d = 2, 8, 2, 300, 64
    q, kc, vc, lens = W.decode_inputs_gqa(B, Hq, Hkv, max_len, d, "f16", 11, [300, 161])
    ref = oracle.decode(f64(q), f64(kc), f64(vc), lens.numpy(), 0.125)
    outs = []
    for chunk in range(32, 320 + 1, 32):
        n_split = -(-max_len // chunk)
        ws = torch.empty(ea.decode_workspace_bytes(B, Hq, n_split, d), dtype=torch.uint8, device=DEV)
        out = ea.decode(q.to(DEV), kc.to(DEV), vc.to(DEV), lens.to(DEV), scale=0.125, chunk=chunk, workspace=ws)
        torch.cuda.synchronize()
        out = f64(out)
        check(out, ref, "f16", f"gqa chunk={chunk}")
        outs.append(out)
    assert max(np.max(np.abs(o - outs[0])) for o in outs) <= TOL["f16"]


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("case", W.DECODE_GQA, ids=lambda c: c.name)
def test_decode_gqa_config(case, seed):
    Hkv = W.DECODE_GQA_HKV[case.name]
    q, kc, vc, lens = W.decode_inputs_gqa(case.B, case.H, Hkv, case.max_len, case.d, case.dtype, seed)
    out = ea.decode(q.to(DEV), kc.to(DEV), vc.to(DEV), lens.to(DEV), scale=case.scale)
    torch.cuda.synchronize()
    ref = oracle.decode(f64(q), f64(kc), f64(vc), lens.numpy(), case.scale)
    check(f64(out), ref, case.dtype, f"{case.name} seed={seed}")


def test_decode_gqa_zero_length_writes_zeros():
    q, kc, vc, _ = W.decode_inputs_gqa(2, 8, 1, 64, 64, "f16", 3, [1, 1])
    lens = torch.tensor([0, 64], dtype=torch.int32)
    out = f64(ea.decode(q.to(DEV), kc.to(DEV), vc.to(DEV), lens.to(DEV), scale=0.125))
    assert np.all(out[0] == 0)
    ref = oracle.decode(f64(q[1:2]), f64(kc[1:2]), f64(vc[1:2]), [64], 0.125)
    check(out[1:2], ref, "f16", "gqa length 64")


def test_gqa_python_errors():
    q = torch.zeros(1, 6, 8, 64, dtype=torch.float16, device=DEV)
    k = torch.zeros(1, 4, 8, 64, dtype=torch.float16, device=DEV)
    with pytest.raises(ValueError):
        ea.prefill(q, k, k.clone())


@pytest.mark.parametrize("max_len", [1, 5, 31, 32, 33, 64, 65])
@pytest.mark.parametrize("g", [4, 32])
def test_decode_gqa_short_caches(g, max_len):
    """Caches shorter than one 32-row tile, or one row past it, on the matrix-core path:
    partial tiles start from zeroed LDS and their missing rows weigh nothing."""
    B, Hkv = 3, 2
    lens = [max_len, 1, max(1, max_len // 2)]
    q, kc, vc, lens = W.decode_inputs_gqa(B, g * Hkv, Hkv, max_len, 128, "bf16", seed=max_len, seq_lens=lens)
    out = ea.decode(q.to(DEV), kc.to(DEV), vc.to(DEV), lens.to(DEV), scale=0.09)
    torch.cuda.synchronize()
    check(f64(out), oracle.decode(f64(q), f64(kc), f64(vc), lens.numpy(), 0.09), "bf16", f"short g={g} L={max_len}")
