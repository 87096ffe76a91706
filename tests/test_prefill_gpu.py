"""Prefill on the GPU against the fp64 oracle, through the C-ABI library."""

import numpy as np
import pytest
import torch

import exact_attention_prefill_amd as ea
import oracle
import workloads as W
from parity import check, f64, plan_form, same_rows

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run(q, k, v, causal, scale):
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    out = ea.prefill(qd, kd, vd, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return out


def full_parity(B, H, N, d, dtype, causal, scale, seed):
    q, k, v = W.prefill_inputs(B, H, N, d, dtype, seed)
    out = run(q, k, v, causal, scale)
    ref = oracle.prefill(f64(q), f64(k), f64(v), causal, scale)
    return check(f64(out), ref, dtype, f"B{B} H{H} N{N} d{d} {dtype} causal={causal} seed={seed}")


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("case", W.SMALL_F16, ids=lambda c: c.name)
def test_small_config(case, seed):
    full_parity(case.B, case.H, case.N, case.d, case.dtype, case.causal, case.scale, seed)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [64, 96, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 17, 63, 64, 65, 127, 128, 129, 200, 333])
def test_ragged_lengths(N, causal, d, dtype):
    scale = 1.0 / np.sqrt(d)
    full_parity(2, 3, N, d, dtype, causal, scale, seed=N)


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("case", W.GPT2_F16, ids=lambda c: c.name)
def test_gpt2_config(case, seed):
    full_parity(case.B, case.H, case.N, case.d, case.dtype, case.causal, case.scale, seed=seed)


@pytest.mark.parametrize("case", [c for c in W.GPT2_SWEEP if c.N <= 1024], ids=lambda c: c.name)
def test_gpt2_sweep(case):
    full_parity(case.B, case.H, case.N, case.d, case.dtype, case.causal, case.scale, seed=1)


def sampled_parity(case, seed, heads, nrows, early=0):
    """Sampled rows (plus rows 1..early) of the given heads against the row oracle."""
    q, k, v = W.prefill_inputs(case.B, case.H, case.N, case.d, case.dtype, seed)
    out = run(q, k, v, case.causal, case.scale)
    worst = 0.0
    rows = sorted(set(W.prefill_rows_sample(case.N, nrows, seed)) | set(range(1, min(case.N, early + 1))))
    for (b, h) in heads:
        # widen only the sampled head to fp64; the oracle reads just these rows of q
        ref = oracle.prefill_rows(f64(q[b, h])[None, None], f64(k[b, h])[None, None], f64(v[b, h])[None, None],
                                  case.causal, case.scale, 0, 0, rows)
        got = f64(out[b, h, rows])
        worst = max(worst, check(got, ref, case.dtype, f"{case.name} seed={seed} b={b} h={h}"))
    assert torch.isfinite(out).all()
    return worst


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("case", W.DENSE_D128, ids=lambda c: c.name)
def test_dense_d128_sampled(case, seed):
    heads = [(0, 0), (case.B - 1, case.H - 1), (case.B // 2, 7)]
    sampled_parity(case, seed, heads, nrows=48)


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("case", W.LONG, ids=lambda c: c.name)
def test_long_sampled(case, seed):
    """The long sequences (B=1, H=24, d=128, bf16: N=32768 full, N=16384 causal) at the
    gate's three seeds.  Causal rows 1..16 average only a handful of values and carry
    the thinnest bf16 margin, so they are always in the sample."""
    heads = [(0, 0), (0, 23), (0, 11)]
    sampled_parity(case, seed, heads, nrows=32, early=16)


@pytest.mark.parametrize("case", [c for c in W.GPT2_SWEEP if c.N == 4096], ids=lambda c: c.name)
def test_gpt2_sweep_4096_sampled(case):
    heads = [(0, 0), (case.B - 1, case.H - 1)]
    sampled_parity(case, 2, heads, nrows=64)


# Grids of at least four 256-row blocks per CU (full: two) take the eight-wave workgroups unless
# the workgroups are short (full: N <= 2048, d = 64: 4096; causal: N <= 8192, d = 96:
# 6144, d = 64: 12288), which keep the four-wave form; these shapes reach both with a
# ragged last block (N not a multiple of 256): the d = 128 causal N = 8300 and
# d = 96 causal N = 7937 cases and the d = 128 full ones (H = 9 at N = 16001: two to
# four blocks per CU) the eight-wave form, the others the four-wave form on a large
# grid.
LARGE_RAGGED = [
    W.PrefillCase("prefill_b1_h9_n16001_d128_bf16_full", 1, 9, 16001, 128, "bf16", False, 1 / np.sqrt(128)),
    W.PrefillCase("prefill_b1_h32_n8300_d128_bf16_causal", 1, 32, 8300, 128, "bf16", True, 1 / np.sqrt(128)),
    W.PrefillCase("prefill_b1_h32_n8000_d128_bf16_causal", 1, 32, 8000, 128, "bf16", True, 1 / np.sqrt(128)),
    W.PrefillCase("prefill_b2_h16_n7937_d96_f16_causal", 2, 16, 7937, 96, "f16", True, 1 / np.sqrt(96)),
    W.PrefillCase("prefill_b1_h64_n4000_d128_bf16_full", 1, 64, 4000, 128, "bf16", False, 1 / np.sqrt(128)),
    W.PrefillCase("prefill_b1_h64_n4000_d128_bf16_causal", 1, 64, 4000, 128, "bf16", True, 1 / np.sqrt(128)),
    W.PrefillCase("prefill_b2_h32_n4001_d64_f16_causal", 2, 32, 4001, 64, "f16", True, 0.125),
    W.PrefillCase("prefill_b2_h32_n4001_d64_f16_full", 2, 32, 4001, 64, "f16", False, 0.125),
]


@pytest.mark.parametrize("case", LARGE_RAGGED, ids=lambda c: c.name)
def test_large_grid_ragged_sampled(case):
    heads = [(0, 0), (case.B - 1, case.H - 1), (0, case.H // 2)]
    sampled_parity(case, 3, heads, nrows=48)


@pytest.mark.parametrize("scale", [0.0, -0.3, 1.0, 1e-3])
@pytest.mark.parametrize("causal", [False, True])
def test_scale_values(scale, causal):
    full_parity(1, 2, 150, 64, "f16", causal, scale, seed=5)
    full_parity(1, 2, 150, 128, "bf16", causal, scale, seed=6)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [64, 96, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_growing_scores_raise_the_running_max(causal, d, dtype):
    """Key magnitudes that grow along the sequence push each row's maximum up again
    and again, well past the 2^8 margin the optimistic softmax keeps, so the rescale
    path runs many times per row."""
    B, H, N = 1, 3, 700
    q, k, v = W.prefill_inputs(B, H, N, d, dtype, 21)
    growth = (1.0 + 6.0 * torch.arange(N, dtype=torch.float32) / N).view(1, 1, N, 1)
    k = (k.float() * growth).to(k.dtype)
    scale = 2.0 / np.sqrt(d)
    out = run(q, k, v, causal, scale)
    ref = oracle.prefill(f64(q), f64(k), f64(v), causal, scale)
    check(f64(out), ref, dtype, f"growing scores d{d} {dtype} causal={causal}")


@pytest.mark.parametrize("d,dtype,causal,nh", [(128, "bf16", False, 4), (128, "f16", True, 4), (96, "bf16", True, 4),
                                                (128, "bf16", True, 8), (96, "f16", True, 8), (64, "bf16", False, 4),
                                                (64, "bf16", False, 8), (32, "f16", False, 4), (32, "f16", False, 8),
                                                (32, "bf16", True, 8)])
def test_small_grid_forms_match_large_grid(d, dtype, causal, nh):
    """nh heads of 8001 rows (63 128-row blocks a head) are a small grid: at most one
    block per CU splits each block's keys between the waves of eight-wave workgroups (key
    groups); one to two per CU keeps four K/V tiles in LDS (loads two tiles ahead; full
    grids at d <= 64, causal grids at every head size).  The 16-head call takes another
    form (two stages, or eight waves).  The nh heads must equal the same heads of the
    16-head call bit for bit when both forms have one key group (a row's arithmetic
    does not depend on such a form), within the gate otherwise; sampled rows are
    checked against the oracle."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    N = 8001
    small_form = plan_form(1, nh, N, d, causal, cus)
    big_form = plan_form(1, 16, N, d, causal, cus)
    assert small_form != big_form and big_form[3] == 1
    assert small_form[2] == 4 or small_form[3] > 1, small_form
    q, k, v = W.prefill_inputs(1, 16, N, d, dtype, 31)
    scale = 1.0 / np.sqrt(d)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    big = ea.prefill(qd, kd, vd, causal=causal, scale=scale)
    sl = slice(4, 4 + nh)
    small = ea.prefill(qd[:, sl].contiguous(), kd[:, sl].contiguous(), vd[:, sl].contiguous(), causal=causal,
                       scale=scale)
    torch.cuda.synchronize()
    for j in range(nh):
        same_rows(small[0, j], big[0, 4 + j], small_form, big_form, dtype, f"d{d} causal={causal} nh={nh} head {4 + j}")
    rows = W.prefill_rows_sample(N, 24, seed=31)
    for h in (4, 3 + nh):
        ref = oracle.prefill_rows(f64(q), f64(k), f64(v), causal, scale, 0, h, rows)
        check(f64(big[0, h, rows]), ref, dtype, f"large grid d{d} h={h} causal={causal}")
        check(f64(small[0, h - 4, rows]), ref, dtype, f"small grid d{d} h={h} causal={causal}")


def test_zero_query_gives_mean():
    q, k, v = W.prefill_inputs(1, 2, 300, 128, "bf16", 3)
    q = torch.zeros_like(q)
    out = f64(run(q, k, v, False, 0.1))
    ref = f64(v).mean(axis=2, keepdims=True) * np.ones_like(out)
    check(out, ref, "bf16", "Q=0 mean")
    outc = f64(run(q, k, v, True, 0.1))
    refc = np.cumsum(f64(v), axis=2) / np.arange(1, 301)[None, None, :, None]
    check(outc, refc, "bf16", "Q=0 prefix mean")


def test_deterministic():
    q, k, v = W.prefill_inputs(2, 4, 1000, 128, "bf16", 9)
    a = run(q, k, v, True, 0.088)
    b = run(q, k, v, True, 0.088)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("d", [64, 128])
def test_causality_bit_identical(d):
    """Rows 0..i are bit-identical when K/V rows after i change: the masked and
    skipped tiles contribute exactly nothing."""
    N, i = 700, 300
    q, k, v = W.prefill_inputs(1, 2, N, d, "f16", 4)
    a = run(q, k, v, True, 0.125)
    k2, v2 = k.clone(), v.clone()
    k2[:, :, i + 1:] = torch.randn(k2[:, :, i + 1:].shape).to(k2.dtype) * 3
    v2[:, :, i + 1:] = 100.0
    b = run(q, k2, v2, True, 0.125)
    assert torch.equal(a[:, :, : i + 1].view(torch.int16), b[:, :, : i + 1].view(torch.int16))


def test_output_canaries_and_nan_prefill():
    B, H, N, d = 1, 3, 257, 128
    q, k, v = (t.to(DEV) for t in W.prefill_inputs(B, H, N, d, "bf16", 8))
    n = B * H * N * d
    guard = 4096
    buf = torch.full((n + 2 * guard,), float("nan"), dtype=torch.bfloat16, device=DEV)
    canary = torch.full((guard,), 12.5, dtype=torch.bfloat16, device=DEV)
    buf[:guard] = canary
    buf[-guard:] = canary
    out = buf[guard:guard + n].view(B, H, N, d)
    ea.prefill(q, k, v, causal=False, scale=0.0884, out=out)
    torch.cuda.synchronize()
    assert torch.equal(buf[:guard], canary) and torch.equal(buf[-guard:], canary)
    assert torch.isfinite(out).all()


def test_last_causal_row_matches_full():
    q, k, v = W.prefill_inputs(1, 4, 999, 64, "f16", 10)
    a = f64(run(q, k, v, False, 0.125))
    b = f64(run(q, k, v, True, 0.125))
    assert np.max(np.abs(a[:, :, -1] - b[:, :, -1])) <= 2e-3


def test_python_errors():
    q = torch.zeros(1, 1, 8, 80, dtype=torch.float16, device=DEV)
    with pytest.raises(ValueError):
        ea.prefill(q, q.clone(), q.clone())
    q = torch.zeros(1, 1, 8, 64, dtype=torch.float32, device=DEV)
    with pytest.raises(ValueError):
        ea.prefill(q, q.clone(), q.clone())


@pytest.mark.parametrize("causal", [False, True])
def test_many_short_sequences(causal):
    """A large batch of short sequences (32 x 8 heads x 65 rows): batch and head indexing
    across many workgroups, each with a ragged last tile."""
    full_parity(32, 8, 65, 64, "f16", causal, 0.125, seed=12)
