"""d = 64 prefill on large grids: two 32-row blocks per wave.

Grids of at least two (full) or four (causal) 256-row blocks per CU (256 CUs:
B*H*ceil(N/256) >= 512 or 1024) whose workgroups are not short (full: N > 4096,
causal: N > 12288) run d = 64 with eight-wave, 512-row workgroups in which every wave
owns two 32-row blocks and reads each K and V operand once for both (full grids keep
four K/V tiles in LDS, causal ones two).  The shapes below reach that form with ragged lengths; smaller
grids (one head at a time) run one block per wave.  A row's arithmetic does not depend
on the workgroup form (among forms with one key group), so every row of the large call
must equal the same head from a call on a slice of the heads (four-wave workgroups)
bit for bit;
sampled rows are also checked against the oracle.
"""

import numpy as np
import pytest
import torch

import exact_attention_prefill_amd as ea
import oracle
import workloads as W
from parity import check, f64, one_group_heads, plan_form

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

TWO_BLOCK = [
    W.PrefillCase("prefill_b1_h24_n12400_d64_bf16_full", 1, 24, 12400, 64, "bf16", False, 0.125),
    W.PrefillCase("prefill_b1_h24_n12400_d64_bf16_causal", 1, 24, 12400, 64, "bf16", True, 0.125),
    W.PrefillCase("prefill_b2_h12_n12350_d64_f16_causal", 2, 12, 12350, 64, "f16", True, 0.125),
    W.PrefillCase("prefill_b4_h16_n4200_d64_f16_full", 4, 16, 4200, 64, "f16", False, -0.2),
]


def reaches_two_block_form(case):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    short = case.N <= (12288 if case.causal else 4096)
    need = 4 if case.causal else 2  # 256-row blocks per CU
    return case.d == 64 and case.B * case.H * -(-case.N // 256) >= need * cus and not short


def one_head(q, k, v, b, h, causal, scale, lse=False):
    """Head (b, h) computed in a call of another form: the smallest slice of heads holding
    it that runs four-wave workgroups of one 32-row block per wave and one key group.
    Returns that head alone, shaped (1, 1, N, d)."""
    H, N, d = q.shape[1], q.shape[2], q.shape[3]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    n = one_group_heads(H, N, d, causal, cus)
    assert n is not None
    f = plan_form(1, n, N, d, causal, cus)
    assert f[0] == 4 and f[1] == 32 and f[3] == 1, f
    h0 = min(h, H - n)
    sl = lambda t: t[b:b + 1, h0:h0 + n].contiguous()  # noqa: E731
    r = ea.prefill(sl(q), sl(k), sl(v), causal=causal, scale=scale, lse=lse)
    if lse:
        return r[0][:, h - h0:h - h0 + 1], r[1][:, h - h0:h - h0 + 1]
    return r[:, h - h0:h - h0 + 1]


def grow_keys(k, N):
    growth = (1.0 + 6.0 * torch.arange(N, dtype=torch.float32) / N).view(1, 1, N, 1)
    return (k.float() * growth).to(k.dtype)


@pytest.mark.parametrize("case", TWO_BLOCK, ids=lambda c: c.name)
def test_two_block_rows_match_one_head_and_oracle(case):
    assert reaches_two_block_form(case)
    q, k, v = W.prefill_inputs(case.B, case.H, case.N, case.d, case.dtype, seed=7)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    out = ea.prefill(qd, kd, vd, causal=case.causal, scale=case.scale)
    torch.cuda.synchronize()
    rows = W.prefill_rows_sample(case.N, 40, seed=7)
    for b, h in ((0, 0), (case.B - 1, case.H - 1), (case.B // 2, 5)):
        single = one_head(qd, kd, vd, b, h, case.causal, case.scale)
        torch.cuda.synchronize()
        assert torch.equal(out[b, h].view(torch.int16), single[0, 0].view(torch.int16)), (case.name, b, h)
        ref = oracle.prefill_rows(f64(q[b:b + 1, h:h + 1]), f64(k[b:b + 1, h:h + 1]), f64(v[b:b + 1, h:h + 1]),
                                  case.causal, case.scale, 0, 0, rows)
        check(f64(out[b, h, rows]), ref, case.dtype, f"{case.name} b={b} h={h}")
    assert torch.isfinite(out).all()


@pytest.mark.parametrize("causal", [False, True])
def test_two_block_growing_scores(causal):
    """Keys growing along the sequence push the row maxima up past the optimistic
    margin again and again, so the redo path runs with both blocks of a wave live."""
    case = TWO_BLOCK[0]
    assert reaches_two_block_form(W.PrefillCase("", case.B, case.H, case.N, case.d, case.dtype, causal, 0.0))
    q, k, v = W.prefill_inputs(case.B, case.H, case.N, case.d, case.dtype, seed=21)
    k = grow_keys(k, case.N)
    scale = 2.0 / np.sqrt(case.d)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    out = ea.prefill(qd, kd, vd, causal=causal, scale=scale)
    torch.cuda.synchronize()
    rows = W.prefill_rows_sample(case.N, 40, seed=21)
    for h in (0, 13, 23):
        single = one_head(qd, kd, vd, 0, h, causal, scale)
        torch.cuda.synchronize()
        assert torch.equal(out[0, h].view(torch.int16), single[0, 0].view(torch.int16)), h
        ref = oracle.prefill_rows(f64(q[:, h:h + 1]), f64(k[:, h:h + 1]), f64(v[:, h:h + 1]), causal, scale, 0, 0,
                                  rows)
        check(f64(out[0, h, rows]), ref, case.dtype, f"growing scores two-block h={h} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_two_block_grouped_heads(causal):
    """24 query heads over 8 K/V heads at d = 64: each query head reads its group's
    K/V head; rows must equal the multi-head call on repeated K/V heads."""
    B, Hq, Hkv, N, d = 1, 24, 8, 12400, 64
    assert reaches_two_block_form(W.PrefillCase("", B, Hq, N, d, "bf16", causal, 0.0))
    scale = 0.125
    q, k, v = W.prefill_inputs_gqa(B, Hq, Hkv, N, d, "bf16", seed=5)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    out = ea.prefill(qd, kd, vd, causal=causal, scale=scale)
    g = Hq // Hkv
    rep = ea.prefill(qd, kd.repeat_interleave(g, dim=1).contiguous(), vd.repeat_interleave(g, dim=1).contiguous(),
                     causal=causal, scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), rep.view(torch.int16))
    rows = W.prefill_rows_sample(N, 32, seed=5)
    for h in (0, 2, 3, 23):
        ref = oracle.prefill_rows(f64(q), f64(k), f64(v), causal, scale, 0, h, rows)
        check(f64(out[0, h, rows]), ref, "bf16", f"two-block gqa h={h} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_two_block_lse(causal):
    """The row log-sum-exp output of the two-block form: against the oracle on sampled
    rows, equal to the one-head call, and the output unchanged by asking for it."""
    case = TWO_BLOCK[0]
    assert reaches_two_block_form(W.PrefillCase("", case.B, case.H, case.N, case.d, case.dtype, causal, 0.0))
    q, k, v = W.prefill_inputs(case.B, case.H, case.N, case.d, case.dtype, seed=9)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    out, lse = ea.prefill(qd, kd, vd, causal=causal, scale=case.scale, lse=True)
    plain = ea.prefill(qd, kd, vd, causal=causal, scale=case.scale)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), plain.view(torch.int16))
    rows = W.prefill_rows_sample(case.N, 40, seed=9)
    for h in (0, 23):
        _, single = one_head(qd, kd, vd, 0, h, causal, case.scale, lse=True)
        torch.cuda.synchronize()
        assert torch.equal(lse[0, h], single[0, 0]), h
        ref = oracle.prefill_lse_rows(f64(q), f64(k), causal, case.scale, 0, h, rows)
        err = float(np.max(np.abs(lse[0, h, rows].double().cpu().numpy() - ref)))
        assert err <= 4.5e-3, f"two-block lse h={h}: {err:.3e}"
