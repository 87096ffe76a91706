"""Every prefill workgroup form the launch rule can select, run on the GPU.

The library picks a workgroup form per launch from the grid (attn_prefill_plan:
waves per workgroup, query rows per wave, K/V stages in LDS).  FORM_CASES holds one
shape per reachable (head size, mask, form), each with a ragged length, and each is
run in both dtypes:
  - the case must take the form it is listed for (on a 256-CU device);
  - sampled rows of three heads, early causal rows included, match the fp64 oracle;
  - those heads' rows equal the same heads computed in a call of another form (a slice
    of the heads): bit for bit when both forms have one key group, since a row's
    arithmetic does not depend on such a form; within the gate when either splits a
    row's keys between waves (another summation order).
tests/test_forms.py checks on the CPU that FORM_CASES reaches every form the rule can
select.
"""

import numpy as np
import pytest
import torch

import exact_attention_prefill_amd as ea
import oracle
import workloads as W
from parity import check, f64, one_group_heads, plan_form, same_rows

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
CUS = 256


def _case(B, H, N, d, causal, form):
    return dict(B=B, H=H, N=N, d=d, causal=causal, form=form)


# (waves, rows per wave, stages, key groups) on 256 CUs.
EIGHT_FULL = {32: (8, 32, 2, 1), 64: (8, 64, 4, 1), 96: (8, 32, 2, 1), 128: (8, 32, 2, 1)}
EIGHT_CAUSAL = {32: (8, 32, 2, 1), 64: (8, 64, 2, 1), 96: (8, 32, 2, 1), 128: (8, 32, 2, 1)}
FORM_CASES = []
for _d in (32, 64, 96, 128):
    # Eight-wave workgroups: at least two (full) or four (causal) 256-row blocks per CU
    # and sequences past the short-workgroup limit.
    FORM_CASES.append(_case(1, 16, 8200, _d, False, EIGHT_FULL[_d]))
    FORM_CASES.append(_case(1, 16, 16400, _d, True, EIGHT_CAUSAL[_d]) if _d == 64
                      else _case(1, 32, 8250, _d, True, EIGHT_CAUSAL[_d]))
    # Grids of at most one 128-row block per CU: eight waves whose key groups split each
    # row block's keys (d <= 64: four groups on 64-row blocks, causal or half-full grids).
    small = (8, 32, 2, 4) if _d <= 64 else (8, 32, 2, 2)
    FORM_CASES.append(_case(1, 2, 333, _d, False, small))
    FORM_CASES.append(_case(1, 2, 333, _d, True, small))
    if _d <= 64:  # the GPT-2-like prompt: 192 blocks, two key groups
        FORM_CASES.append(_case(1, 12, 2000, _d, False, (8, 32, 2, 2)))
    # Causal grids of one to two 128-row blocks per CU: two key groups on 128-row blocks.
    FORM_CASES.append(_case(1, 24, 2000, _d, True, (8, 32, 2, 2)))
    # Four-wave workgroups with four LDS stages: full grids of one to two 128-row blocks
    # per CU at d <= 64; d = 64 causal on any larger grid of short workgroups.
    if _d <= 64:
        FORM_CASES.append(_case(1, 24, 2000, _d, False, (4, 32, 4, 1)))
    if _d == 64:
        FORM_CASES.append(_case(4, 40, 1000, _d, True, (4, 32, 4, 1)))
    # Four-wave workgroups with two stages: larger grids of short workgroups.
    FORM_CASES.append(_case(4, 40, 1000, _d, False, (4, 32, 2, 1)))
    if _d != 64:
        FORM_CASES.append(_case(4, 40, 1000, _d, True, (4, 32, 2, 1)))
    if _d > 64:
        FORM_CASES.append(_case(1, 24, 2000, _d, False, (4, 32, 2, 1)))
FORM_CASES.append(_case(1, 2, 333, 256, False, (4, 32, 2, 1)))
FORM_CASES.append(_case(1, 2, 333, 256, True, (4, 32, 2, 1)))


def case_id(c):
    w, r, st, kg = c["form"]
    return f"d{c['d']}_{'causal' if c['causal'] else 'full'}_b{c['B']}h{c['H']}n{c['N']}_w{w}r{r}s{st}g{kg}"


def plan_of(c, cus=CUS):
    return plan_form(c["B"], c["H"], c["N"], c["d"], c["causal"], cus)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("c", FORM_CASES, ids=case_id)
def test_form_parity_and_bits(c, dtype):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert plan_of(c, cus) == c["form"], (case_id(c), plan_of(c, cus))
    B, H, N, d, causal = c["B"], c["H"], c["N"], c["d"], c["causal"]
    seed = (N + d + 7 * causal) % 1000
    scale = 1 / np.sqrt(d)
    q, k, v = W.prefill_inputs(B, H, N, d, dtype, seed=seed)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    out = ea.prefill(qd, kd, vd, causal=causal, scale=scale)
    torch.cuda.synchronize()
    rows = sorted(set(W.prefill_rows_sample(N, 24, seed=seed)) | set(range(1, min(N, 17))))
    heads = [(0, 0), (B - 1, H - 1), (B // 2, H // 2)]
    for b, h in heads:
        ref = oracle.prefill_rows(f64(q[b:b + 1, h:h + 1]), f64(k[b:b + 1, h:h + 1]), f64(v[b:b + 1, h:h + 1]),
                                  causal, scale, 0, 0, rows)
        check(f64(out[b, h, rows]), ref, dtype, f"{case_id(c)} {dtype} b={b} h={h}")
    # The same heads from a call of another form: a slice of k heads that runs a form
    # with one key group (bit-identical rows when this form has one too), else one head.
    k = one_group_heads(H, N, d, causal, cus, avoid=c["form"]) or 1
    ref_form = plan_form(1, k, N, d, causal, cus)
    for b, h in heads:
        h0 = min(h, H - k)
        sl = lambda t: t[b:b + 1, h0:h0 + k].contiguous()  # noqa: E731
        ref = ea.prefill(sl(qd), sl(kd), sl(vd), causal=causal, scale=scale)
        torch.cuda.synchronize()
        same_rows(out[b, h], ref[0, h - h0], c["form"], ref_form, dtype, f"{case_id(c)} b={b} h={h} k={k}")
    assert torch.isfinite(out).all()
