"""Every prefill workgroup form the launch rule can select, run on the GPU.

The library picks a workgroup form per launch from the grid (attn_prefill_plan:
waves per workgroup, query rows per wave, K/V stages in LDS).  FORM_CASES holds one
shape per reachable (head size, mask, form), each with a ragged length, and each is
run in both dtypes:
  - the case must take the form it is listed for (on a 256-CU device);
  - sampled rows of three heads, early causal rows included, match the fp64 oracle;
  - those heads' rows equal, bit for bit, the same heads computed in a call of another
    form (a two-head slice, a small grid): a row's arithmetic does not depend on the
    form.
tests/test_forms.py checks on the CPU that FORM_CASES reaches every form the rule can
select.
"""

import numpy as np
import pytest
import torch

import exact_attention_prefill_amd as ea
import oracle
import workloads as W
from parity import check, f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
CUS = 256


def _case(B, H, N, d, causal, form):
    return dict(B=B, H=H, N=N, d=d, causal=causal, form=form)


# (waves, rows per wave, stages) on 256 CUs.
EIGHT_FULL = {32: (8, 32, 2), 64: (8, 64, 4), 96: (8, 32, 2), 128: (8, 32, 2)}
EIGHT_CAUSAL = {32: (8, 32, 2), 64: (8, 64, 2), 96: (8, 32, 2), 128: (8, 32, 2)}
FORM_CASES = []
for _d in (32, 64, 96, 128):
    # Eight-wave workgroups: at least two (full) or four (causal) 256-row blocks per CU
    # and sequences past the short-workgroup limit.
    FORM_CASES.append(_case(1, 16, 8200, _d, False, EIGHT_FULL[_d]))
    FORM_CASES.append(_case(1, 16, 16400, _d, True, EIGHT_CAUSAL[_d]) if _d == 64
                      else _case(1, 32, 8250, _d, True, EIGHT_CAUSAL[_d]))
    # Four-wave workgroups with four LDS stages: small grids.
    FORM_CASES.append(_case(1, 2, 333, _d, False, (4, 32, 4)))
    FORM_CASES.append(_case(1, 2, 333, _d, True, (4, 32, 4)))
    # Four-wave workgroups with two stages: large grids of short workgroups (d = 64
    # causal always takes four stages).
    FORM_CASES.append(_case(4, 40, 1000, _d, False, (4, 32, 2)))
    if _d != 64:
        FORM_CASES.append(_case(4, 40, 1000, _d, True, (4, 32, 2)))
FORM_CASES.append(_case(1, 2, 333, 256, False, (4, 32, 2)))
FORM_CASES.append(_case(1, 2, 333, 256, True, (4, 32, 2)))


def case_id(c):
    return f"d{c['d']}_{'causal' if c['causal'] else 'full'}_b{c['B']}h{c['H']}n{c['N']}_w{c['form'][0]}r{c['form'][1]}s{c['form'][2]}"


def plan_of(c, cus=CUS):
    p = ea.prefill_plan(c["B"], c["H"], c["N"], c["d"], c["causal"], cus)
    return (p["waves"], p["rows_per_wave"], p["stages"])


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
    # The same heads from a small-grid call (another form, unless this is that form).
    sl = lambda t, b, h: t[b:b + 1, h:h + 2].contiguous() if h + 2 <= H else t[b:b + 1, h - 1:h + 1].contiguous()  # noqa: E731
    small = dict(c, B=1, H=2)
    if plan_of(small, cus) != c["form"]:
        for b, h in heads:
            two = ea.prefill(sl(qd, b, h), sl(kd, b, h), sl(vd, b, h), causal=causal, scale=scale)
            torch.cuda.synchronize()
            j = 0 if h + 2 <= H else 1
            assert torch.equal(out[b, h].view(torch.int16), two[0, j].view(torch.int16)), (case_id(c), b, h)
    assert torch.isfinite(out).all()
