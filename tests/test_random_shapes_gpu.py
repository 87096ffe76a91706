"""Prefill on seeded random shapes, drawn around the launcher's switch between workgroup
forms: grids of B*H*ceil(N/256) blocks just below, at and above four per CU (causal;
full grids switch at two per CU) take the four-wave form, the eight-wave form, or
(d = 64) two 32-row blocks per wave; short
workgroups (full N <= 2048, d = 64 N <= 4096; causal N <= 8192, d = 96 N <= 6144,
d = 64 N <= 12288) keep the four-wave form on any grid.

A second set draws small grids, of B*H*ceil(N/128) blocks around one and two per CU,
where the number of LDS stages changes (four on small grids, by head size and mask).

Every case is checked on sampled rows against the fp64 oracle, and whole heads are
compared with the same heads from a call of another form (a slice of whole K/V groups):
bit for bit when both forms have one key group (a row's arithmetic does not depend on
such a form), within the gate when either splits the keys between waves.
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


def _cases(n=18, seed=20261203):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        d = int(rng.choice([32, 64, 64, 96, 128]))
        dtype = str(rng.choice(["f16", "bf16"]))
        causal = bool(rng.integers(0, 2))
        g = int(rng.choice([1, 1, 2, 4]))
        B = int(rng.integers(1, 3))
        Hkv = int(rng.choice([4, 8, 16]))
        H = Hkv * g
        # target blocks per CU of 256 rows: just below, at, or above the switch (4 per CU)
        target = int(rng.choice([3.8 * 256, 4 * 256, 4.3 * 256]))
        nb = max(1, round(target / (B * H)))
        N = int(max(1, nb * 256 - int(rng.integers(0, 200))))  # ragged last block
        scale = float(rng.choice([1 / np.sqrt(d), 0.125, -0.3]))
        out.append((i, B, H, Hkv, N, d, dtype, causal, scale))
    return out


CASES = _cases()


def _small_cases(n=14, seed=20261205):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        d = int(rng.choice([32, 64, 96, 128]))
        dtype = str(rng.choice(["f16", "bf16"]))
        causal = bool(rng.integers(0, 2))
        g = int(rng.choice([1, 2]))
        B = int(rng.integers(1, 3))
        Hkv = int(rng.choice([2, 4, 8]))
        H = Hkv * g
        # target 128-row blocks per CU: around the one- and two-per-CU switches
        target = float(rng.choice([0.9, 1.0, 1.1, 1.9, 2.0, 2.1]))
        nb = max(1, round(target * 256 / (B * H)))
        N = int(max(1, nb * 128 - int(rng.integers(0, 100))))  # ragged last block
        scale = float(rng.choice([1 / np.sqrt(d), 0.125, -0.3]))
        out.append((100 + i, B, H, Hkv, N, d, dtype, causal, scale))
    return out


SMALL_CASES = _small_cases()


@pytest.mark.parametrize("case", CASES + SMALL_CASES,
                         ids=lambda c: f"c{c[0]}_B{c[1]}_H{c[2]}_Hkv{c[3]}_N{c[4]}_d{c[5]}_{c[6]}"
                         + ("_causal" if c[7] else ""))
def test_random_shape(case):
    i, B, H, Hkv, N, d, dtype, causal, scale = case
    q, k, v = W.prefill_inputs_gqa(B, H, Hkv, N, d, dtype, seed=100 + i)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    out = ea.prefill(qd, kd, vd, causal=causal, scale=scale)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    rows = W.prefill_rows_sample(N, 24, seed=i)
    g = H // Hkv
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    form = plan_form(B, H, N, d, causal, cus)
    # Reference: the head inside a slice of whole K/V groups that runs another form with
    # one key group (bit-identical rows when this form has one key group too), else the
    # head's own group alone.
    kk = one_group_heads(H // g, N, d, causal, cus, avoid=form)
    ng = kk if kk is not None else 1
    ref_form = plan_form(1, ng * g, N, d, causal, cus)
    for b, h in ((0, 0), (B - 1, H - 1), (B // 2, H // 2)):
        kvh = h // g
        k0 = min(kvh, H // g - ng)
        single = ea.prefill(qd[b:b + 1, k0 * g:(k0 + ng) * g].contiguous(), kd[b:b + 1, k0:k0 + ng].contiguous(),
                            vd[b:b + 1, k0:k0 + ng].contiguous(), causal=causal, scale=scale)
        torch.cuda.synchronize()
        same_rows(out[b, h], single[0, h - k0 * g], form, ref_form, dtype, f"case {case} b={b} h={h}")
        ref = oracle.prefill_rows(f64(q[b:b + 1, h:h + 1]), f64(k[b:b + 1, kvh:kvh + 1]),
                                  f64(v[b:b + 1, kvh:kvh + 1]), causal, scale, 0, 0, rows)
        check(f64(out[b, h, rows]), ref, dtype, f"case {case} b={b} h={h}")
        check(f64(single[0, h - k0 * g, rows]), ref, dtype, f"case {case} b={b} h={h} reference form")
