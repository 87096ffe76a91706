"""Row log-sum-exp from the prefill kernel (attn_prefill_ex) against the fp64 oracle.

Bound: the kernel's l sums P after rounding to the input type, each term off by at
most a relative u (2^-8 bf16, 2^-11 fp16), so log l is off by at most log(1 + u);
fp32 accumulation of up to 16K terms per lane and the fp32 m add at most ~5e-4 more.
Gate: 4.5e-3 (bf16), 1e-3 (fp16), absolute."""

import numpy as np
import pytest
import torch

import exact_attention_prefill_amd as ea
import oracle
import workloads as W
from parity import check, f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
LSE_TOL = {"bf16": 4.5e-3, "f16": 1e-3}


def lse_check(got, ref, dtype, what):
    err = np.max(np.abs(got - ref))
    assert np.all(np.isfinite(got)), what
    assert err <= LSE_TOL[dtype], f"{what}: lse max err {err:.3e}"
    return err


CASES = [
    # B, Hq, Hkv, N, d, dtype, scale
    (1, 2, 2, 333, 64, "f16", 0.125),
    (2, 4, 2, 200, 128, "bf16", 1 / np.sqrt(128)),
    (1, 3, 1, 65, 128, "f16", -0.2),
    (1, 2, 2, 129, 64, "bf16", 0.0),
    (1, 2, 2, 150, 64, "f16", 1.0),  # the fp16 form that scales fp32 scores
    (1, 6, 3, 1000, 128, "bf16", 2.0 / np.sqrt(128)),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "b{}_hq{}_hkv{}_n{}_d{}_{}_s{:.3g}".format(*c))
def test_lse_parity(case, causal):
    B, Hq, Hkv, N, d, dtype, scale = case
    q, k, v = W.prefill_inputs_gqa(B, Hq, Hkv, N, d, dtype, seed=N + d)
    out, lse = ea.prefill(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, scale=scale, lse=True)
    torch.cuda.synchronize()
    lse_check(lse.double().cpu().numpy(), oracle.prefill_lse(f64(q), f64(k), causal, scale), dtype, str(case))
    check(f64(out), oracle.prefill(f64(q), f64(k), f64(v), causal, scale), dtype, f"out with lse {case}")


def test_lse_leaves_output_unchanged():
    q, k, v = (t.to(DEV) for t in W.prefill_inputs(1, 4, 500, 128, "bf16", 3))
    for causal in (False, True):
        a = ea.prefill(q, k, v, causal=causal, scale=0.09)
        b, _ = ea.prefill(q, k, v, causal=causal, scale=0.09, lse=True)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_lse_growing_scores():
    """Many raises of the running maximum: the reference m changes, m + log2 l must not."""
    B, H, N, d = 1, 2, 700, 128
    q, k, v = W.prefill_inputs(B, H, N, d, "bf16", 21)
    growth = (1.0 + 6.0 * torch.arange(N, dtype=torch.float32) / N).view(1, 1, N, 1)
    k = (k.float() * growth).to(k.dtype)
    for causal in (False, True):
        _, lse = ea.prefill(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, scale=2.0 / np.sqrt(d), lse=True)
        torch.cuda.synchronize()
        lse_check(lse.double().cpu().numpy(), oracle.prefill_lse(f64(q), f64(k), causal, 2.0 / np.sqrt(d)), "bf16",
                  f"growing causal={causal}")


def test_lse_headline_sampled():
    P = W.HEADLINE
    q, k, v = W.prefill_inputs(P.B, P.H, P.N, P.d, P.dtype, 0)
    _, lse = ea.prefill(q.to(DEV), k.to(DEV), v.to(DEV), causal=P.causal, scale=P.scale, lse=True)
    torch.cuda.synchronize()
    rows = W.prefill_rows_sample(P.N, 24, 0)
    for h in (0, P.H - 1):
        qh, kh = f64(q[0, h])[None, None], f64(k[0, h])[None, None]
        ref = oracle.prefill_lse_rows(qh, kh, P.causal, P.scale, 0, 0, rows)
        lse_check(lse[0, h, rows].double().cpu().numpy(), ref, P.dtype, f"headline h={h}")
