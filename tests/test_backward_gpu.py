"""Backward pass (attn_backward) on the GPU against the fp64 oracle's gradients.

The gate is elementwise (tests/parity.py, check_grad): the rounding of the 16-bit
gradient itself plus twice the unit roundoff times a bound built from absolute values
of the products whose one factor the kernels round (P, dS) and of the delta error."""

import numpy as np
import pytest
import torch

import exact_attention_prefill_amd as ea
import oracle
import workloads as W
from parity import backward_bounds, check_grad, f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run_backward(B, Hq, Hkv, N, d, dtype, causal, scale, seed):
    q, k, v = W.prefill_inputs_gqa(B, Hq, Hkv, N, d, dtype, seed)
    g = torch.Generator("cpu").manual_seed(seed + 1000)
    dout = torch.randn(B, Hq, N, d, generator=g, dtype=torch.float32).to(q.dtype)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, dout))
    out, lse = ea.prefill(qd, kd, vd, causal=causal, scale=scale, lse=True)
    dq, dk, dv = ea.backward(qd, kd, vd, out, dod, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return (q, k, v, dout), (dq, dk, dv)


def parity(B, Hq, Hkv, N, d, dtype, causal, scale, seed):
    (q, k, v, dout), (dq, dk, dv) = run_backward(B, Hq, Hkv, N, d, dtype, causal, scale, seed)
    qf, kf, vf, df = (f64(t) for t in (q, k, v, dout))
    rq, rk, rv = oracle.backward(qf, kf, vf, df, causal, scale)
    lse = oracle.prefill_lse(qf, kf, causal, scale)
    bq, bk, bv = backward_bounds(qf, kf, vf, df, causal, scale, lse)
    what = f"B{B} Hq{Hq} Hkv{Hkv} N{N} d{d} {dtype} causal={causal} scale={scale:.3g}"
    check_grad(f64(dq), rq, bq, dtype, "dq " + what)
    check_grad(f64(dk), rk, bk, dtype, "dk " + what)
    check_grad(f64(dv), rv, bv, dtype, "dv " + what)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [32, 64, 96, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 31, 33, 63, 64, 65, 130, 257])
def test_backward_parity(N, causal, d, dtype):
    parity(1, 2, 2, N, d, dtype, causal, 1 / np.sqrt(d), seed=N + d)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("heads", [(4, 2), (6, 1), (8, 8)], ids=lambda h: f"hq{h[0]}_hkv{h[1]}")
def test_backward_grouped_heads(heads, causal):
    parity(2, heads[0], heads[1], 200, 128, "bf16", causal, 0.0884, seed=heads[0])
    parity(1, heads[0], heads[1], 150, 96, "f16", causal, 0.1, seed=heads[0] + 1)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [32, 64, 96, 128, 256])
def test_backward_many_tiles(d, causal):
    parity(1, 4, 2, 700, d, "f16" if d in (32, 64) else "bf16", causal, 1 / np.sqrt(d), seed=7)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_d256(causal):
    """Head size 256 (one wave per SIMD; dK and dV summed in two passes over the halves
    of d): grouped heads (groups of 3 and of 1), a negative scale, several key blocks
    and a ragged last tile, both dtypes."""
    parity(2, 6, 2, 300, 256, "bf16", causal, 0.0625, seed=256)
    parity(1, 3, 3, 161, 256, "f16", causal, -0.05, seed=257)
    parity(1, 4, 1, 129, 256, "bf16", causal, 0.0625, seed=258)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_d256_sampled_long(causal):
    """d = 256 at 8 heads of 4100 tokens (many key blocks and Q/dO tiles, ragged last
    tile): sampled dq rows and dk/dv key rows against the row-sampled oracle."""
    from parity import backward_bounds_keys, backward_bounds_rows

    B, H, N, d = 1, 8, 4100, 256
    scale = 1 / np.sqrt(d)
    q, k, v = W.prefill_inputs(B, H, N, d, "bf16", seed=41)
    dout = W.prefill_inputs(B, H, N, d, "bf16", seed=42)[0]
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, dout))
    out, lse = ea.prefill(qd, kd, vd, causal=causal, scale=scale, lse=True)
    dq, dk, dv = ea.backward(qd, kd, vd, out, dod, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    rows = sorted(set(W.prefill_rows_sample(N, 10, seed=43)) | {1, 2, 31, 32, 33, 4096, 4099})
    for h in (0, H - 1):
        qf, kf, vf, df = (f64(t[:, h:h + 1]) for t in (q, k, v, dout))
        ref = oracle.backward_dq_rows(qf, kf, vf, df, causal, scale, 0, 0, rows)
        bq = backward_bounds_rows(qf, kf, vf, df, causal, scale, 0, 0, rows)
        check_grad(f64(dq[0, h, rows]), ref, bq, "bf16", f"d256 dq h={h} causal={causal}")
        rk, rv = oracle.backward_dkdv_rows(qf, kf, vf, df, causal, scale, 0, 0, rows)
        bk, bv = backward_bounds_keys(qf, kf, vf, df, causal, scale, 0, 0, rows)
        check_grad(f64(dk[0, h, rows]), rk, bk, "bf16", f"d256 dk h={h} causal={causal}")
        check_grad(f64(dv[0, h, rows]), rv, bv, "bf16", f"d256 dv h={h} causal={causal}")
    for t in (dq, dk, dv):
        assert torch.isfinite(t).all()


@pytest.mark.parametrize("scale", [0.0, -0.3, 0.5])
def test_backward_scales(scale):
    parity(1, 2, 1, 150, 64, "f16", True, scale, seed=11)
    parity(1, 2, 2, 150, 128, "bf16", False, scale, seed=12)


def test_backward_deterministic():
    a = run_backward(1, 4, 2, 333, 128, "bf16", True, 0.09, 3)[1]
    b = run_backward(1, 4, 2, 333, 128, "bf16", True, 0.09, 3)[1]
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_backward_workspace_and_errors():
    (q, k, v, dout), _ = run_backward(1, 2, 2, 100, 64, "f16", False, 0.125, 5)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, dout))
    out, lse = ea.prefill(qd, kd, vd, scale=0.125, lse=True)
    ws = torch.full((ea.backward_workspace_bytes(1, 2, 100) // 4,), float("nan"), device=DEV)
    a = ea.backward(qd, kd, vd, out, dod, lse, scale=0.125, workspace=ws)
    b = ea.backward(qd, kd, vd, out, dod, lse, scale=0.125)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    small = torch.empty(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(ea.AttnError) as e:
        ea.backward(qd, kd, vd, out, dod, lse, scale=0.125, workspace=small)
    assert e.value.status == ea.ATTN_ERR_WORKSPACE


@pytest.mark.parametrize("causal", [False, True])
def test_backward_headline_sampled(causal):
    """The forward's headline shape (B=1, H=16, N=16384, d=128, bf16), in the launch
    configuration the benchmark times: dq at sampled query rows and dk, dv at sampled
    key rows of the first and last heads against the row-sampled oracle."""
    from parity import backward_bounds_keys, backward_bounds_rows

    P = W.HEADLINE
    q, k, v = W.prefill_inputs(P.B, P.H, P.N, P.d, P.dtype, seed=0)
    dout = W.prefill_inputs(P.B, P.H, P.N, P.d, P.dtype, seed=1)[0]
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, dout))
    out, lse = ea.prefill(qd, kd, vd, causal=causal, scale=P.scale, lse=True)
    dq, dk, dv = ea.backward(qd, kd, vd, out, dod, lse, causal=causal, scale=P.scale)
    torch.cuda.synchronize()
    rows = W.prefill_rows_sample(P.N, 12, seed=2)
    qf, kf, vf, df = (f64(t[:, [0, P.H - 1]]) for t in (q, k, v, dout))
    for i, h in enumerate((0, P.H - 1)):
        what = f"headline causal={causal} h={h}"
        ref = oracle.backward_dq_rows(qf, kf, vf, df, causal, P.scale, 0, i, rows)
        bq = backward_bounds_rows(qf, kf, vf, df, causal, P.scale, 0, i, rows)
        check_grad(f64(dq[0, h, rows]), ref, bq, P.dtype, "dq " + what)
        rk, rv = oracle.backward_dkdv_rows(qf, kf, vf, df, causal, P.scale, 0, i, rows)
        bk, bv = backward_bounds_keys(qf, kf, vf, df, causal, P.scale, 0, i, rows)
        check_grad(f64(dk[0, h, rows]), rk, bk, P.dtype, "dk " + what)
        check_grad(f64(dv[0, h, rows]), rv, bv, P.dtype, "dv " + what)
    for t in (dq, dk, dv):
        assert torch.isfinite(t).all()


@pytest.mark.parametrize("Hq,N", [(64, 4000), (32, 8000), (16, 8001)])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_eight_wave_dq_sampled(causal, Hq, N):
    """Query heads over 8 K/V heads with enough 256-row blocks for the eight-wave dQ
    workgroups, and a ragged last block: at 4000 tokens the causal workgroups are short
    and keep the four-wave form, at 8000 every case takes the eight-wave form, and at
    16 heads of 8001 (two blocks per CU) the full case takes it and the causal one does
    not; sampled dq rows and dk/dv key rows against the row-sampled oracle."""
    from parity import backward_bounds_keys, backward_bounds_rows

    B, Hkv, d = 1, 8, 128
    scale = 1 / np.sqrt(d)
    q, k, v = W.prefill_inputs_gqa(B, Hq, Hkv, N, d, "bf16", seed=31)
    dout = W.prefill_inputs(B, Hq, N, d, "bf16", seed=32)[0]
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, dout))
    out, lse = ea.prefill(qd, kd, vd, causal=causal, scale=scale, lse=True)
    dq, dk, dv = ea.backward(qd, kd, vd, out, dod, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    qf, kf, vf, df = (f64(t) for t in (q, k, v, dout))
    rows = W.prefill_rows_sample(N, 10, seed=33)
    for h in (0, Hq - 1):
        ref = oracle.backward_dq_rows(qf, kf, vf, df, causal, scale, 0, h, rows)
        bq = backward_bounds_rows(qf, kf, vf, df, causal, scale, 0, h, rows)
        check_grad(f64(dq[0, h, rows]), ref, bq, "bf16", f"dq h={h} causal={causal}")
    rk, rv = oracle.backward_dkdv_rows(qf, kf, vf, df, causal, scale, 0, 7, rows)
    bk, bv = backward_bounds_keys(qf, kf, vf, df, causal, scale, 0, 7, rows)
    check_grad(f64(dk[0, 7, rows]), rk, bk, "bf16", f"dk causal={causal}")
    check_grad(f64(dv[0, 7, rows]), rv, bv, "bf16", f"dv causal={causal}")
