"""Head sizes 32, 96 and 256 (page 3, "Future work": head dimensions beyond its 64) on
the GPU, through the C-ABI library, against the fp64 oracle: prefill (both masks,
ragged lengths, both dtypes, grouped heads, the row log-sum-exp), decode over ragged
caches with every legal chunk, and decode row t equal to causal prefill row t."""

import numpy as np
import pytest
import torch

import exact_attention_prefill_amd as ea
import oracle
import workloads as W
from parity import TOL, check, f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
NEW_D = [32, 96, 256]
LSE_TOL = {"bf16": 4.5e-3, "f16": 1e-3}  # the same derivation as for d = 64 and 128


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 63, 65, 200, 333])
@pytest.mark.parametrize("d", NEW_D)
def test_prefill_parity(d, N, causal, dtype):
    B, H = 2, 2
    q, k, v = W.prefill_inputs(B, H, N, d, dtype, seed=N + d)
    scale = 1 / np.sqrt(d)
    out = ea.prefill(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, scale=scale)
    torch.cuda.synchronize()
    check(f64(out), oracle.prefill(f64(q), f64(k), f64(v), causal, scale), dtype, f"d={d} N={N} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", NEW_D)
def test_prefill_many_tiles_sampled(d, causal):
    """A mid-sized grid (16 heads of 3000 rows: 192 256-row blocks, fewer than the
    eight-wave forms need, so four-wave workgroups of two stages at d = 32 and 96; d = 256
    always runs four waves) with a ragged last tile."""
    B, H, N = 1, 16, 3000
    scale = 1 / np.sqrt(d)
    q, k, v = W.prefill_inputs(B, H, N, d, "bf16", seed=d)
    out = ea.prefill(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, scale=scale)
    torch.cuda.synchronize()
    rows = W.prefill_rows_sample(N, 24, seed=d)
    for h in (0, H - 1):
        ref = oracle.prefill_rows(f64(q), f64(k), f64(v), causal, scale, 0, h, rows)
        check(f64(out[0, h, rows]), ref, "bf16", f"d={d} h={h} causal={causal}")
    assert torch.isfinite(out).all()


@pytest.mark.parametrize("scale", [-0.2, 0.0, 0.5])
@pytest.mark.parametrize("d", NEW_D)
def test_prefill_scales(d, scale):
    q, k, v = W.prefill_inputs(1, 2, 150, d, "f16", seed=7)
    for causal in (False, True):
        out = ea.prefill(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, scale=scale)
        torch.cuda.synchronize()
        check(f64(out), oracle.prefill(f64(q), f64(k), f64(v), causal, scale), "f16", f"d={d} scale={scale}")


@pytest.mark.parametrize("d", NEW_D)
def test_prefill_grouped_heads_and_lse(d):
    B, Hq, Hkv, N = 1, 6, 2, 300
    q, k, v = W.prefill_inputs_gqa(B, Hq, Hkv, N, d, "bf16", seed=d + 1)
    scale = 1 / np.sqrt(d)
    for causal in (False, True):
        out, lse = ea.prefill(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, scale=scale, lse=True)
        torch.cuda.synchronize()
        check(f64(out), oracle.prefill(f64(q), f64(k), f64(v), causal, scale), "bf16", f"gqa d={d}")
        err = np.max(np.abs(lse.double().cpu().numpy() - oracle.prefill_lse(f64(q), f64(k), causal, scale)))
        assert err <= LSE_TOL["bf16"], (d, causal, err)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", NEW_D)
def test_decode_parity(d, dtype):
    B, H, max_len = 4, 3, 1000
    q, kc, vc, lens = W.decode_inputs(B, H, max_len, d, dtype, seed=d, seq_lens=[1000, 1, 517, 64])
    scale = 1 / np.sqrt(d)
    out = ea.decode(q.to(DEV), kc.to(DEV), vc.to(DEV), lens.to(DEV), scale=scale)
    torch.cuda.synchronize()
    check(f64(out), oracle.decode(f64(q), f64(kc), f64(vc), lens.numpy(), scale), dtype, f"decode d={d} {dtype}")


@pytest.mark.parametrize("d", NEW_D)
def test_decode_every_chunk(d):
    B, H, max_len = 2, 2, 300
    q, kc, vc, lens = W.decode_inputs(B, H, max_len, d, "f16", seed=3, seq_lens=[300, 161])
    ref = oracle.decode(f64(q), f64(kc), f64(vc), lens.numpy(), 0.1)
    outs = []
    for chunk in range(32, 320 + 1, 32):
        n_split = -(-max_len // chunk)
        ws = torch.empty(ea.decode_workspace_bytes(B, H, n_split, d), dtype=torch.uint8, device=DEV)
        out = ea.decode(q.to(DEV), kc.to(DEV), vc.to(DEV), lens.to(DEV), scale=0.1, chunk=chunk, workspace=ws)
        torch.cuda.synchronize()
        out = f64(out)
        check(out, ref, "f16", f"d={d} chunk={chunk}")
        outs.append(out)
    assert max(np.max(np.abs(o - outs[0])) for o in outs) <= TOL["f16"]


@pytest.mark.parametrize("g", [1, 4, 8])
@pytest.mark.parametrize("d", NEW_D)
def test_decode_grouped_heads(d, g):
    B, Hkv, max_len = 3, 2, 700
    q, kc, vc, lens = W.decode_inputs_gqa(B, g * Hkv, Hkv, max_len, d, "bf16", seed=g + d, seq_lens=[700, 5, 333])
    out = ea.decode(q.to(DEV), kc.to(DEV), vc.to(DEV), lens.to(DEV), scale=0.11)
    torch.cuda.synchronize()
    check(f64(out), oracle.decode(f64(q), f64(kc), f64(vc), lens.numpy(), 0.11), "bf16", f"decode gqa d={d} g={g}")


@pytest.mark.parametrize("d", NEW_D)
def test_decode_row_equals_prefill_row(d):
    """Decoding token t over a cache of t + 1 rows equals causal prefill row t (page 3,
    "What can it do"): each GPU result within the gate of the oracle and of the other."""
    N, H = 260, 2
    q, k, v = W.prefill_inputs(1, H, N, d, "f16", seed=d + 9)
    pre = f64(ea.prefill(q.to(DEV), k.to(DEV), v.to(DEV), causal=True, scale=0.125))
    ref = oracle.prefill(f64(q), f64(k), f64(v), True, 0.125)
    for t in (0, 64, 259):
        qd = q[:, :, t : t + 1].contiguous()
        lens = torch.tensor([t + 1], dtype=torch.int32)
        dec = f64(ea.decode(qd.to(DEV), k.to(DEV), v.to(DEV), lens.to(DEV), scale=0.125))
        torch.cuda.synchronize()
        check(dec[:, :, 0], ref[:, :, t], "f16", f"decode d={d} t={t}")
        assert np.max(np.abs(dec[:, :, 0] - pre[:, :, t])) <= TOL["f16"]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", NEW_D)
def test_prefill_growing_scores(d, causal):
    """Key magnitudes growing along the sequence push each row's maximum past the
    optimistic softmax's 2^8 margin again and again (the rescale path)."""
    q, k, v = W.prefill_inputs(1, 2, 700, d, "bf16", 21)
    growth = (1.0 + 6.0 * torch.arange(700, dtype=torch.float32) / 700).view(1, 1, 700, 1)
    k = (k.float() * growth).to(k.dtype)
    scale = 2.0 / np.sqrt(d)
    out = ea.prefill(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, scale=scale)
    torch.cuda.synchronize()
    check(f64(out), oracle.prefill(f64(q), f64(k), f64(v), causal, scale), "bf16", f"growing d={d}")


@pytest.mark.parametrize("d", NEW_D)
def test_prefill_causality_and_canaries(d):
    """Causal rows 0..i are bit-identical when K/V rows after i change, and writes stay
    inside the output (NaN-filled, with canaries on both sides)."""
    N, i = 500, 200
    q, k, v = W.prefill_inputs(1, 2, N, d, "f16", 4)
    n = q.numel()
    guard = 4096
    buf = torch.full((n + 2 * guard,), float("nan"), dtype=torch.float16, device=DEV)
    canary = torch.full((guard,), 12.5, dtype=torch.float16, device=DEV)
    buf[:guard] = canary
    buf[-guard:] = canary
    a = buf[guard:guard + n].view(q.shape)
    ea.prefill(q.to(DEV), k.to(DEV), v.to(DEV), causal=True, scale=0.125, out=a)
    k2, v2 = k.clone(), v.clone()
    k2[:, :, i + 1:] = torch.randn(k2[:, :, i + 1:].shape).to(k2.dtype) * 3
    v2[:, :, i + 1:] = 100.0
    b = ea.prefill(q.to(DEV), k2.to(DEV), v2.to(DEV), causal=True, scale=0.125)
    torch.cuda.synchronize()
    assert torch.equal(buf[:guard], canary) and torch.equal(buf[-guard:], canary)
    assert torch.isfinite(a).all()
    assert torch.equal(a[:, :, : i + 1].view(torch.int16), b[:, :, : i + 1].view(torch.int16))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", NEW_D)
def test_prefill_sixteen_k_sampled(d, dtype):
    """B=1, H=16, N=16384, non-causal: the shape and launch form of the benchmark's
    head-size sweep (eight-wave workgroups at d = 32 and 96, four waves at d = 256, as
    the launch plan asserts), sampled rows of three heads against the row-sampled
    oracle."""
    B, H, N = 1, 16, 16384
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert ea.prefill_plan(B, H, N, d, False, cus)["waves"] == (4 if d == 256 else 8)
    scale = 1 / np.sqrt(d)
    q, k, v = W.prefill_inputs(B, H, N, d, dtype, seed=d + 3)
    out = ea.prefill(q.to(DEV), k.to(DEV), v.to(DEV), scale=scale)
    torch.cuda.synchronize()
    rows = W.prefill_rows_sample(N, 16, seed=d)
    for h in (0, 7, H - 1):
        ref = oracle.prefill_rows(f64(q[:, h:h + 1]), f64(k[:, h:h + 1]), f64(v[:, h:h + 1]), False, scale, 0, 0, rows)
        check(f64(out[0, h, rows]), ref, dtype, f"d={d} {dtype} N=16384 h={h}")
    assert torch.isfinite(out).all()
