"""Split-K decode on the GPU against the fp64 oracle, through the C-ABI library."""

import numpy as np
import pytest
import torch

import exact_attention_prefill_amd as ea
import oracle
import workloads as W
from parity import TOL, check, f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run(q, kc, vc, lens, scale, **kw):
    out = ea.decode(q.to(DEV), kc.to(DEV), vc.to(DEV), lens.to(DEV), scale=scale, **kw)
    torch.cuda.synchronize()
    return out


def parity(B, H, max_len, d, dtype, scale, seed, seq_lens=None, **kw):
    q, kc, vc, lens = W.decode_inputs(B, H, max_len, d, dtype, seed, seq_lens)
    out = run(q, kc, vc, lens, scale, **kw)
    ref = oracle.decode(f64(q), f64(kc), f64(vc), lens.numpy(), scale)
    return check(f64(out), ref, dtype, f"decode B{B} H{H} max_len{max_len} d{d} {dtype} seed={seed} {kw}")


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("case", W.DECODE, ids=lambda c: c.name)
def test_decode_config(case, seed):
    parity(case.B, case.H, case.max_len, case.d, case.dtype, case.scale, seed)


def test_decode_seed0_lengths_recorded():
    _, _, _, lens = W.decode_inputs(8, 12, 4096, 64, "f16", 0)
    assert lens.tolist() == [2654, 1016, 3651, 900, 2779, 4081, 4033, 2006]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
def test_edge_lengths(d, dtype):
    lens = [1, 31, 32, 33, 63, 64, 65, 700, 4095, 4096]
    parity(len(lens), 3, 4096, d, dtype, 1.0 / np.sqrt(d), seed=d, seq_lens=lens)


@pytest.mark.parametrize("max_len", [1, 5, 32, 100])
def test_short_caches(max_len):
    lens = sorted({1, max_len, (max_len + 1) // 2})
    parity(len(lens), 2, max_len, 64, "f16", 0.125, seed=max_len, seq_lens=lens)


def test_every_legal_chunk_gives_the_same_result():
    """Page 3: output invariance across every legal split size."""
    B, H, max_len, d = 3, 4, 300, 64
    q, kc, vc, lens = W.decode_inputs(B, H, max_len, d, "f16", 11, [300, 1, 161])
    ref = oracle.decode(f64(q), f64(kc), f64(vc), lens.numpy(), 0.125)
    outs = []
    for chunk in range(32, 320 + 1, 32):
        n_split = -(-max_len // chunk)
        ws = torch.empty(ea.decode_workspace_bytes(B, H, n_split, d), dtype=torch.uint8, device=DEV)
        out = f64(run(q, kc, vc, lens, 0.125, chunk=chunk, workspace=ws))
        check(out, ref, "f16", f"chunk={chunk}")
        outs.append(out)
    spread = max(np.max(np.abs(o - outs[0])) for o in outs)
    assert spread <= TOL["f16"]


def test_chunks_at_config_size():
    q, kc, vc, lens = W.decode_inputs(8, 12, 4096, 64, "f16", 1)
    ref = oracle.decode(f64(q), f64(kc), f64(vc), lens.numpy(), 0.125)
    for chunk in (32, 96, 704, 1024, 4096):
        check(f64(run(q, kc, vc, lens, 0.125, chunk=chunk)), ref, "f16", f"chunk={chunk}")


def test_decode_equals_prefill_row():
    """Page 3: decoding token t from the cache equals row t of causal prefill."""
    B, H, N, d = 2, 12, 777, 64
    q, k, v = W.prefill_inputs(B, H, N, d, "f16", 12)
    pre = f64(ea.prefill(q.to(DEV), k.to(DEV), v.to(DEV), causal=True, scale=0.125))
    ref = oracle.prefill(f64(q), f64(k), f64(v), True, 0.125)
    for t in (0, 1, 63, 64, 500, 776):
        lens = torch.full((B,), t + 1, dtype=torch.int32)
        dec = f64(run(q[:, :, t:t + 1].contiguous(), k, v, lens, 0.125))
        check(dec[:, :, 0], ref[:, :, t], "f16", f"decode t={t}")
        assert np.max(np.abs(dec[:, :, 0] - pre[:, :, t])) <= TOL["f16"]


def test_deterministic():
    q, kc, vc, lens = (t.to(DEV) for t in W.decode_inputs(8, 12, 4096, 64, "f16", 2))
    a = ea.decode(q, kc, vc, lens, scale=0.125)
    b = ea.decode(q, kc, vc, lens, scale=0.125)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_workspace_contents_do_not_matter():
    B, H, max_len, d = 4, 3, 1000, 128
    q, kc, vc, lens = W.decode_inputs(B, H, max_len, d, "bf16", 13)
    chunk, n = 128, -(-1000 // 128)
    ws = torch.full((ea.decode_workspace_bytes(B, H, n, d) // 4,), float("nan"), device=DEV)
    a = run(q, kc, vc, lens, 0.0884, chunk=chunk, workspace=ws)
    ws.fill_(1e30)
    b = run(q, kc, vc, lens, 0.0884, chunk=chunk, workspace=ws)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    ref = oracle.decode(f64(q), f64(kc), f64(vc), lens.numpy(), 0.0884)
    check(f64(a), ref, "bf16", "poisoned workspace")


def test_out_of_range_lengths_are_clamped():
    """Lengths outside [1, max_len] are invalid; the kernels clamp them for memory
    safety: 0 (or negative) writes zeros, above max_len reads max_len rows."""
    B, H, max_len, d = 3, 2, 200, 64
    q, kc, vc, _ = W.decode_inputs(B, H, max_len, d, "f16", 14, [1, 1, 1])
    lens = torch.tensor([0, 500, -7], dtype=torch.int32)
    out = f64(run(q, kc, vc, lens, 0.125))
    assert np.all(out[0] == 0) and np.all(out[2] == 0)
    ref = oracle.decode(f64(q[1:2]), f64(kc[1:2]), f64(vc[1:2]), [max_len], 0.125)
    check(out[1:2], ref, "f16", "clamped length")
    with pytest.raises(ValueError):
        ea.decode(q.to(DEV), kc.to(DEV), vc.to(DEV), lens.to(DEV), scale=0.125, validate=True)


@pytest.mark.parametrize("scale", [0.0, -0.5, 2.0])
def test_decode_scales(scale):
    parity(2, 3, 500, 64, "f16", scale, seed=15, seq_lens=[500, 77])


def test_nan_prefilled_out_and_canaries():
    B, H, max_len, d = 8, 12, 4096, 64
    q, kc, vc, lens = (t.to(DEV) for t in W.decode_inputs(B, H, max_len, d, "f16", 0))
    n, guard = B * H * d, 1024
    buf = torch.full((n + 2 * guard,), float("nan"), dtype=torch.float16, device=DEV)
    buf[:guard] = 3.0
    buf[-guard:] = 3.0
    out = buf[guard:guard + n].view(B, H, 1, d)
    ea.decode(q, kc, vc, lens, scale=0.125, out=out)
    torch.cuda.synchronize()
    assert torch.all(buf[:guard] == 3.0) and torch.all(buf[-guard:] == 3.0)
    assert torch.isfinite(out).all()


def test_workspace_too_small_raises():
    q, kc, vc, lens = (t.to(DEV) for t in W.decode_inputs(2, 2, 256, 64, "f16", 0))
    ws = torch.empty(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(ea.AttnError) as e:
        ea.decode(q, kc, vc, lens, chunk=64, workspace=ws)
    assert e.value.status == ea.ATTN_ERR_WORKSPACE


@pytest.mark.parametrize("heads", [(4, 4), (16, 4)], ids=["mha", "grouped"])
def test_long_cache_many_splits(heads):
    """A 65536-row cache: hundreds of splits per sequence, so the merge runs several
    rounds, on both split kernels (vector ALUs, and the matrix cores for the group)."""
    Hq, Hkv = heads
    B, max_len, d = 2, 65536, 128
    q, kc, vc, lens = W.decode_inputs_gqa(B, Hq, Hkv, max_len, d, "bf16", seed=77, seq_lens=[65536, 40001])
    out = ea.decode(q.to(DEV), kc.to(DEV), vc.to(DEV), lens.to(DEV), scale=1 / np.sqrt(d))
    torch.cuda.synchronize()
    chunk, n_split = ea.decode_gqa_choose_split(B, Hq, Hkv, max_len, d, torch.cuda.get_device_properties(0).multi_processor_count)
    assert n_split >= 64, (chunk, n_split)
    ref = oracle.decode(f64(q), f64(kc), f64(vc), lens.numpy(), 1 / np.sqrt(d))
    check(f64(out), ref, "bf16", f"long cache {heads} chunk={chunk} n_split={n_split}")


@pytest.mark.parametrize("Hq,Hkv,d,dtype", [(12, 12, 64, "f16"), (8, 4, 128, "bf16"), (32, 8, 128, "bf16"), (6, 6, 96, "f16")])
def test_split_then_merge_equals_decode(Hq, Hkv, d, dtype):
    """attn_decode_split then attn_decode_merge (the two passes as separate calls) give
    exactly the one-call decode's output with the same chunk and workspace, on the vector
    (multi-head, pairs of heads) and matrix-core (groups of four) split kernels."""
    B, max_len = 5, 1500
    q, kc, vc, lens = W.decode_inputs_gqa(B, Hq, Hkv, max_len, d, dtype, seed=Hq + d, seq_lens=[1500, 1, 733, 64, 1100])
    qd, kd, vd, ld = (t.to(DEV) for t in (q, kc, vc, lens))
    for chunk in (64, 224):
        ns = -(-max_len // chunk)
        ws = torch.empty(ea.decode_workspace_bytes(B, Hq, ns, d), dtype=torch.uint8, device=DEV)
        one = ea.decode(qd, kd, vd, ld, scale=0.1, chunk=chunk, workspace=ws).clone()
        ws2 = torch.empty_like(ws)
        ea.decode_split(qd, kd, vd, ld, 0.1, chunk, ws2)
        two = ea.decode_merge(ws2, torch.empty_like(qd), max_len, chunk)
        torch.cuda.synchronize()
        assert torch.equal(one.view(torch.int16), two.view(torch.int16)), chunk
        check(f64(two), oracle.decode(f64(q), f64(kc), f64(vc), lens.numpy(), 0.1), dtype, f"two passes chunk={chunk}")


def test_measure_read_writes_nothing():
    """The measurement read streams a buffer and leaves its sink untouched (its loads
    fold into a checksum that is stored only on a sentinel value the data avoids)."""
    buf = torch.zeros(3 << 20, dtype=torch.uint8, device=DEV)
    for waves in (1, 7, 1380, 4096):
        sink = torch.zeros(waves * 64, dtype=torch.int32, device=DEV)
        ea.measure_read(buf, waves, sink)
        torch.cuda.synchronize()
        assert int(sink.abs().sum()) == 0
