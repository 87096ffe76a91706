"""attn_decode_noalloc: decode with the partials in the library's fixed device scratch
array, for callers that cannot allocate.  Through the C-ABI, two calls in a row (the
second smaller), each against attn_decode_gqa with a caller workspace and the same
chunk (bit for bit) and against the fp64 oracle; grouped heads; the scratch-size
limits."""

import numpy as np
import pytest
import torch

import exact_attention_prefill_amd as ea
import oracle
import workloads as W
from parity import check, f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def reference(q, kc, vc, lens, scale, chunk):
    """attn_decode_gqa with a caller-owned workspace and the given chunk."""
    B, H, _, d = q.shape
    max_len = kc.shape[2]
    ns = -(-max_len // chunk)
    ws = torch.empty(ea.decode_workspace_bytes(B, H, ns, d), dtype=torch.uint8, device=DEV)
    return ea.decode(q, kc, vc, lens, scale=scale, chunk=chunk, workspace=ws)


def auto_chunk(B, H, Hkv, max_len, d):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return ea.decode_gqa_choose_split(B, H, Hkv, max_len, d, cus)[0]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_two_calls_second_smaller(dtype):
    """The headline ragged batch (B=8, H=12, d=64, cache 4096), then a smaller call
    (B=3, H=4, cache 700) on the same scratch: each equals the workspace path."""
    shapes = [(8, 12, 12, 4096, 64, None), (3, 4, 4, 700, 64, [700, 1, 333])]
    for i, (B, H, Hkv, max_len, d, lens) in enumerate(shapes):
        q, kc, vc, ln = W.decode_inputs(B, H, max_len, d, dtype, seed=i, seq_lens=lens)
        qd, kd, vd, ld = (t.to(DEV) for t in (q, kc, vc, ln))
        out = torch.empty_like(qd)
        ea.decode_noalloc(qd, kd, vd, ld, out, scale=0.125)
        ref = reference(qd, kd, vd, ld, 0.125, auto_chunk(B, H, Hkv, max_len, d))
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), (i, B, H, max_len)
        check(f64(out), oracle.decode(f64(q), f64(kc), f64(vc), ln.numpy(), 0.125), dtype, f"noalloc call {i}")


@pytest.mark.parametrize("chunk", [0, 32, 96, 320])
def test_grouped_heads_and_explicit_chunks(chunk):
    """Grouped heads on the matrix-core form (32 over 8 heads of 128) and the vector
    form (8 over 4), explicit chunks and the automatic one."""
    for (B, Hq, Hkv, d) in ((4, 32, 8, 128), (3, 8, 4, 64)):
        q, kc, vc, ln = W.decode_inputs_gqa(B, Hq, Hkv, 300, d, "bf16", seed=Hq + chunk,
                                            seq_lens=[300, 17, 250, 1][:B])
        qd, kd, vd, ld = (t.to(DEV) for t in (q, kc, vc, ln))
        out = torch.empty_like(qd)
        ea.decode_noalloc(qd, kd, vd, ld, out, scale=0.09, chunk=chunk)
        ref = reference(qd, kd, vd, ld, 0.09, chunk or auto_chunk(B, Hq, Hkv, 300, d))
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), (B, Hq, Hkv, d, chunk)
        check(f64(out), oracle.decode(f64(q), f64(kc), f64(vc), ln.numpy(), 0.09), "bf16", f"noalloc gqa {Hq}/{Hkv}")


def test_scratch_limits():
    """An explicit chunk whose partials exceed the scratch is refused before any work;
    the automatic chunk grows until the partials fit, and the result stays exact."""
    B, H, max_len, d = 64, 32, 4096, 64
    q, kc, vc, ln = W.decode_inputs(B, H, max_len, d, "f16", seed=4)
    qd, kd, vd, ld = (t.to(DEV) for t in (q, kc, vc, ln))
    out = torch.empty_like(qd)
    ns32 = -(-max_len // 32)
    assert ea.decode_workspace_bytes(B, H, ns32, d) > ea.DECODE_SCRATCH_BYTES
    with pytest.raises(ea.AttnError) as ei:
        ea.decode_noalloc(qd, kd, vd, ld, out, scale=0.125, chunk=32)
    assert ei.value.status == ea.ATTN_ERR_WORKSPACE
    ea.decode_noalloc(qd, kd, vd, ld, out, scale=0.125)
    torch.cuda.synchronize()
    check(f64(out), oracle.decode(f64(q), f64(kc), f64(vc), ln.numpy(), 0.125), "f16", "noalloc B=64 H=32")
    # Multi-query heads of 256 over a long cache: the automatic split's partials (32 query
    # heads x 512 splits x 258 floats) exceed the scratch, so the chunk grows to fit.
    B, Hq, Hkv, max_len, d = 1, 32, 1, 32768, 256
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    c0, n0 = ea.decode_gqa_choose_split(B, Hq, Hkv, max_len, d, cus)
    assert ea.decode_workspace_bytes(B, Hq, n0, d) > ea.DECODE_SCRATCH_BYTES, (c0, n0)
    c = c0
    while ea.decode_workspace_bytes(B, Hq, -(-max_len // c), d) > ea.DECODE_SCRATCH_BYTES:
        c += 32
    q, kc, vc, ln = W.decode_inputs_gqa(B, Hq, Hkv, max_len, d, "bf16", seed=5)
    qd, kd, vd, ld = (t.to(DEV) for t in (q, kc, vc, ln))
    out = torch.empty_like(qd)
    ea.decode_noalloc(qd, kd, vd, ld, out, scale=0.0625)
    ref = reference(qd, kd, vd, ld, 0.0625, c)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), (c0, c)
    check(f64(out), oracle.decode(f64(q), f64(kc), f64(vc), ln.numpy(), 0.0625), "bf16", "noalloc grown chunk")
