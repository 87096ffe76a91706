"""HIP graph capture of the library's calls (prefill, decode with a caller workspace, the
backward pass with a caller workspace): torch captures the launches on its capture
stream, and every replay, with eager work and synchronisations between replays, gives
the eager results bit for bit.  None of these calls allocates or clears memory with a
memset, so the captured graphs hold kernel nodes only."""

import pytest
import torch

import exact_attention_prefill_amd as ea
import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def bits(t):
    return t.view(torch.int16).clone()


def test_graph_replays_match_eager():
    q, k, v = (t.to(DEV) for t in W.prefill_inputs_gqa(1, 8, 2, 700, 128, "bf16", seed=3))
    dq_, kc, vc, lens = (t.to(DEV) for t in W.decode_inputs_gqa(4, 16, 4, 1000, 128, "bf16", 4, [1000, 3, 517, 64]))
    dmha = [t.to(DEV) for t in W.decode_inputs(4, 6, 500, 64, "f16", 5, [500, 1, 250, 33])]
    dout = W.prefill_inputs(1, 8, 700, 128, "bf16", seed=6)[0].to(DEV)
    out = torch.empty_like(q)
    lse = torch.empty(1, 8, 700, dtype=torch.float32, device=DEV)
    dec = torch.empty_like(dq_)
    dec2 = torch.empty_like(dmha[0])
    chunk, ns = ea.decode_gqa_choose_split(4, 16, 4, 1000, 128, 256)
    ws = torch.empty(ea.decode_workspace_bytes(4, 16, ns, 128), dtype=torch.uint8, device=DEV)
    ws2 = torch.empty(ea.decode_workspace_bytes(4, 6, -(-500 // 64), 64), dtype=torch.uint8, device=DEV)
    bws = torch.empty(ea.backward_workspace_bytes(1, 8, 700) // 4, dtype=torch.float32, device=DEV)
    grads = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)]

    def work():
        ea.prefill(q, k, v, causal=True, scale=0.09, out=out, lse=lse)
        ea.decode(dq_, kc, vc, lens, scale=0.09, out=dec, chunk=chunk, workspace=ws)
        ea.decode(*dmha, scale=0.125, out=dec2, chunk=64, workspace=ws2)
        ea.backward(q, k, v, out, dout, lse, causal=True, scale=0.09, dq=grads[0], dk=grads[1], dv=grads[2],
                    workspace=bws)

    work()
    torch.cuda.synchronize()
    ref = [bits(t) for t in (out, dec, dec2, *grads)] + [lse.clone()]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm up on a side stream, as capture requires
        work()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        work()
    torch.cuda.synchronize()

    for rep in range(4):
        for t in (out, dec, dec2, *grads):
            t.zero_()
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [bits(t) for t in (out, dec, dec2, *grads)] + [lse.clone()]
        for i, (a, b) in enumerate(zip(got, ref)):
            assert torch.equal(a, b), (rep, i)
        # eager work between replays, on the same buffers
        work()
        torch.cuda.synchronize()


def test_graph_replays_no_alloc_and_split_merge():
    """The calls meant for callers that capture: decode with its partials in the
    library's fixed scratch array (attn_decode_noalloc), and the decode's two passes as
    separate calls (attn_decode_split, attn_decode_merge) on a caller workspace.  Every
    replay, with eager work between, equals the eager results bit for bit."""
    q, kc, vc, lens = (t.to(DEV) for t in W.decode_inputs(8, 12, 4096, 64, "f16", 0))
    qg, kg, vg, lg = (t.to(DEV) for t in W.decode_inputs_gqa(4, 32, 8, 900, 128, "bf16", 7, [900, 5, 450, 77]))
    out_na = torch.empty_like(q)
    out_gq = torch.empty_like(qg)
    out_sm = torch.empty_like(q)
    chunk = 192
    ws = torch.empty(ea.decode_workspace_bytes(8, 12, -(-4096 // chunk), 64), dtype=torch.uint8, device=DEV)

    def work():
        ea.decode_noalloc(q, kc, vc, lens, out_na, scale=0.125)
        ea.decode_noalloc(qg, kg, vg, lg, out_gq, scale=0.09, chunk=64)
        ea.decode_split(q, kc, vc, lens, scale=0.125, chunk=chunk, workspace=ws)
        ea.decode_merge(ws, out_sm, max_len=4096, chunk=chunk)

    work()  # the first no-alloc call on a device also looks up the scratch address
    torch.cuda.synchronize()
    ref = [bits(t) for t in (out_na, out_gq, out_sm)]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        work()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        work()
    torch.cuda.synchronize()

    for rep in range(4):
        for t in (out_na, out_gq, out_sm):
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [bits(t) for t in (out_na, out_gq, out_sm)]
        for i, (a, b) in enumerate(zip(got, ref)):
            assert torch.equal(a, b), (rep, i)
        work()
        torch.cuda.synchronize()
