"""The C-ABI library on the CPU: it loads, exports every declared symbol, and rejects
invalid arguments before any HIP call (no compute call is made here)."""

import ctypes
import os
import re

import pytest

import exact_attention_prefill_amd as ea

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

# Fake, 16-byte aligned "device" addresses: validation must fail before they are used.
P = [0x10000 + 0x100 * i for i in range(8)]


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_]+)\s*\(", text)))


def test_header_declares_the_exports():
    assert declared_functions() == sorted(ea.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = ea.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
        assert getattr(L, name) is not None


def _prefill(**kw):
    a = dict(q=P[0], k=P[1], v=P[2], out=P[3], B=1, H=1, N=128, d=64, dt=0, causal=0, scale=0.125, s=None)
    a.update(kw)
    return ea.lib().attn_prefill(a["q"], a["k"], a["v"], a["out"], a["B"], a["H"], a["N"], a["d"], a["dt"],
                                 a["causal"], a["scale"], a["s"])


@pytest.mark.parametrize(
    "kw,status",
    [
        (dict(B=0), ea.ATTN_ERR_INVALID_ARG),
        (dict(H=-1), ea.ATTN_ERR_INVALID_ARG),
        (dict(N=0), ea.ATTN_ERR_INVALID_ARG),
        (dict(d=80), ea.ATTN_ERR_UNSUPPORTED),
        (dict(d=48), ea.ATTN_ERR_UNSUPPORTED),
        (dict(d=512), ea.ATTN_ERR_UNSUPPORTED),
        (dict(d=16), ea.ATTN_ERR_UNSUPPORTED),
        (dict(dt=2), ea.ATTN_ERR_INVALID_ARG),
        (dict(causal=2), ea.ATTN_ERR_INVALID_ARG),
        (dict(scale=float("nan")), ea.ATTN_ERR_INVALID_ARG),
        (dict(scale=float("inf")), ea.ATTN_ERR_INVALID_ARG),
        (dict(q=None), ea.ATTN_ERR_INVALID_ARG),
        (dict(out=None), ea.ATTN_ERR_INVALID_ARG),
        (dict(k=P[1] + 8), ea.ATTN_ERR_ALIGNMENT),
        (dict(out=P[0]), ea.ATTN_ERR_INVALID_ARG),
        (dict(out=P[2]), ea.ATTN_ERR_INVALID_ARG),
    ],
)
def test_prefill_validation(kw, status):
    assert _prefill(**kw) == status
    assert ea.last_error() != ""


def _decode_ex(**kw):
    a = dict(q=P[0], k=P[1], v=P[2], lens=P[4], out=P[3], B=2, H=3, max_len=100, d=64, dt=0, scale=0.125,
             chunk=32, ws=P[5], ws_bytes=1 << 20, s=None)
    a.update(kw)
    return ea.lib().attn_decode_ex(a["q"], a["k"], a["v"], a["lens"], a["out"], a["B"], a["H"], a["max_len"],
                                   a["d"], a["dt"], a["scale"], a["chunk"], a["ws"], a["ws_bytes"], a["s"])


@pytest.mark.parametrize(
    "kw,status",
    [
        (dict(B=0), ea.ATTN_ERR_INVALID_ARG),
        (dict(max_len=0), ea.ATTN_ERR_INVALID_ARG),
        (dict(d=192), ea.ATTN_ERR_UNSUPPORTED),
        (dict(d=160), ea.ATTN_ERR_UNSUPPORTED),
        (dict(lens=None), ea.ATTN_ERR_INVALID_ARG),
        (dict(lens=P[4] + 2), ea.ATTN_ERR_ALIGNMENT),
        (dict(chunk=16), ea.ATTN_ERR_INVALID_ARG),
        (dict(chunk=33), ea.ATTN_ERR_INVALID_ARG),
        (dict(chunk=160), ea.ATTN_ERR_INVALID_ARG),  # above roundup(100, 32) = 128
        (dict(chunk=-32), ea.ATTN_ERR_INVALID_ARG),
        (dict(ws=P[5] + 4), ea.ATTN_ERR_ALIGNMENT),
        (dict(ws=None, ws_bytes=64), ea.ATTN_ERR_INVALID_ARG),
        (dict(ws_bytes=100), ea.ATTN_ERR_WORKSPACE),
        (dict(scale=float("-inf")), ea.ATTN_ERR_INVALID_ARG),
        (dict(out=P[1]), ea.ATTN_ERR_INVALID_ARG),
        (dict(B=65536, max_len=32, chunk=32), ea.ATTN_ERR_INVALID_ARG),  # the launch grid's batch limit
        (dict(B=1, H=65536, max_len=32, chunk=32), ea.ATTN_ERR_INVALID_ARG),  # and its head limit
    ],
)
def test_decode_validation(kw, status):
    assert _decode_ex(**kw) == status
    assert ea.last_error() != ""


def test_decode_workspace_check_is_exact():
    need = ea.decode_workspace_bytes(2, 3, 4, 64)  # max_len 100, chunk 32 -> 4 splits
    assert need == 2 * 3 * 4 * 66 * 4
    assert _decode_ex(ws_bytes=need - 1) == ea.ATTN_ERR_WORKSPACE


def test_plain_decode_validation():
    L = ea.lib()
    assert L.attn_decode(P[0], P[1], P[2], P[4], P[3], 1, 1, 0, 64, 0, 0.125, None) == ea.ATTN_ERR_INVALID_ARG
    assert L.attn_decode(P[0], P[1], P[2], P[4], P[3], 1, 1, 8, 80, 0, 0.125, None) == ea.ATTN_ERR_UNSUPPORTED


def test_status_strings():
    for s in (0, -1, -2, -3, -4, -5):
        assert ea.status_string(s) and ea.status_string(s) != "unknown status"
    assert ea.status_string(7) == "unknown status"


def test_last_error_is_thread_local():
    import threading

    assert _prefill(B=0) == ea.ATTN_ERR_INVALID_ARG
    seen = []
    t = threading.Thread(target=lambda: seen.append(ea.last_error()))
    t.start()
    t.join()
    assert seen == [""]
    assert ea.last_error() != ""


def test_workspace_bytes():
    assert ea.decode_workspace_bytes(8, 12, 6, 64) == 8 * 12 * 6 * 66 * 4
    assert ea.decode_workspace_bytes(0, 12, 6, 64) == 0


def _prefill_gqa(**kw):
    a = dict(q=P[0], k=P[1], v=P[2], out=P[3], B=1, Hq=8, Hkv=2, N=128, d=64, dt=0, causal=0, scale=0.125, s=None)
    a.update(kw)
    return ea.lib().attn_prefill_gqa(a["q"], a["k"], a["v"], a["out"], a["B"], a["Hq"], a["Hkv"], a["N"], a["d"],
                                     a["dt"], a["causal"], a["scale"], a["s"])


@pytest.mark.parametrize(
    "kw,status",
    [
        (dict(Hkv=0), ea.ATTN_ERR_INVALID_ARG),
        (dict(Hkv=3), ea.ATTN_ERR_INVALID_ARG),  # does not divide 8
        (dict(Hkv=16), ea.ATTN_ERR_INVALID_ARG),  # more K/V heads than query heads
        (dict(Hq=0), ea.ATTN_ERR_INVALID_ARG),
        (dict(d=80), ea.ATTN_ERR_UNSUPPORTED),
        (dict(k=P[1] + 4), ea.ATTN_ERR_ALIGNMENT),
        (dict(out=P[1]), ea.ATTN_ERR_INVALID_ARG),
    ],
)
def test_prefill_gqa_validation(kw, status):
    assert _prefill_gqa(**kw) == status
    assert ea.last_error() != ""


def _decode_gqa(**kw):
    a = dict(q=P[0], k=P[1], v=P[2], lens=P[4], out=P[3], B=2, Hq=6, Hkv=2, max_len=100, d=128, dt=1, scale=0.1,
             chunk=32, ws=P[5], ws_bytes=1 << 20, s=None)
    a.update(kw)
    return ea.lib().attn_decode_gqa(a["q"], a["k"], a["v"], a["lens"], a["out"], a["B"], a["Hq"], a["Hkv"],
                                    a["max_len"], a["d"], a["dt"], a["scale"], a["chunk"], a["ws"], a["ws_bytes"],
                                    a["s"])


@pytest.mark.parametrize(
    "kw,status",
    [
        (dict(Hkv=4), ea.ATTN_ERR_INVALID_ARG),
        (dict(Hkv=0), ea.ATTN_ERR_INVALID_ARG),
        (dict(Hkv=12), ea.ATTN_ERR_INVALID_ARG),
        (dict(B=65536, max_len=32, chunk=32), ea.ATTN_ERR_INVALID_ARG),  # the launch grid's batch limit
        (dict(chunk=48), ea.ATTN_ERR_INVALID_ARG),
        (dict(lens=None), ea.ATTN_ERR_INVALID_ARG),
        (dict(ws_bytes=ea.decode_workspace_bytes(2, 6, 4, 128) - 1), ea.ATTN_ERR_WORKSPACE),
        (dict(ws_bytes=ea.decode_workspace_bytes(2, 2, 4, 128)), ea.ATTN_ERR_WORKSPACE),  # sized per K/V head: too small
    ],
)
def test_decode_gqa_validation(kw, status):
    assert _decode_gqa(**kw) == status
    assert ea.last_error() != ""


def test_gqa_chooser():
    # Equal head counts choose exactly as multi-head decode does.
    for B, H in ((1, 12), (8, 12), (4, 32)):
        assert ea.decode_gqa_choose_split(B, H, H, 4096, 64, 256) == ea.decode_choose_split(B, H, 4096, 64, 256)
    # Pairs and groups past 32 heads (vector ALUs): one wave serves the largest divisor
    # of the group size that is at most 8; fewer waves per split, as for that many
    # fewer heads.  (Groups of 3..32 run on the matrix cores with their own target:
    # tests/test_chooser.py.)
    for Hq, Hkv, waves in ((64, 1, 8), (66, 1, 11), (40, 1, 5), (16, 8, 8), (2, 1, 1), (70, 2, 10)):
        assert ea.decode_gqa_choose_split(8, Hq, Hkv, 4096, 128, 256) == ea.decode_choose_split(8, waves, 4096, 128, 256)
    with pytest.raises(ValueError):
        ea.decode_gqa_choose_split(1, 8, 3, 100, 64, 256)


def _prefill_ex(**kw):
    a = dict(q=P[0], k=P[1], v=P[2], out=P[3], lse=P[6], B=1, Hq=4, Hkv=2, N=64, d=128, dt=1, causal=1, scale=0.1,
             s=None)
    a.update(kw)
    return ea.lib().attn_prefill_ex(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["N"],
                                    a["d"], a["dt"], a["causal"], a["scale"], a["s"])


@pytest.mark.parametrize(
    "kw,status",
    [
        (dict(lse=P[6] + 2), ea.ATTN_ERR_ALIGNMENT),
        (dict(lse=P[3]), ea.ATTN_ERR_INVALID_ARG),  # aliases out
        (dict(lse=P[0]), ea.ATTN_ERR_INVALID_ARG),  # aliases q
        (dict(Hkv=3), ea.ATTN_ERR_INVALID_ARG),
        (dict(N=0), ea.ATTN_ERR_INVALID_ARG),
        (dict(d=64, dt=5), ea.ATTN_ERR_INVALID_ARG),
    ],
)
def test_prefill_ex_validation(kw, status):
    assert _prefill_ex(**kw) == status
    assert ea.last_error() != ""


def _backward(**kw):
    a = dict(q=P[0], k=P[1], v=P[2], out=P[3], dout=P[4], lse=P[5], dq=P[6], dk=P[7], dv=0x30000, B=1, Hq=4, Hkv=2,
             N=64, d=128, dt=1, causal=0, scale=0.1, ws=None, ws_bytes=0, s=None)
    a.update(kw)
    return ea.lib().attn_backward(a["q"], a["k"], a["v"], a["out"], a["dout"], a["lse"], a["dq"], a["dk"], a["dv"],
                                  a["B"], a["Hq"], a["Hkv"], a["N"], a["d"], a["dt"], a["causal"], a["scale"],
                                  a["ws"], a["ws_bytes"], a["s"])


@pytest.mark.parametrize(
    "kw,status",
    [
        (dict(Hkv=3), ea.ATTN_ERR_INVALID_ARG),
        (dict(d=192), ea.ATTN_ERR_UNSUPPORTED),
        (dict(d=80), ea.ATTN_ERR_UNSUPPORTED),
        (dict(lse=None), ea.ATTN_ERR_INVALID_ARG),
        (dict(lse=P[5] + 2), ea.ATTN_ERR_ALIGNMENT),
        (dict(dq=P[0]), ea.ATTN_ERR_INVALID_ARG),  # gradient aliases q
        (dict(dv=P[6]), ea.ATTN_ERR_INVALID_ARG),  # dv aliases dq
        (dict(dout=None), ea.ATTN_ERR_INVALID_ARG),
        (dict(causal=3), ea.ATTN_ERR_INVALID_ARG),
        (dict(ws=0x40000, ws_bytes=16), ea.ATTN_ERR_WORKSPACE),
        (dict(ws=None, ws_bytes=16), ea.ATTN_ERR_INVALID_ARG),
        (dict(ws=0x40008, ws_bytes=1 << 20), ea.ATTN_ERR_ALIGNMENT),
    ],
)
def test_backward_validation(kw, status):
    assert _backward(**kw) == status
    assert ea.last_error() != ""


def test_backward_workspace_bytes():
    assert ea.backward_workspace_bytes(2, 8, 100) == 2 * (2 * 8 * 100 * 4)
    assert ea.backward_workspace_bytes(0, 8, 100) == 0


def test_library_was_built_from_these_sources():
    from exact_attention_prefill_amd import build

    assert ea.build_id() == build.source_hash()


def test_noalloc_decode_validation():
    """attn_decode_noalloc validates like attn_decode_gqa and refuses, before any HIP
    call, an explicit chunk whose partials exceed the device scratch."""
    L = ea.lib()
    call = lambda B, H, Hkv, max_len, d, chunk: L.attn_decode_noalloc(  # noqa: E731
        P[0], P[1], P[2], P[4], P[3], B, H, Hkv, max_len, d, 0, 0.125, chunk, None)
    assert call(0, 1, 1, 64, 64, 0) == ea.ATTN_ERR_INVALID_ARG
    assert call(1, 6, 4, 64, 64, 0) == ea.ATTN_ERR_INVALID_ARG  # Hkv does not divide H
    assert call(1, 1, 1, 64, 80, 0) == ea.ATTN_ERR_UNSUPPORTED
    assert call(1, 1, 1, 64, 64, 48) == ea.ATTN_ERR_INVALID_ARG  # not a multiple of the granule
    assert call(65536, 1, 1, 32, 32, 0) == ea.ATTN_ERR_INVALID_ARG  # the launch grid's batch limit
    assert ea.decode_workspace_bytes(64, 32, 128, 64) > ea.DECODE_SCRATCH_BYTES
    assert call(64, 32, 32, 4096, 64, 32) == ea.ATTN_ERR_WORKSPACE
    assert "scratch" in ea.last_error()
    # One split per head already too large: B*H*(d+2)*4 bytes over the scratch.
    assert call(64, 256, 256, 64, 256, 0) == ea.ATTN_ERR_WORKSPACE


def test_decode_pass_and_read_validation():
    """The separate decode passes and the measurement read refuse bad arguments before
    any HIP call."""
    L = ea.lib()
    split = lambda chunk, ws, wsb: L.attn_decode_split(  # noqa: E731
        P[0], P[1], P[2], P[4], 2, 3, 3, 100, 64, 0, 0.125, chunk, ws, wsb, None)
    need = ea.decode_workspace_bytes(2, 3, 4, 64)  # chunk 32 -> 4 splits
    assert split(0, P[5], need) == ea.ATTN_ERR_INVALID_ARG  # the split pass needs a chunk
    assert split(32, None, 0) == ea.ATTN_ERR_INVALID_ARG  # and a workspace
    assert split(32, P[5], need - 1) == ea.ATTN_ERR_WORKSPACE
    assert split(48, P[5], need) == ea.ATTN_ERR_INVALID_ARG
    merge = lambda chunk, wsb, out=P[3]: L.attn_decode_merge(P[5], wsb, out, 2, 3, 100, 64, 0, chunk, None)  # noqa: E731
    assert merge(32, need - 1) == ea.ATTN_ERR_WORKSPACE
    assert merge(0, need) == ea.ATTN_ERR_INVALID_ARG
    assert merge(32, need, out=P[5]) == ea.ATTN_ERR_INVALID_ARG  # out aliases the workspace
    assert merge(32, need, out=None) == ea.ATTN_ERR_INVALID_ARG
    big = lambda B, H: L.attn_decode_merge(P[5], 1 << 40, P[3], B, H, 32, 64, 0, 32, None)  # noqa: E731
    assert big(65536, 1) == ea.ATTN_ERR_INVALID_ARG  # the launch grid's batch limit
    assert big(1, 65536) == ea.ATTN_ERR_INVALID_ARG
    read = lambda nbytes, waves, sink_bytes: L.attn_measure_read(P[0], nbytes, waves, P[6], sink_bytes, None)  # noqa: E731
    assert read(100, 1, 256) == ea.ATTN_ERR_INVALID_ARG  # not a multiple of 16
    assert read(1024, 0, 256) == ea.ATTN_ERR_INVALID_ARG
    assert read(1024, 65, 65 * 256) == ea.ATTN_ERR_INVALID_ARG  # more waves than 16-byte elements
    assert read(1024, 4, 4 * 256 - 1) == ea.ATTN_ERR_WORKSPACE
