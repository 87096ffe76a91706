"""Host logic of the automatic decode split (no GPU): page 3, "Kernel design" - the
chunk is chosen at launch so that even batch size 1 fills every compute unit."""

import itertools

import pytest

import exact_attention_prefill_amd as ea

WGS_PER_CU = ea.DECODE_WGS_PER_CU
G = ea.DECODE_ROW_GRANULE
CMIN = ea.DECODE_MIN_CHUNK


def min_chunk(max_len):
    return min(CMIN, -(-max_len // G) * G)


@pytest.mark.parametrize(
    "B,H,max_len,cus", list(itertools.product([1, 2, 8, 64], [1, 12, 32], [1, 31, 32, 33, 1000, 4096, 131072], [82, 256]))
)
def test_split_is_legal_and_covers(B, H, max_len, cus):
    chunk, n = ea.decode_choose_split(B, H, max_len, 64, cus)
    assert chunk % G == 0 and chunk >= min_chunk(max_len)
    assert chunk <= -(-max_len // G) * G
    assert n == -(-max_len // chunk)
    assert (n - 1) * chunk < max_len <= n * chunk
    # Enough splits to give every CU its share, unless the chunk is already the smallest.
    if n * B * H < WGS_PER_CU * cus:
        assert chunk == min_chunk(max_len)


def test_batch_one_fills_the_chip():
    # 12 heads x 4096 rows: the smallest automatic chunk (64 rows) gives 12 * 64 waves,
    # three per CU.
    chunk, n = ea.decode_choose_split(1, 12, 4096, 64, 256)
    assert (chunk, n) == (64, 64)
    assert 12 * n >= 256


def test_batch_eight():
    assert ea.decode_choose_split(8, 12, 4096, 64, 256) == (192, 22)


def test_more_cus_never_larger_chunks():
    prev = None
    for cus in (32, 64, 82, 128, 256, 304):
        c, _ = ea.decode_choose_split(1, 12, 4096, 64, cus)
        assert prev is None or c <= prev
        prev = c


@pytest.mark.parametrize("bad", [dict(B=0), dict(H=0), dict(max_len=0), dict(cus=0), dict(d=48)])
def test_chooser_rejects(bad):
    a = dict(B=1, H=1, max_len=10, d=64, cus=10)
    a.update(bad)
    with pytest.raises(ValueError):
        ea.decode_choose_split(a["B"], a["H"], a["max_len"], a["d"], a["cus"])


def test_binding_constants_match_header():
    import os
    import re

    hdr = open(os.path.join(os.path.dirname(__file__), "..", "include", "attn.h")).read()
    defs = dict(re.findall(r"#define (ATTN_DECODE_\w+) (\d+)", hdr))
    assert int(defs["ATTN_DECODE_ROW_GRANULE"]) == ea.DECODE_ROW_GRANULE
    assert int(defs["ATTN_DECODE_WGS_PER_CU"]) == ea.DECODE_WGS_PER_CU
    assert int(defs["ATTN_DECODE_MIN_CHUNK"]) == ea.DECODE_MIN_CHUNK
