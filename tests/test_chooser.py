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
    assert int(defs["ATTN_DECODE_MFMA_LDS_BYTES"]) == ea.DECODE_MFMA_LDS_BYTES


def split_rule(cols, max_len, target):
    """The documented rule, written out: n = ceil(target / cols) clamped to what the
    smallest chunk allows, chunk = ceil(max_len / n) rounded up to the granule (at least
    the smallest chunk), then shrunk one granule at a time while the split count is
    short of the target."""
    cmin = min_chunk(max_len)
    n = max(1, -(-target // cols))
    n = min(n, -(-max_len // cmin))
    c = max(cmin, -(-(-(-max_len // n)) // G) * G)
    while c - G >= cmin and cols * (-(-max_len // c)) < target:
        c -= G
    return c, -(-max_len // c)


@pytest.mark.parametrize("B,H,max_len,cus", list(itertools.product([1, 8, 64], [1, 12, 32], [100, 4096, 65536], [82, 256])))
def test_rule_matches_library(B, H, max_len, cus):
    assert ea.decode_choose_split(B, H, max_len, 64, cus) == split_rule(B * H, max_len, WGS_PER_CU * cus)


def mfma_waves_per_cu(d):
    pitch = {32: 128, 64: 128, 96: 256, 128: 256, 256: 512}[d]
    return ea.DECODE_MFMA_LDS_BYTES // (4 * 32 * pitch)


@pytest.mark.parametrize("d", [32, 64, 96, 128, 256])
@pytest.mark.parametrize("B,Hq,Hkv", [(8, 32, 8), (1, 32, 8), (8, 12, 4), (4, 64, 2), (2, 96, 3)])
def test_grouped_matrix_core_target(B, Hq, Hkv, d):
    """Groups of 3..32 heads: one wave column per K/V head, aiming at the waves whose
    LDS tiles fit on a CU (10, 5 or 2)."""
    assert 3 <= Hq // Hkv <= 32
    assert mfma_waves_per_cu(d) == {32: 10, 64: 10, 96: 5, 128: 5, 256: 2}[d]
    got = ea.decode_gqa_choose_split(B, Hq, Hkv, 4096, d, 256)
    assert got == split_rule(B * Hkv, 4096, mfma_waves_per_cu(d) * 256)


def test_grouped_headline_chunk():
    # 8 sequences, 32 query heads over 8 K/V heads of 128: 64 columns aiming at 1280
    # waves give 192-row chunks (22 splits), the fastest chunk measured for it.
    assert ea.decode_gqa_choose_split(8, 32, 8, 4096, 128, 256) == (192, 22)
