"""Host-side checks of the prefill launch rule (attn_prefill_plan; no GPU needed):
every form the rule can select on a 256-CU device is reached by a case of
tests/test_forms_gpu.py, each case is listed with the form it takes, and the rule's
documented boundaries hold."""

import itertools

import exact_attention_prefill_amd as ea
from test_forms_gpu import CUS, FORM_CASES, case_id, plan_of


def reachable_forms():
    """(d, causal, form) over a scan of grid sizes and lengths around every threshold."""
    bhs = sorted({1, 2, 3, 4, 6, 8, 12, 16, 24, 32, 40, 48, 64, 96, 128, 160, 256, 512, 1024, 4096})
    ns = sorted({1, 31, 64, 100, 128, 129, 255, 256, 257, 1000, 2047, 2048, 2049, 4095, 4096, 4097, 6143, 6144,
                 6145, 8191, 8192, 8193, 12287, 12288, 12289, 16384, 16385, 32768, 65536})
    found = set()
    for d, causal, bh, n in itertools.product((32, 64, 96, 128, 256), (False, True), bhs, ns):
        p = ea.prefill_plan(1, bh, n, d, causal, CUS)
        found.add((d, causal, (p["waves"], p["rows_per_wave"], p["stages"], p["key_groups"])))
    return found


def test_every_case_takes_its_listed_form():
    for c in FORM_CASES:
        assert plan_of(c) == c["form"], (case_id(c), plan_of(c))


def test_cases_reach_every_form():
    reached = {(c["d"], c["causal"], c["form"]) for c in FORM_CASES}
    missing = reachable_forms() - reached
    assert not missing, sorted(missing)


def test_rule_boundaries():
    # The headline shape (B=1, H=16, N=16384, d=128, full) runs eight waves of one
    # 32-row block each, two stages; d = 64 there runs two blocks per wave.
    P = lambda *a: ea.prefill_plan(*a)  # noqa: E731
    assert P(1, 16, 16384, 128, False, 256) == {"waves": 8, "rows_per_wave": 32, "stages": 2, "key_groups": 1}
    assert P(1, 16, 16384, 64, False, 256) == {"waves": 8, "rows_per_wave": 64, "stages": 4, "key_groups": 1}
    # The GPT-2-like prompt (B=1, H=12, N=2048, d=64: 192 128-row blocks on 256 CUs) splits
    # each block's keys: two groups full, four causal (64-row blocks).
    assert P(1, 12, 2048, 64, False, 256) == {"waves": 8, "rows_per_wave": 32, "stages": 2, "key_groups": 2}
    assert P(1, 12, 2048, 64, True, 256) == {"waves": 8, "rows_per_wave": 32, "stages": 2, "key_groups": 4}
    # Key groups stop above one 128-row block per CU.
    assert P(1, 2, 128 * 128, 128, False, 256)["key_groups"] == 2
    assert P(1, 2, 128 * 128 + 1, 128, False, 256)["key_groups"] == 1
    # d = 256 always runs four waves, two stages, one key group.
    for n in (1, 5000, 40000):
        assert P(1, 64, n, 256, True, 256) == {"waves": 4, "rows_per_wave": 32, "stages": 2, "key_groups": 1}
