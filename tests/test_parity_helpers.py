"""The sampled gradient bounds used at large sizes equal the full ones on small inputs."""

import numpy as np

import oracle
from parity import backward_bounds, backward_bounds_keys, backward_bounds_rows


def test_sampled_bounds_match_full():
    r = np.random.default_rng(7)
    B, Hq, Hkv, N, d = 2, 4, 2, 70, 5
    q, do = r.standard_normal((B, Hq, N, d)), r.standard_normal((B, Hq, N, d))
    k, v = r.standard_normal((B, Hkv, N, d)), r.standard_normal((B, Hkv, N, d))
    rows = [0, 31, 32, 69]
    for causal in (False, True):
        lse = oracle.prefill_lse(q, k, causal, 0.4)
        bq, bk, bv = backward_bounds(q, k, v, do, causal, 0.4, lse)
        for h in (0, 3):
            assert np.allclose(backward_bounds_rows(q, k, v, do, causal, 0.4, 1, h, rows), bq[1, h, rows],
                               rtol=1e-12, atol=0)
        for kv in (0, 1):
            sk, sv = backward_bounds_keys(q, k, v, do, causal, 0.4, 1, kv, rows, block=32)
            assert np.allclose(sk, bk[1, kv, rows], rtol=1e-12, atol=0)
            assert np.allclose(sv, bv[1, kv, rows], rtol=1e-12, atol=0)
