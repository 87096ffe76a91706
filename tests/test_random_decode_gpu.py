"""Decode on seeded random shapes: batch, query heads over K/V heads (which select the
multi-head form, the grouped form on the vector ALUs, or the grouped form on the
matrix cores), head size, dtype, cache length and ragged lengths.

Every case is checked in full against the fp64 oracle with the automatic split, and
again with a smaller split of the rows (the result may not depend on the split beyond
the gate).
"""

import numpy as np
import pytest
import torch

import exact_attention_prefill_amd as ea
import oracle
import workloads as W
from parity import check, f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _cases(n=16, seed=20261204):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        d = int(rng.choice([32, 64, 96, 128, 256]))
        dtype = str(rng.choice(["f16", "bf16"]))
        Hkv = int(rng.choice([1, 2, 4, 8]))
        g = int(rng.choice([1, 1, 2, 3, 4, 8]))
        B = int(rng.integers(1, 17))
        max_len = int(rng.choice([int(rng.integers(1, 200)), int(rng.integers(200, 3000)),
                                  int(rng.integers(3000, 9000))]))
        max_len = max(1, min(max_len, (1 << 24) // (B * Hkv * d)))  # caches of at most 16M elements
        lens = rng.integers(1, max_len + 1, size=B).tolist()
        scale = float(rng.choice([1 / np.sqrt(d), 0.125, -0.4]))
        out.append((i, B, Hkv * g, Hkv, max_len, d, dtype, scale, lens))
    return out


CASES = _cases()


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"c{c[0]}_B{c[1]}_H{c[2]}_Hkv{c[3]}_L{c[4]}_d{c[5]}_{c[6]}")
def test_random_decode(case):
    i, B, H, Hkv, max_len, d, dtype, scale, lens = case
    q, k, v, sl = W.decode_inputs_gqa(B, H, Hkv, max_len, d, dtype, seed=200 + i, seq_lens=lens)
    qd, kd, vd, sld = (t.to(DEV) for t in (q, k, v, sl))
    out = ea.decode(qd, kd, vd, sld, scale=scale)
    torch.cuda.synchronize()
    ref = oracle.decode(f64(q), f64(k), f64(v), np.asarray(lens), scale)
    check(f64(out), ref, dtype, f"decode case {case[:8]}")
    chunk = 64 if max_len > 64 else 32  # a multiple of the 32-row granule, at most max_len rounded up
    ns = -(-max_len // chunk)
    ws = torch.empty(ea.decode_workspace_bytes(B, H, ns, d), dtype=torch.uint8, device=DEV)
    out2 = ea.decode(qd, kd, vd, sld, scale=scale, chunk=chunk, workspace=ws)
    torch.cuda.synchronize()
    check(f64(out2), ref, dtype, f"decode case {case[:8]} chunk={chunk}")
