"""Checks that pin the fp64 oracle to facts outside itself.

Each pin takes an oracle namespace (``prefill``, ``prefill_rows``, ``decode``,
``decode_split``) and raises AssertionError when the oracle disagrees with the
pages or with the mathematics: brute force on tiny inputs, closed forms, the
worked weights printed on page 3, invariants of the definition, and the
equalities page 3 states (decode row t equals prefill row t; every split size
gives the same decode output).  The same pins run against deliberately broken
copies of the oracle (tests/test_oracle_mutants.py) to show each planted
mistake is caught.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np

import brute_force

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _bf(x):
    return np.asarray(x, dtype=np.float64).tolist()


def pin_brute_force_prefill(O):
    """Oracle prefill equals pure-Python brute force for N <= 16, d in {1, 2, 4, 64}."""
    for seed, (B, H, N, d) in enumerate([(1, 1, 1, 1), (1, 2, 5, 2), (2, 1, 9, 4), (1, 1, 16, 64), (1, 3, 7, 3)]):
        r = _rng(seed)
        q, k, v = (r.standard_normal((B, H, N, d)) for _ in range(3))
        for causal in (False, True):
            scale = 0.37 + 0.1 * seed
            got = O.prefill(q, k, v, causal, scale)
            ref = np.array(brute_force.prefill(_bf(q), _bf(k), _bf(v), causal, scale))
            assert np.max(np.abs(got - ref)) <= 1e-13, (B, H, N, d, causal)


def pin_brute_force_decode(O):
    """Oracle decode equals brute force for every cache length L <= N."""
    r = _rng(7)
    B, H, N, d = 2, 2, 12, 4
    q = r.standard_normal((B, H, 1, d))
    kc, vc = r.standard_normal((B, H, N, d)), r.standard_normal((B, H, N, d))
    for L in range(1, N + 1):
        lens = [L, N + 1 - L]
        got = O.decode(q, kc, vc, lens, 0.5)
        ref = np.array(brute_force.decode(_bf(q), _bf(kc), _bf(vc), lens, 0.5))
        assert np.max(np.abs(got - ref)) <= 1e-13, L


def pin_students_example(O):
    """Page 3's worked weights (10/20/50/20 %) reproduce as the output with one-hot values."""
    with open(os.path.join(GOLDEN, "students_weights.json")) as f:
        g = json.load(f)
    w = np.array(g["weights"])
    n = len(w)
    q = np.zeros((1, 1, 1, n))
    q[0, 0, 0, 0] = 1.0
    kc = np.zeros((1, 1, n, n))
    kc[0, 0, :, 0] = np.log(w)
    vc = np.eye(n)[None, None]
    out = O.decode(q, kc, vc, [n], 1.0)[0, 0, 0]
    assert np.max(np.abs(out - np.array(g["expected_output"]))) <= g["tolerance"], out


def pin_zero_query_is_mean(O):
    """Q = 0 (or scale = 0): uniform weights, so full rows are the column mean of V,
    causal row i is the mean of V[0..i], decode is the mean of the first L rows."""
    r = _rng(11)
    B, H, N, d = 2, 2, 33, 8
    k, v = r.standard_normal((B, H, N, d)), r.standard_normal((B, H, N, d))
    q0 = np.zeros((B, H, N, d))
    qr = r.standard_normal((B, H, N, d))
    prefix_mean = np.cumsum(v, axis=2) / np.arange(1, N + 1)[None, None, :, None]
    for q, scale in ((q0, 0.125), (qr, 0.0)):
        full = O.prefill(q, k, v, False, scale)
        assert np.max(np.abs(full - v.mean(axis=2, keepdims=True))) <= 1e-14
        causal = O.prefill(q, k, v, True, scale)
        assert np.max(np.abs(causal - prefix_mean)) <= 1e-14
    lens = [5, 33]
    dec = O.decode(np.zeros((B, H, 1, d)), k, v, lens, 0.3)
    for b, L in enumerate(lens):
        assert np.max(np.abs(dec[b, :, 0] - v[b, :, :L].mean(axis=1))) <= 1e-14


def pin_causal_row0_and_decode_len1(O):
    """Causal row 0 sees only key 0, so it is V[0] exactly; decode with L = 1 is v_cache[0]."""
    r = _rng(12)
    q, k, v = (r.standard_normal((1, 3, 10, 16)) for _ in range(3))
    out = O.prefill(q, k, v, True, 0.9)
    assert np.array_equal(out[:, :, 0], v[:, :, 0])
    dec = O.decode(q[:, :, :1], k, v, [1], 0.9)
    assert np.array_equal(dec[:, :, 0], v[:, :, 0])


def pin_constant_values(O):
    """All value rows equal to w: any weights that sum to one return w."""
    r = _rng(13)
    B, H, N, d = 1, 2, 20, 6
    q, k = r.standard_normal((B, H, N, d)), r.standard_normal((B, H, N, d))
    w = r.standard_normal(d)
    v = np.broadcast_to(w, (B, H, N, d)).copy()
    for causal in (False, True):
        out = O.prefill(q, k, v, causal, 0.7)
        assert np.max(np.abs(out - w)) <= 1e-14


def pin_two_level_closed_form(O):
    """One-hot q and k give score a on key j* and 0 elsewhere over n keys:
    O = (e^a v_j* + sum_{j != j*} v_j) / (e^a + n - 1)."""
    r = _rng(14)
    n, d, jstar, a_raw, scale = 9, 9, 4, 3.0, 0.5
    q = np.zeros((1, 1, n, d))
    q[0, 0, :, 0] = a_raw
    k = np.zeros((1, 1, n, d))
    k[0, 0, jstar, 0] = 1.0
    v = r.standard_normal((1, 1, n, d))
    a = scale * a_raw
    expect = (math.exp(a) * v[0, 0, jstar] + (v[0, 0].sum(axis=0) - v[0, 0, jstar])) / (math.exp(a) + n - 1)
    out = O.prefill(q, k, v, False, scale)
    assert np.max(np.abs(out[0, 0] - expect)) <= 1e-14
    # causal row i >= j* sees keys 0..i: the same form with n = i + 1
    outc = O.prefill(q, k, v, True, scale)
    for i in range(jstar, n):
        vi = v[0, 0, : i + 1]
        e = (math.exp(a) * v[0, 0, jstar] + (vi.sum(axis=0) - v[0, 0, jstar])) / (math.exp(a) + i)
        assert np.max(np.abs(outc[0, 0, i] - e)) <= 1e-14
    for i in range(jstar):
        assert np.max(np.abs(outc[0, 0, i] - v[0, 0, : i + 1].mean(axis=0))) <= 1e-14


def pin_large_separated_scores(O):
    """Scores far apart (here ~1e4) put all weight on the largest; no overflow to NaN."""
    r = _rng(15)
    N, d = 12, 4
    q = np.zeros((1, 1, N, d))
    q[..., 0] = 100.0
    k = np.zeros((1, 1, N, d))
    k[0, 0, :, 0] = np.arange(N) * 100.0  # key N-1 dominates every non-causal row
    v = r.standard_normal((1, 1, N, d))
    out = O.prefill(q, k, v, False, 1.0)
    assert np.all(np.isfinite(out))
    assert np.max(np.abs(out[0, 0] - v[0, 0, N - 1])) <= 1e-14
    outc = O.prefill(q, k, v, True, 1.0)
    assert np.max(np.abs(outc[0, 0] - v[0, 0])) <= 1e-14  # row i's largest visible key is i
    dec = O.decode(q[:, :, :1], k, v, [5], 1.0)
    assert np.max(np.abs(dec[0, 0, 0] - v[0, 0, 4])) <= 1e-14


def pin_key_shift_invariance(O):
    """K + 1 u^T adds q_i . u to every score of row i: weights, hence O, unchanged."""
    r = _rng(16)
    q, k, v = (r.standard_normal((2, 2, 24, 8)) for _ in range(3))
    u = r.standard_normal(8)
    for causal in (False, True):
        a = O.prefill(q, k, v, causal, 0.4)
        b = O.prefill(q, k + u, v, causal, 0.4)
        assert np.max(np.abs(a - b)) <= 1e-12


def pin_value_shift(O):
    """V + 1 w^T gives O + w, because the weights sum to one."""
    r = _rng(17)
    q, k, v = (r.standard_normal((1, 2, 24, 8)) for _ in range(3))
    w = r.standard_normal(8)
    for causal in (False, True):
        a = O.prefill(q, k, v, causal, 0.4)
        b = O.prefill(q, k, v + w, causal, 0.4)
        assert np.max(np.abs((a + w) - b)) <= 1e-12


def pin_permutation_equivariance(O):
    """Full attention: permuting K and V rows together changes nothing; permuting Q rows permutes O."""
    r = _rng(18)
    q, k, v = (r.standard_normal((1, 2, 20, 8)) for _ in range(3))
    perm = r.permutation(20)
    a = O.prefill(q, k, v, False, 0.6)
    b = O.prefill(q, k[:, :, perm], v[:, :, perm], False, 0.6)
    assert np.max(np.abs(a - b)) <= 1e-12
    c = O.prefill(q[:, :, perm], k, v, False, 0.6)
    assert np.max(np.abs(a[:, :, perm] - c)) <= 1e-14


def pin_last_causal_row_is_full_row(O):
    r = _rng(19)
    q, k, v = (r.standard_normal((2, 2, 17, 8)) for _ in range(3))
    a = O.prefill(q, k, v, False, 0.5)
    b = O.prefill(q, k, v, True, 0.5)
    assert np.max(np.abs(a[:, :, -1] - b[:, :, -1])) <= 1e-14


def pin_causality(O):
    """Changing K, V rows after i leaves causal row i bit-identical."""
    r = _rng(20)
    q, k, v = (r.standard_normal((1, 1, 30, 8)) for _ in range(3))
    a = O.prefill(q, k, v, True, 0.5)
    for i in (0, 7, 28):
        k2, v2 = k.copy(), v.copy()
        k2[:, :, i + 1 :] = r.standard_normal(k2[:, :, i + 1 :].shape)
        v2[:, :, i + 1 :] = 1e3
        b = O.prefill(q, k2, v2, True, 0.5)
        assert np.array_equal(a[:, :, : i + 1], b[:, :, : i + 1])


def pin_decode_equals_prefill_row(O):
    """Page 3: decoding token t from the cache equals row t of causal prefill."""
    r = _rng(21)
    B, H, N, d = 2, 3, 40, 16
    q, k, v = (r.standard_normal((B, H, N, d)) for _ in range(3))
    pre = O.prefill(q, k, v, True, 0.25)
    for t in (0, 1, 17, 39):
        dec = O.decode(q[:, :, t : t + 1], k, v, [t + 1] * B, 0.25)
        assert np.max(np.abs(dec[:, :, 0] - pre[:, :, t])) <= 1e-12


def pin_prefill_rows_matches_prefill(O):
    r = _rng(22)
    q, k, v = (r.standard_normal((2, 2, 50, 8)) for _ in range(3))
    for causal in (False, True):
        full = O.prefill(q, k, v, causal, 0.3)
        rows = [0, 3, 49, 20]
        part = O.prefill_rows(q, k, v, causal, 0.3, 1, 1, rows)
        assert np.max(np.abs(part - full[1, 1, rows])) <= 1e-14


def pin_split_invariance(O):
    """Page 3: every legal chunk size gives the same decode output (to fp64 rounding)."""
    r = _rng(23)
    B, H, N, d = 2, 2, 37, 8
    q = r.standard_normal((B, H, 1, d)) * 2.0
    kc, vc = r.standard_normal((B, H, N, d)), r.standard_normal((B, H, N, d))
    lens = [37, 23]
    base = O.decode(q, kc, vc, lens, 0.7)
    for C in range(1, N + 1):
        got = O.decode_split(q, kc, vc, lens, 0.7, C)
        assert np.max(np.abs(got - base)) <= 1e-12, C


def pin_library_sdpa(O):
    """Special case that reduces to a library routine: torch SDPA in fp64 on the CPU."""
    import torch

    r = _rng(24)
    q, k, v = (r.standard_normal((2, 3, 70, 32)) for _ in range(3))
    for causal in (False, True):
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), is_causal=causal, scale=0.2
        ).numpy()
        got = O.prefill(q, k, v, causal, 0.2)
        assert np.max(np.abs(got - ref)) <= 1e-12


def pin_grouped_heads_brute_force(O):
    """Grouped K/V heads: the oracle agrees with brute force, which builds each query
    head's K/V by repeating every K/V head for its group."""
    r = _rng(30)
    for (B, Hq, Hkv, N, d) in [(1, 6, 2, 7, 3), (2, 4, 1, 5, 2), (1, 3, 3, 6, 4)]:
        q = r.standard_normal((B, Hq, N, d))
        k, v = r.standard_normal((B, Hkv, N, d)), r.standard_normal((B, Hkv, N, d))
        for causal in (False, True):
            got = O.prefill(q, k, v, causal, 0.6)
            ref = np.array(brute_force.prefill(_bf(q), _bf(k), _bf(v), causal, 0.6))
            assert np.max(np.abs(got - ref)) <= 1e-13, (Hq, Hkv, causal)
    q = r.standard_normal((2, 8, 1, 4))
    kc, vc = r.standard_normal((2, 2, 9, 4)), r.standard_normal((2, 2, 9, 4))
    for lens in ([9, 1], [4, 7]):
        got = O.decode(q, kc, vc, lens, 0.8)
        ref = np.array(brute_force.decode(_bf(q), _bf(kc), _bf(vc), lens, 0.8))
        assert np.max(np.abs(got - ref)) <= 1e-13, lens


def pin_grouped_heads_are_repeated_heads(O):
    """Grouped K/V heads equal ordinary multi-head attention on K/V whose heads are
    each repeated for their group, in prefill, row-sampled prefill, decode and split
    decode."""
    r = _rng(31)
    B, Hq, Hkv, N, d = 2, 6, 3, 40, 8
    g = Hq // Hkv
    q = r.standard_normal((B, Hq, N, d))
    k, v = r.standard_normal((B, Hkv, N, d)), r.standard_normal((B, Hkv, N, d))
    kr, vr = np.repeat(k, g, axis=1), np.repeat(v, g, axis=1)
    for causal in (False, True):
        a = O.prefill(q, k, v, causal, 0.4)
        assert np.max(np.abs(a - O.prefill(q, kr, vr, causal, 0.4))) <= 1e-14
        rows = [0, 17, 39]
        for h in (0, 3, 5):
            part = O.prefill_rows(q, k, v, causal, 0.4, 1, h, rows)
            assert np.max(np.abs(part - a[1, h, rows])) <= 1e-14
    qd = r.standard_normal((B, Hq, 1, d))
    lens = [40, 13]
    base = O.decode(qd, k, v, lens, 0.4)
    assert np.max(np.abs(base - O.decode(qd, kr, vr, lens, 0.4))) <= 1e-14
    for C in (1, 7, 40):
        assert np.max(np.abs(O.decode_split(qd, k, v, lens, 0.4, C) - base)) <= 1e-12, C


def pin_grouped_heads_library_sdpa(O):
    """Library special case for grouped heads: torch SDPA with enable_gqa, fp64 on the CPU."""
    import torch

    r = _rng(32)
    q = r.standard_normal((2, 8, 33, 16))
    k, v = r.standard_normal((2, 2, 33, 16)), r.standard_normal((2, 2, 33, 16))
    for causal in (False, True):
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), is_causal=causal, scale=0.3, enable_gqa=True
        ).numpy()
        got = O.prefill(q, k, v, causal, 0.3)
        assert np.max(np.abs(got - ref)) <= 1e-12


def pin_lse_brute_force(O):
    """Row log-sum-exp equals brute force (exact sums), multi-head and grouped heads."""
    r = _rng(40)
    for (B, Hq, Hkv, N, d) in [(1, 2, 2, 9, 4), (2, 4, 2, 6, 3), (1, 3, 1, 16, 8)]:
        q = r.standard_normal((B, Hq, N, d)) * 1.5
        k = r.standard_normal((B, Hkv, N, d))
        for causal in (False, True):
            got = O.prefill_lse(q, k, causal, 0.7)
            ref = np.array(brute_force.prefill_lse(_bf(q), _bf(k), causal, 0.7))
            assert np.max(np.abs(got - ref)) <= 1e-13, (Hq, Hkv, causal)


def pin_lse_closed_forms(O):
    """Q = 0: every visible key weighs 1, so lse = log(number of visible keys): log N
    for full rows, log(i + 1) for causal row i.  Causal row 0 sees key 0 alone:
    lse = scale q_0 . k_0.  One-hot q and k giving score a on one key and 0 on the
    other n - 1: lse = log(e^a + n - 1)."""
    r = _rng(41)
    B, H, N, d = 1, 2, 11, 5
    k = r.standard_normal((B, H, N, d))
    q0 = np.zeros((B, H, N, d))
    assert np.max(np.abs(O.prefill_lse(q0, k, False, 0.9) - np.log(N))) <= 1e-14
    assert np.max(np.abs(O.prefill_lse(q0, k, True, 0.9) - np.log(np.arange(1, N + 1))[None, None])) <= 1e-14
    q = r.standard_normal((B, H, N, d))
    got = O.prefill_lse(q, k, True, 0.9)[:, :, 0]
    assert np.max(np.abs(got - 0.9 * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]))) <= 1e-14
    n, a = 7, 2.5
    q1 = np.zeros((1, 1, 1, n))
    q1[0, 0, 0, 0] = 1.0
    k1 = np.zeros((1, 1, n, n))
    k1[0, 0, 3, 0] = a
    # a single query row against n keys: pad q to n rows and read row n - 1 of the full form
    qn = np.repeat(q1, n, axis=2)
    got = O.prefill_lse(qn, k1, False, 1.0)[0, 0, n - 1]
    assert abs(got - math.log(math.exp(a) + n - 1)) <= 1e-14


def pin_lse_reconstructs_output(O):
    """The output row is sum_j exp(scale q_i . k_j - lse_i) v_j (the normaliser the
    definition divides by), for full and causal rows."""
    r = _rng(42)
    B, H, N, d = 2, 2, 30, 6
    q, k, v = (r.standard_normal((B, H, N, d)) for _ in range(3))
    for causal in (False, True):
        lse = O.prefill_lse(q, k, causal, 0.5)
        s = 0.5 * np.einsum("bhid,bhjd->bhij", q, k)
        if causal:
            s = np.where(np.tril(np.ones((N, N), dtype=bool))[None, None], s, -np.inf)
        recon = np.einsum("bhij,bhjd->bhid", np.exp(s - lse[..., None]), v)
        assert np.max(np.abs(recon - O.prefill(q, k, v, causal, 0.5))) <= 1e-12


def pin_lse_rows_matches_lse(O):
    """Row-sampled log-sum-exp equals the full one (grouped heads, both masks)."""
    r = _rng(43)
    q = r.standard_normal((2, 4, 40, 8))
    k = r.standard_normal((2, 2, 40, 8))
    for causal in (False, True):
        full = O.prefill_lse(q, k, causal, 0.6)
        rows = [0, 5, 39, 17]
        for h in (0, 1, 3):
            part = O.prefill_lse_rows(q, k, causal, 0.6, 1, h, rows)
            assert np.max(np.abs(part - full[1, h, rows])) <= 1e-14


def pin_backward_finite_differences(O):
    """The gradients equal central finite differences of sum(dO * prefill(...)) on tiny
    inputs, for every element of q, k and v (multi-head and grouped, both masks)."""
    r = _rng(50)
    eps = 1e-6
    for (Hq, Hkv) in ((2, 2), (2, 1)):
        q = r.standard_normal((1, Hq, 4, 3))
        k, v = r.standard_normal((1, Hkv, 4, 3)), r.standard_normal((1, Hkv, 4, 3))
        do = r.standard_normal((1, Hq, 4, 3))
        for causal in (False, True):
            grads = O.backward(q, k, v, do, causal, 0.8)
            for which, x in enumerate((q, k, v)):
                num = np.zeros_like(x)
                for idx in np.ndindex(x.shape):
                    xp, xm = x.copy(), x.copy()
                    xp[idx] += eps
                    xm[idx] -= eps
                    args_p = [q, k, v]
                    args_m = [q, k, v]
                    args_p[which], args_m[which] = xp, xm
                    lp = np.sum(do * O.prefill(*args_p, causal, 0.8))
                    lm = np.sum(do * O.prefill(*args_m, causal, 0.8))
                    num[idx] = (lp - lm) / (2 * eps)
                assert np.max(np.abs(grads[which] - num)) <= 1e-7, (Hq, Hkv, causal, which)


def pin_backward_library_autograd(O):
    """Library special case: torch autograd through SDPA in fp64 on the CPU
    (enable_gqa for grouped heads)."""
    import torch

    r = _rng(51)
    for (Hq, Hkv) in ((3, 3), (4, 2)):
        q = r.standard_normal((2, Hq, 37, 8))
        k, v = r.standard_normal((2, Hkv, 37, 8)), r.standard_normal((2, Hkv, 37, 8))
        do = r.standard_normal((2, Hq, 37, 8))
        for causal in (False, True):
            Q, K, V = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
            out = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=causal, scale=0.45,
                                                                   enable_gqa=Hq != Hkv)
            (out * torch.from_numpy(do)).sum().backward()
            dq, dk, dv = O.backward(q, k, v, do, causal, 0.45)
            for got, ref in ((dq, Q.grad), (dk, K.grad), (dv, V.grad)):
                assert np.max(np.abs(got - ref.numpy())) <= 1e-12, (Hq, Hkv, causal)


def pin_backward_invariants(O):
    """Each softmax row sums to one, so the V gradients sum to the dO rows (full and
    causal); shifting every key by one vector leaves all gradients unchanged (the rows
    of dS sum to zero); a zero scale gives zero dQ and dK; with causal masking, a dO
    that only touches row 0 reaches key 0 alone."""
    r = _rng(52)
    B, H, N, d = 2, 2, 20, 5
    q, k, v, do = (r.standard_normal((B, H, N, d)) for _ in range(4))
    for causal in (False, True):
        dq, dk, dv = O.backward(q, k, v, do, causal, 0.7)
        assert np.max(np.abs(dv.sum(axis=2) - do.sum(axis=2))) <= 1e-12
        u = r.standard_normal(d)
        g2 = O.backward(q, k + u, v, do, causal, 0.7)
        for a, b in zip((dq, dk, dv), g2):
            assert np.max(np.abs(a - b)) <= 1e-11
        z = O.backward(q, k, v, do, causal, 0.0)
        assert np.max(np.abs(z[0])) == 0.0 and np.max(np.abs(z[1])) == 0.0
    do0 = np.zeros_like(do)
    do0[:, :, 0] = do[:, :, 0]
    _, dk0, dv0 = O.backward(q, k, v, do0, True, 0.7)
    assert np.max(np.abs(dk0[:, :, 1:])) == 0.0 and np.max(np.abs(dv0[:, :, 1:])) == 0.0
    assert np.max(np.abs(dv0[:, :, 0] - do[:, :, 0])) <= 1e-14


def pin_backward_grouped_heads(O):
    """Grouped heads: dQ equals multi-head dQ on repeated K/V, and dK, dV equal the
    repeated-head gradients summed over each group."""
    r = _rng(53)
    B, Hq, Hkv, N, d = 1, 6, 2, 15, 4
    g = Hq // Hkv
    q, do = r.standard_normal((B, Hq, N, d)), r.standard_normal((B, Hq, N, d))
    k, v = r.standard_normal((B, Hkv, N, d)), r.standard_normal((B, Hkv, N, d))
    for causal in (False, True):
        dq, dk, dv = O.backward(q, k, v, do, causal, 0.5)
        rq, rk, rv = O.backward(q, np.repeat(k, g, axis=1), np.repeat(v, g, axis=1), do, causal, 0.5)
        assert np.max(np.abs(dq - rq)) <= 1e-13
        assert np.max(np.abs(dk - rk.reshape(B, Hkv, g, N, d).sum(axis=2))) <= 1e-13
        assert np.max(np.abs(dv - rv.reshape(B, Hkv, g, N, d).sum(axis=2))) <= 1e-13


def pin_backward_sampled_matches_backward(O):
    """Row-sampled dq and key-row-sampled dk, dv equal the full backward (grouped heads,
    both masks, more query rows than one block of rows)."""
    r = _rng(54)
    B, Hq, Hkv, N, d = 2, 4, 2, 1100, 3
    q, do = r.standard_normal((B, Hq, N, d)), r.standard_normal((B, Hq, N, d))
    k, v = r.standard_normal((B, Hkv, N, d)), r.standard_normal((B, Hkv, N, d))
    rows = [0, 1, 517, 1023, 1024, 1099]
    for causal in (False, True):
        dq, dk, dv = O.backward(q, k, v, do, causal, 0.6)
        for h in (0, 3):
            part = O.backward_dq_rows(q, k, v, do, causal, 0.6, 1, h, rows)
            assert np.max(np.abs(part - dq[1, h, rows])) <= 1e-13, (causal, h)
        for g in (0, 1):
            pk, pv = O.backward_dkdv_rows(q, k, v, do, causal, 0.6, 1, g, rows)
            assert np.max(np.abs(pk - dk[1, g, rows])) <= 1e-12, (causal, g)
            assert np.max(np.abs(pv - dv[1, g, rows])) <= 1e-12, (causal, g)


PINS = [
    pin_brute_force_prefill,
    pin_brute_force_decode,
    pin_students_example,
    pin_zero_query_is_mean,
    pin_causal_row0_and_decode_len1,
    pin_constant_values,
    pin_two_level_closed_form,
    pin_large_separated_scores,
    pin_key_shift_invariance,
    pin_value_shift,
    pin_permutation_equivariance,
    pin_last_causal_row_is_full_row,
    pin_causality,
    pin_decode_equals_prefill_row,
    pin_prefill_rows_matches_prefill,
    pin_split_invariance,
    pin_library_sdpa,
    pin_grouped_heads_brute_force,
    pin_grouped_heads_are_repeated_heads,
    pin_grouped_heads_library_sdpa,
    pin_lse_brute_force,
    pin_lse_closed_forms,
    pin_lse_reconstructs_output,
    pin_lse_rows_matches_lse,
    pin_backward_finite_differences,
    pin_backward_library_autograd,
    pin_backward_invariants,
    pin_backward_grouped_heads,
    pin_backward_sampled_matches_backward,
]
