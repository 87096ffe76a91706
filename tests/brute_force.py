"""Pure-Python brute-force attention on tiny inputs (N <= 16).

An independent second computation of the definition used to pin the oracle:
plain loops, exactly rounded sums (math.fsum) and math.exp, no NumPy.  Page 3,
"What is Attention?": scores against every visible key, weights that sum to one,
weighted combination of the values.
"""

import math


def _attend(qrow, krows, vrows, scale):
    scores = [scale * math.fsum(a * b for a, b in zip(qrow, kr)) for kr in krows]
    top = max(scores)
    w = [math.exp(s - top) for s in scores]
    total = math.fsum(w)
    d = len(vrows[0])
    return [math.fsum(w[j] * vrows[j][c] for j in range(len(vrows))) / total for c in range(d)]


def _expand(heads, hq):
    """The K/V heads a query-head list of length hq reads: each of the Hkv heads
    serves the next run of hq // Hkv query heads (grouped-query attention served by
    repeating every K/V head for its group)."""
    group = hq // len(heads)
    assert group * len(heads) == hq
    return [kvh for kvh in heads for _ in range(group)]


def prefill(q, k, v, causal, scale):
    """q [B][H][N][d], k and v [B][Hkv][N][d] nested lists; returns [B][H][N][d]."""
    out = []
    for qb, kb, vb in zip(q, k, v):
        ob = []
        for qh, kh, vh in zip(qb, _expand(kb, len(qb)), _expand(vb, len(qb))):
            oh = []
            for i, qrow in enumerate(qh):
                n = i + 1 if causal else len(kh)
                oh.append(_attend(qrow, kh[:n], vh[:n], scale))
            ob.append(oh)
        out.append(ob)
    return out


def decode(q, k_cache, v_cache, seq_lens, scale):
    """q [B][H][1][d], caches [B][Hkv][max_len][d]; returns [B][H][1][d]."""
    out = []
    for b, (qb, kb, vb) in enumerate(zip(q, k_cache, v_cache)):
        L = int(seq_lens[b])
        out.append([[_attend(qh[0], kh[:L], vh[:L], scale)]
                    for qh, kh, vh in zip(qb, _expand(kb, len(qb)), _expand(vb, len(qb)))])
    return out


def prefill_lse(q, k, causal, scale):
    """Row log-sum-exp, natural log: log of the exactly rounded sum of exp(score - top),
    plus top.  q [B][H][N][d], k [B][Hkv][N][d]; returns [B][H][N]."""
    out = []
    for qb, kb in zip(q, k):
        ob = []
        for qh, kh in zip(qb, _expand(kb, len(qb))):
            oh = []
            for i, qrow in enumerate(qh):
                n = i + 1 if causal else len(kh)
                scores = [scale * math.fsum(a * b for a, b in zip(qrow, kr)) for kr in kh[:n]]
                top = max(scores)
                oh.append(top + math.log(math.fsum(math.exp(sc - top) for sc in scores)))
            ob.append(oh)
        out.append(ob)
    return out
