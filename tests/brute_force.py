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


def prefill(q, k, v, causal, scale):
    """q, k, v nested lists [B][H][N][d] of floats; returns the same nesting."""
    out = []
    for qb, kb, vb in zip(q, k, v):
        ob = []
        for qh, kh, vh in zip(qb, kb, vb):
            oh = []
            for i, qrow in enumerate(qh):
                n = i + 1 if causal else len(kh)
                oh.append(_attend(qrow, kh[:n], vh[:n], scale))
            ob.append(oh)
        out.append(ob)
    return out


def decode(q, k_cache, v_cache, seq_lens, scale):
    """q [B][H][1][d], caches [B][H][max_len][d]; returns [B][H][1][d]."""
    out = []
    for b, (qb, kb, vb) in enumerate(zip(q, k_cache, v_cache)):
        L = int(seq_lens[b])
        out.append([[_attend(qh[0], kh[:L], vh[:L], scale)] for qh, kh, vh in zip(qb, kb, vb)])
    return out
