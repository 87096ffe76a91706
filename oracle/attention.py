"""Plain fp64 CPU oracle for exact attention (prefill and decode).

TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this module.  The product path (the HIP
library and its Python binding) never calls it and has no CPU fallback.

What it computes is the plain definition on page 3 of the pages ("What is
Attention?", "The Problem", and the usage block under "Installation"): every
query scores each visible key with a scaled dot product, the scores are turned
into weights that are positive and sum to one, and the output row is the
weight-averaged value rows.  There is no tiling and no online recurrence here:
the method on the pages (page 3 "Kernel design"; page 2 "Technical details")
reaches the same numbers by streaming tiles, which is exactly what this file is
used to check.

Conventions (readings of the pages, all explicit):
  * inputs are the stored fp16/bf16 values converted exactly to float64;
    ``scale`` is the float32 value that crosses the C interface, widened to
    float64;
  * causal: key j is visible to query row i iff j <= i (one sequence length for
    queries and keys);
  * decode over a cache of length L attends to rows 0..L-1, the current token's
    own row included, so decode with L = t + 1 equals causal prefill row t
    (page 3, "What can it do": decoding token t equals prefill row t);
  * masked scores are -inf, i.e. exactly zero weight.

Grouped heads (a reading of page 3, "Future work", where grouped-query attention
is served by repeating each K/V head for its group of query heads): K and V may
carry fewer heads than Q.  With Hq query heads and Hkv K/V heads, Hkv divides Hq,
and query head h reads K/V head h // (Hq // Hkv), the head that repeating each K/V
head Hq // Hkv times in order would place at position h.  Hkv = Hq is ordinary
multi-head attention, Hkv = 1 shares one K/V head among all query heads.

Every function follows the definition above; ``decode_split`` additionally
follows the split-and-merge description on page 3 ("Kernel design": split-K
decode with partial (m, l, acc) merged exactly by a second pass) and is used only
to pin split-size invariance.
"""

from __future__ import annotations

import numpy as np

ROW_BLOCK = 1024  # rows per matrix product; row blocking does not change any row's value


def kv_head(h: int, hq: int, hkv: int) -> int:
    """K/V head read by query head h (see the module notes on grouped heads)."""
    assert hkv >= 1 and hq % hkv == 0, "the K/V head count must divide the query head count"
    return h // (hq // hkv)


def _softmax_average(s: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Rows of weights exp(s - max) / sum, applied to v.  s: (R, K) with -inf allowed."""
    m = np.max(s, axis=1, keepdims=True)
    w = np.exp(s - m)
    l = np.sum(w, axis=1, keepdims=True)
    return (w @ v) / l


def prefill(q: np.ndarray, k: np.ndarray, v: np.ndarray, causal: bool, scale: float) -> np.ndarray:
    """Exact attention for q (B, H, N, d) and k, v (B, Hkv, N, d); returns (B, H, N, d).

    Page 3, "What is Attention?" / "The Problem": each row scores every
    (previous, if causal) key; the weights sum to one and combine the values.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    assert k.shape == (B, Hkv, N, d) and v.shape == (B, Hkv, N, d)
    out = np.empty((B, H, N, d), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            g = kv_head(h, H, Hkv)
            for r0 in range(0, N, ROW_BLOCK):
                rows = np.arange(r0, min(N, r0 + ROW_BLOCK))
                out[b, h, rows] = _rows(q[b, h], k[b, g], v[b, g], rows, causal, scale)
    return out


def _rows(qh, kh, vh, rows, causal, scale):
    s = float(scale) * (qh[rows] @ kh.T)  # (R, N)
    if causal:
        keys = np.arange(kh.shape[0])
        s = np.where(keys[None, :] <= rows[:, None], s, -np.inf)
    return _softmax_average(s, vh)


def prefill_lse(q, k, causal: bool, scale: float) -> np.ndarray:
    """Row log-sum-exp of the scaled scores: lse[b, h, i] = log sum_j exp(scale q_i . k_j)
    over the visible keys j, natural log; returns (B, H, N) float64.

    The normaliser of the softmax in the definition above (its log): the output row
    equals sum_j exp(scale q_i . k_j - lse_i) v_j.  Computed as m + log(sum exp(s - m))
    with m the row max, which is the same number without overflow.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    assert k.shape == (B, Hkv, N, d)
    out = np.empty((B, H, N), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            g = kv_head(h, H, Hkv)
            for r0 in range(0, N, ROW_BLOCK):
                rows = np.arange(r0, min(N, r0 + ROW_BLOCK))
                out[b, h, rows] = _lse_rows(q[b, h], k[b, g], rows, causal, scale)
    return out


def _lse_rows(qh, kh, rows, causal, scale):
    s = (qh[rows] @ kh.T) * float(scale)
    if causal:  # key j visible to row i iff j <= i
        keys = np.arange(kh.shape[0])
        s = np.where(rows[:, None] >= keys[None, :], s, -np.inf)
    m = np.max(s, axis=1)
    return m + np.log(np.sum(np.exp(s - m[:, None]), axis=1))


def prefill_lse_rows(q, k, causal: bool, scale: float, b: int, h: int, rows) -> np.ndarray:
    """prefill_lse for selected rows of one (b, h) only; returns (len(rows),)."""
    rows = np.asarray(rows, dtype=np.int64)
    g = kv_head(h, q.shape[1], k.shape[1])
    return _lse_rows(np.asarray(q[b, h], dtype=np.float64), np.asarray(k[b, g], dtype=np.float64), rows, causal, scale)


def prefill_rows(q, k, v, causal: bool, scale: float, b: int, h: int, rows) -> np.ndarray:
    """The same definition for selected rows of one (b, h) only; returns (len(rows), d).

    Used to check outputs at sizes where the full oracle would take minutes.
    """
    rows = np.asarray(rows, dtype=np.int64)
    g = kv_head(h, q.shape[1], k.shape[1])
    qh = np.asarray(q[b, h], dtype=np.float64)
    kh = np.asarray(k[b, g], dtype=np.float64)
    vh = np.asarray(v[b, g], dtype=np.float64)
    return _rows(qh, kh, vh, rows, causal, scale)


def decode(q, k_cache, v_cache, seq_lens, scale: float) -> np.ndarray:
    """One query row per (b, h) over the first L_b cache rows; returns (B, H, 1, d).
    The caches may carry Hkv heads (grouped heads).

    Page 3, "What can it do": one new token attends over a KV cache, with a
    different current length per sequence in the batch.
    """
    q = np.asarray(q, dtype=np.float64)
    kc = np.asarray(k_cache, dtype=np.float64)
    vc = np.asarray(v_cache, dtype=np.float64)
    B, H, one, d = q.shape
    assert one == 1
    Hkv = kc.shape[1]
    out = np.empty((B, H, 1, d), dtype=np.float64)
    for b in range(B):
        L = int(seq_lens[b])
        assert 1 <= L <= kc.shape[2], "cache length must lie in [1, max_len]"
        for h in range(H):
            g = kv_head(h, H, Hkv)
            s = float(scale) * (q[b, h] @ kc[b, g, :L].T)  # (1, L)
            out[b, h] = _softmax_average(s, vc[b, g, :L])
    return out


def decode_split(q, k_cache, v_cache, seq_lens, scale: float, chunk: int) -> np.ndarray:
    """Decode computed as chunks of ``chunk`` cache rows, then merged exactly.

    Page 3, "Kernel design": the cache is split into chunks, each chunk yields a
    partial (m, l, acc), and a second pass merges the partials with the (m, l)
    rescale.  For chunk c over rows J_c: m_c = max s, l_c = sum exp(s - m_c),
    a_c = sum exp(s - m_c) v.  With M = max_c m_c the result is
    sum_c exp(m_c - M) a_c / sum_c exp(m_c - M) l_c.  Empty chunks do not exist
    here because chunks only cover [0, L).
    """
    assert chunk >= 1
    q = np.asarray(q, dtype=np.float64)
    kc = np.asarray(k_cache, dtype=np.float64)
    vc = np.asarray(v_cache, dtype=np.float64)
    B, H, _, d = q.shape
    Hkv = kc.shape[1]
    out = np.empty((B, H, 1, d), dtype=np.float64)
    for b in range(B):
        L = int(seq_lens[b])
        assert 1 <= L <= kc.shape[2]
        for h in range(H):
            g = kv_head(h, H, Hkv)
            ms, ls, accs = [], [], []
            for c0 in range(0, L, chunk):
                c1 = min(L, c0 + chunk)
                s = float(scale) * (kc[b, g, c0:c1] @ q[b, h, 0])  # (C,)
                m = np.max(s)
                p = np.exp(s - m)
                ms.append(m)
                ls.append(np.sum(p))
                accs.append(p @ vc[b, g, c0:c1])
            M = max(ms)
            wts = [np.exp(m - M) for m in ms]
            num = sum(w * a for w, a in zip(wts, accs))
            den = sum(w * l for w, l in zip(wts, ls))
            out[b, h, 0] = num / den
    return out


def backward(q, k, v, dout, causal: bool, scale: float):
    """Gradients of the loss sum(dout * O) for O = prefill(q, k, v, causal, scale);
    returns (dq, dk, dv) float64, shaped like q, k, v.

    The chain rule through the definition (page 3, "Future work", asks for the
    backward pass), per (b, h) with P the row-softmax of S = scale q k^T (masked
    entries exactly 0):
      dV = P^T dO;   dP = dO V^T;   dS = P * (dP - rowsum(dP * P));
      dQ = scale dS K;   dK = scale dS^T Q.
    rowsum(dP * P) equals rowsum(dO * O), the form the method uses.  With grouped
    heads, a K/V head's gradient sums those of the query heads that read it.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(dout, dtype=np.float64)
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    assert k.shape == (B, Hkv, N, d) and v.shape == (B, Hkv, N, d) and do.shape == q.shape
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    keys = np.arange(N)
    for b in range(B):
        for h in range(H):
            g = kv_head(h, H, Hkv)
            s = float(scale) * (q[b, h] @ k[b, g].T)
            if causal:
                s = np.where(keys[None, :] <= keys[:, None], s, -np.inf)
            m = np.max(s, axis=1, keepdims=True)
            e = np.exp(s - m)
            pm = e / np.sum(e, axis=1, keepdims=True)
            dv[b, g] += pm.T @ do[b, h]
            dp = do[b, h] @ v[b, g].T
            ds = pm * (dp - np.sum(dp * pm, axis=1, keepdims=True))
            dq[b, h] = float(scale) * (ds @ k[b, g])
            dk[b, g] += float(scale) * (ds.T @ q[b, h])
    return dq, dk, dv


def _head_grads_block(qh, kh, vh, doh, rows, causal, scale):
    """For a block of query rows of one head: P and dS (the chain rule above, per row;
    every row's values depend on that row alone).  Returns (pm, ds), each (R, N)."""
    s = float(scale) * np.matmul(qh[rows], kh.T)
    if causal:  # key j visible to row i iff j <= i
        s = np.where(np.arange(kh.shape[0]) <= rows[:, None], s, -np.inf)
    m = np.max(s, axis=1, keepdims=True)
    e = np.exp(s - m)
    pm = e / np.sum(e, axis=1, keepdims=True)
    dp = doh[rows] @ vh.T
    ds = pm * (dp - (dp * pm).sum(axis=1, keepdims=True))
    return pm, ds


def backward_dq_rows(q, k, v, dout, causal: bool, scale: float, b: int, h: int, rows) -> np.ndarray:
    """Rows of dq for query head h of batch b (the backward definition above, only the
    selected rows: dq_i depends on row i's P and dP alone); returns (len(rows), d)."""
    rows = np.asarray(rows, dtype=np.int64)
    g = kv_head(h, q.shape[1], k.shape[1])
    f = lambda t: np.asarray(t, dtype=np.float64)  # noqa: E731
    kh = f(k[b, g])
    _, ds = _head_grads_block(f(q[b, h]), kh, f(v[b, g]), f(dout[b, h]), rows, causal, scale)
    return float(scale) * (ds @ kh)


def backward_dkdv_rows(q, k, v, dout, causal: bool, scale: float, b: int, g: int, keys):
    """Rows ``keys`` of dk and dv for K/V head g of batch b, summed over the query heads
    that read it (the backward definition above).  Each key row's gradient gathers
    column j of P and dS over every query row, so every query row is formed, one block
    of rows at a time; returns (dk, dv), each (len(keys), d)."""
    keys = np.asarray(keys, dtype=np.int64)
    f = lambda t: np.asarray(t, dtype=np.float64)  # noqa: E731
    H, Hkv, N = q.shape[1], k.shape[1], q.shape[2]
    kh, vh = f(k[b, g]), f(v[b, g])
    dk = np.zeros((len(keys), kh.shape[1]))
    dv = np.zeros((len(keys), kh.shape[1]))
    for h in range(H):
        if kv_head(h, H, Hkv) != g:
            continue
        qh, doh = f(q[b, h]), f(dout[b, h])
        for r0 in range(0, N, ROW_BLOCK):
            rows = np.arange(r0, min(N, r0 + ROW_BLOCK))
            pm, ds = _head_grads_block(qh, kh, vh, doh, rows, causal, scale)
            dv += pm[:, keys].T @ doh[rows]
            dk += float(scale) * (ds[:, keys].T @ qh[rows])
    return dk, dv
