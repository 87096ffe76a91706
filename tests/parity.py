"""Tolerance rules and conversions shared by the GPU parity tests."""

import numpy as np
import torch

# Max |GPU - oracle| allowed per element, by storage dtype.
TOL = {"f16": 2e-3, "bf16": 1e-2}


def f64(t: torch.Tensor) -> np.ndarray:
    """Exact widening of a fp16/bf16 tensor to a float64 array (on the CPU)."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def bf16_half_ulp(x: np.ndarray) -> np.ndarray:
    """Half a bf16 unit in the last place at |x| (8 significant bits)."""
    ax = np.maximum(np.abs(x), np.finfo(np.float64).tiny)
    return 0.5 * np.exp2(np.floor(np.log2(ax)) - 7)


def allowed(ref: np.ndarray, dtype: str) -> np.ndarray:
    """Per-element bound.  bf16 outputs with |oracle| >= 2 may also be off by the final
    rounding to bf16 itself (half an ulp is 7.8e-3 in [2, 4) and 1.6e-2 in [4, 8)), so
    there the bound is the gate plus half an ulp of the oracle value."""
    tol = np.full(ref.shape, TOL[dtype])
    if dtype == "bf16":
        big = np.abs(ref) >= 2
        tol = np.where(big, TOL[dtype] + bf16_half_ulp(ref), tol)
    return tol


def check(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = ""):
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    bound = allowed(ref, dtype)
    bad = err > bound
    if np.any(bad):
        idx = np.argwhere(bad)[:5]
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {err.size} elements over the bound; max err {err.max():.3e}; "
            f"first at {idx.tolist()} got {got[tuple(idx[0])]:.6f} ref {ref[tuple(idx[0])]:.6f}"
        )
    return float(err.max())


UNIT_ROUNDOFF = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}


def _bound_terms(qh, kh, vh, doh, rows, causal, scale, lse_rows):
    """For query rows ``rows`` of one head: the softmax P (from the oracle's lse) and
    |dS| + P * sum_d |dO||O|, the magnitude that bounds the rounded dS and delta terms."""
    s = scale * (qh[rows] @ kh.T)
    if causal:
        s = np.where(np.arange(kh.shape[0])[None, :] <= rows[:, None], s, -np.inf)
    pm = np.exp(s - lse_rows[:, None])
    o = pm @ vh
    dp = doh[rows] @ vh.T
    delta = np.sum(doh[rows] * o, axis=1, keepdims=True)
    ds = pm * (dp - delta)
    ddelta = np.sum(np.abs(doh[rows]) * np.abs(o), axis=1, keepdims=True)
    return pm, np.abs(ds) + pm * ddelta


def backward_bounds(q, k, v, dout, causal, scale, lse):
    """Per-element magnitudes that bound the rounding error of the kernels' gradients
    (all fp64 arrays; lse from the oracle).  Each gradient is a sum of products whose
    one rounded factor is P (dV) or dS (dQ, dK), off by at most a relative u; dS also
    carries the error of delta = rowsum(dO * O) computed from the 16-bit O, at most
    u * sum_d |dO||O| per row.  Returns (bq, bk, bv) such that
    |error| <= u |gradient| (the 16-bit output) + 2 u b + fp32 accumulation."""
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    g = H // Hkv
    bq = np.zeros_like(q)
    bk = np.zeros_like(k)
    bv = np.zeros_like(v)
    rows = np.arange(N)
    for b in range(B):
        for h in range(H):
            kh, vh = k[b, h // g], v[b, h // g]
            pm, dsb = _bound_terms(q[b, h], kh, vh, dout[b, h], rows, causal, scale, lse[b, h])
            bq[b, h] = abs(scale) * (dsb @ np.abs(kh))
            bk[b, h // g] += abs(scale) * (dsb.T @ np.abs(q[b, h]))
            bv[b, h // g] += pm.T @ np.abs(dout[b, h])
    return bq, bk, bv


def backward_bounds_rows(q, k, v, dout, causal, scale, b, h, rows):
    """backward_bounds' bq at query rows ``rows`` of head h of batch b (fp64 inputs)."""
    import oracle

    rows = np.asarray(rows, dtype=np.int64)
    g = q.shape[1] // k.shape[1]
    kh, vh = k[b, h // g], v[b, h // g]
    lse = oracle.prefill_lse_rows(q, k, causal, scale, b, h, rows)
    _, dsb = _bound_terms(q[b, h], kh, vh, dout[b, h], rows, causal, scale, lse)
    return abs(scale) * (dsb @ np.abs(kh))


def backward_bounds_keys(q, k, v, dout, causal, scale, b, kv, keys, block=1024):
    """backward_bounds' bk, bv at key rows ``keys`` of K/V head kv of batch b."""
    import oracle

    keys = np.asarray(keys, dtype=np.int64)
    H, N = q.shape[1], q.shape[2]
    g = H // k.shape[1]
    kh, vh = k[b, kv], v[b, kv]
    bk = np.zeros((len(keys), k.shape[3]))
    bv = np.zeros((len(keys), k.shape[3]))
    for h in range(kv * g, (kv + 1) * g):
        for r0 in range(0, N, block):
            rows = np.arange(r0, min(N, r0 + block))
            lse = oracle.prefill_lse_rows(q, k, causal, scale, b, h, rows)
            pm, dsb = _bound_terms(q[b, h], kh, vh, dout[b, h], rows, causal, scale, lse)
            bk += abs(scale) * (dsb[:, keys].T @ np.abs(q[b, h, rows]))
            bv += pm[:, keys].T @ np.abs(dout[b, h, rows])
    return bk, bv


def check_grad(got, ref, bound, dtype, what):
    """|got - ref| <= u |ref| + 2 u bound + 1e-5 bound + 1e-6 elementwise (see backward_bounds)."""
    u = UNIT_ROUNDOFF[dtype]
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got)), f"{what}: non-finite gradient"
    err = np.abs(got - ref)
    gate = u * np.abs(ref) + (2 * u + 1e-5) * bound + 1e-6
    bad = err > gate
    if np.any(bad):
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} of {err.size} over the gate; first at {list(i)} "
                             f"got {got[i]:.6g} ref {ref[i]:.6g} gate {gate[i]:.3g}; max err {err.max():.3e}")
    return float(err.max())


def plan_form(B, H, N, d, causal, cus):
    """The prefill workgroup form a shape takes (attn_prefill_plan), as a tuple."""
    import exact_attention_prefill_amd as ea

    p = ea.prefill_plan(B, H, N, d, causal, cus)
    return (p["waves"], p["rows_per_wave"], p["stages"], p["key_groups"])


def one_group_heads(H, N, d, causal, cus, avoid=None):
    """Smallest number of heads k <= H whose (1, k, N) prefill runs a form with one key
    group (and not the form `avoid`), or None.  Forms with one key group give every row
    the same bits, so a k-head slice is a bit-exact reference for another such form."""
    for k in range(1, H + 1):
        f = plan_form(1, k, N, d, causal, cus)
        if f[3] == 1 and f != avoid:
            return k
    return None


def ulp16(x: np.ndarray, dtype: str) -> np.ndarray:
    """The 16-bit dtype's unit in the last place at |x| (normal range; fp16 subnormals
    share the smallest normal's spacing)."""
    bits = {"f16": 10, "bf16": 7}[dtype]
    lo = {"f16": -14, "bf16": -126}[dtype]
    e = np.floor(np.log2(np.maximum(np.abs(x), np.finfo(np.float64).tiny)))
    return np.exp2(np.maximum(e, lo) - bits)


def same_rows(got, ref, got_form, ref_form, dtype, what=""):
    """Rows of one head from two launch forms: bit-identical when both forms have one
    key group.  Otherwise the keys are summed in another order, so the two fp32 results
    differ by a few fp32 roundings and their 16-bit outputs by at most about one unit in
    the last place: within the gate plus one ulp of the value."""
    if got_form[3] == 1 and ref_form[3] == 1:
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), (what, got_form, ref_form)
    else:
        a, b = f64(got), f64(ref)
        err = np.abs(a - b)
        bound = TOL[dtype] + ulp16(np.maximum(np.abs(a), np.abs(b)), dtype)
        assert np.all(err <= bound), (what, got_form, ref_form, float(err.max()))
