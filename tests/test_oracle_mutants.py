"""Plant plausible mistakes in copies of the oracle and check a pin catches each.

The mutants are built on the CPU from the oracle's own source text with one
substitution each; the real oracle is never modified.
"""

import os
import types

import pytest

import oracle_pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "attention.py")

MUTATIONS = {
    "mask_strict": ("keys[None, :] <= rows[:, None]", "keys[None, :] < rows[:, None]"),
    "mask_reversed": ("keys[None, :] <= rows[:, None]", "keys[None, :] >= rows[:, None]"),
    "dropped_scale": ("s = float(scale) * (qh[rows] @ kh.T)", "s = (qh[rows] @ kh.T)"),
    "swapped_qk": ("s = float(scale) * (qh[rows] @ kh.T)", "s = float(scale) * (kh[rows] @ qh.T)"),
    "no_max_subtraction": ("w = np.exp(s - m)", "w = np.exp(s)"),
    "no_normalisation": ("return (w @ v) / l", "return (w @ v)"),
    "wrong_sum_axis": ("l = np.sum(w, axis=1, keepdims=True)", "l = np.sum(w, axis=0, keepdims=True)"),
    "reversed_values": ("return (w @ v) / l", "return (w @ v[::-1]) / l"),
    "decode_excludes_current": ("(q[b, h] @ kc[b, g, :L].T)", "(q[b, h] @ kc[b, g, :L - 1].T)"),
    "decode_values_offset": ("out[b, h] = _softmax_average(s, vc[b, g, :L])", "out[b, h] = _softmax_average(s, vc[b, g, 1:L + 1])"),
    "kv_head_modulo": ("return h // (hq // hkv)", "return h % hkv"),
    "kv_head_last_of_group": ("return h // (hq // hkv)", "return min(hkv - 1, (h + 1) // (hq // hkv))"),
    "lse_without_max": ("return m + np.log(np.sum(np.exp(s - m[:, None]), axis=1))", "return np.log(np.sum(np.exp(s - m[:, None]), axis=1))"),
    "lse_base_two": ("return m + np.log(np.sum(np.exp(s - m[:, None]), axis=1))", "return m + np.log2(np.sum(np.exp(s - m[:, None]), axis=1))"),
    "lse_mask_strict": ("np.where(rows[:, None] >= keys[None, :], s, -np.inf)", "np.where(rows[:, None] > keys[None, :], s, -np.inf)"),
    "lse_unscaled": ("s = (qh[rows] @ kh.T) * float(scale)", "s = (qh[rows] @ kh.T)"),
    "lse_rows_wrong_head": ("g = kv_head(h, q.shape[1], k.shape[1])\n    return _lse_rows", "g = 0\n    return _lse_rows"),
    "bwd_no_rowsum_term": ("ds = pm * (dp - np.sum(dp * pm, axis=1, keepdims=True))", "ds = pm * dp"),
    "bwd_dv_untransposed": ("dv[b, g] += pm.T @ do[b, h]", "dv[b, g] += pm @ do[b, h]"),
    "bwd_dk_unscaled": ("dk[b, g] += float(scale) * (ds.T @ q[b, h])", "dk[b, g] += (ds.T @ q[b, h])"),
    "bwd_dq_uses_dst": ("dq[b, h] = float(scale) * (ds @ k[b, g])", "dq[b, h] = float(scale) * (ds.T @ k[b, g])"),
    "bwd_group_overwrites": ("dk[b, g] += float(scale) * (ds.T @ q[b, h])", "dk[b, g] = float(scale) * (ds.T @ q[b, h])"),
    "bwd_mask_reversed": ("s = np.where(keys[None, :] <= keys[:, None], s, -np.inf)", "s = np.where(keys[None, :] >= keys[:, None], s, -np.inf)"),
    "bwd_rows_no_rowsum_term": ("ds = pm * (dp - (dp * pm).sum(axis=1, keepdims=True))", "ds = pm * dp"),
    "bwd_rows_mask_strict": ("np.where(np.arange(kh.shape[0]) <= rows[:, None]", "np.where(np.arange(kh.shape[0]) < rows[:, None]"),
    "bwd_rows_one_head_per_group": ("if kv_head(h, H, Hkv) != g:", "if h != g:"),
    "bwd_rows_dk_unscaled": ("dk += float(scale) * (ds[:, keys].T @ qh[rows])", "dk += ds[:, keys].T @ qh[rows]"),
    "prefill_values_head_zero": ("_rows(q[b, h], k[b, g], v[b, g], rows, causal, scale)", "_rows(q[b, h], k[b, g], v[b, 0], rows, causal, scale)"),
    "split_no_rescale": ("wts = [np.exp(m - M) for m in ms]", "wts = [1.0 for m in ms]"),
    "split_den_unweighted": ("den = sum(w * l for w, l in zip(wts, ls))", "den = sum(ls)"),
    "split_sign": ("wts = [np.exp(m - M) for m in ms]", "wts = [np.exp(M - m) for m in ms]"),
    "split_drops_last_row": ("c1 = min(L, c0 + chunk)", "c1 = min(L - 1, c0 + chunk)"),
    "split_acc_unweighted": ("num = sum(w * a for w, a in zip(wts, accs))", "num = sum(accs)"),
    "split_unscaled": ("s = float(scale) * (kc[b, g, c0:c1] @ q[b, h, 0])", "s = (kc[b, g, c0:c1] @ q[b, h, 0])"),
    "decode_unscaled": ("s = float(scale) * (q[b, h] @ kc[b, g, :L].T)", "s = (q[b, h] @ kc[b, g, :L].T)"),
    "bwd_dq_unscaled": ("dq[b, h] = float(scale) * (ds @ k[b, g])", "dq[b, h] = (ds @ k[b, g])"),
    "bwd_dv_scaled": ("dv[b, g] += pm.T @ do[b, h]", "dv[b, g] += float(scale) * (pm.T @ do[b, h])"),
    "bwd_ds_sign": ("ds = pm * (dp - np.sum(dp * pm, axis=1, keepdims=True))",
                    "ds = pm * (np.sum(dp * pm, axis=1, keepdims=True) - dp)"),
    "bwd_rows_dq_unscaled": ("return float(scale) * (ds @ kh)", "return ds @ kh"),
    "bwd_rows_dv_from_ds": ("dv += pm[:, keys].T @ doh[rows]", "dv += ds[:, keys].T @ doh[rows]"),
    "bwd_rows_values_unmasked": ("s = np.where(np.arange(kh.shape[0]) <= rows[:, None], s, -np.inf)",
                                 "s = s"),
}


def _mutant(old, new):
    with open(SRC) as f:
        text = f.read()
    assert text.count(old) == 1, old
    mod = types.ModuleType("oracle_mutant")
    exec(compile(text.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutant(name):
    mod = _mutant(*MUTATIONS[name])
    caught = []
    for pin in oracle_pins.PINS:
        try:
            with __import__("numpy").errstate(all="ignore"):
                pin(mod)
        except Exception:  # an AssertionError, or the broken code raising on its own
            caught.append(pin.__name__)
    assert caught, f"no pin catches mutant {name}"
