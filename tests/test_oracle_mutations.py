"""Planted mistakes in the oracle (CPU only).

Each mutation below is a plausible slip in one oracle function: a dropped
term or factor, a flipped comparison, a wrong tie order, an off-by-one, a
swapped operand.  It is applied to an in-memory copy of the oracle's source
text, and every pin in test_oracle_pins.py is run against that copy; at least
one pin must fail.  A mutation that no pin notices marks a part of the
oracle that nothing independent checks.
"""
import inspect
import sys
import types

import pytest

import tests.test_oracle_pins as pins
from oracle import bsa_oracle

SRC = inspect.getsource(bsa_oracle)

# (id, text in the oracle, replacement)
MUTATIONS = [
    # pooling and block geometry
    ("pool_divides_by_block", "x[lo:hi].mean(axis=0) for lo, hi in spans",
     "x[lo:hi].sum(axis=0) / block for lo, hi in spans"),
    ("spans_unclamped", "(i * block, min((i + 1) * block, n_tokens))", "(i * block, (i + 1) * block)"),
    ("sub_block_width_off", "    w = block // sub_blocks\n", "    w = block // sub_blocks + 1\n"),
    ("forced_prefix_inclusive", "j * block < keep_prefix_tokens", "j * block <= keep_prefix_tokens"),
    # pooled scores
    ("estimator_drops_scale", "logits = float(scale) * (qbar @ kbar.T)", "logits = qbar @ kbar.T"),
    ("estimator_transposed_scores", "logits = float(scale) * (qbar @ kbar.T)",
     "logits = float(scale) * (kbar @ qbar.T)"),
    ("hierarchical_max_not_lse", "out[:, j] = mx + np.log(np.exp(s - mx[:, None]).sum(axis=1))",
     "out[:, j] = mx"),
    ("hierarchical_log_mean_exp", "out[:, j] = mx + np.log(np.exp(s - mx[:, None]).sum(axis=1))",
     "out[:, j] = mx + np.log(np.exp(s - mx[:, None]).mean(axis=1))"),
    # Top-p over pooled scores
    ("ties_to_higher_id", "order = np.lexsort((cand, -s))", "order = np.lexsort((-cand, -s))"),
    ("softmax_temperature", "e = np.exp(s - s.max())\n    prob = e / e.sum()",
     "e = np.exp(2.0 * (s - s.max()))\n    prob = e / e.sum()"),
    ("cut_exclusive", "        hit = np.nonzero(cum >= p)[0]\n        k_star = int(hit[0]) + 1 if hit.size else n\n"
     "    sel = np.union1d(ranked[:k_star], forced).astype(np.int64)\n    return RowSelection(cand,",
     "        hit = np.nonzero(cum > p)[0]\n        k_star = int(hit[0]) + 1 if hit.size else n\n"
     "    sel = np.union1d(ranked[:k_star], forced).astype(np.int64)\n    return RowSelection(cand,"),
    ("k_star_off_by_one", "        k_star = int(hit[0]) + 1 if hit.size else n\n"
     "    sel = np.union1d(ranked[:k_star], forced).astype(np.int64)\n    return RowSelection(cand,",
     "        k_star = int(hit[0]) if hit.size else n\n"
     "    sel = np.union1d(ranked[:k_star], forced).astype(np.int64)\n    return RowSelection(cand,"),
    ("forced_ignored", "    sel = np.union1d(ranked[:k_star], forced).astype(np.int64)\n    return RowSelection(cand,",
     "    sel = np.sort(ranked[:k_star]).astype(np.int64)\n    return RowSelection(cand,"),
    ("candidate_ids_unfiltered", "            cand = cand[(cand >= 0) & (cand < nb)]\n", ""),
    ("candidates_ignored", "rows.append(top_p_select(cand, logits[i, cand], top_p, forced))",
     "rows.append(top_p_select(np.arange(nb), logits[i], top_p, forced))"),
    # estimator over whole [B, H, N, D] tensors
    ("candidate_slice_ignores_batch", "        base = (b * H + h) * nb\n", "        base = h * nb\n"),
    ("rows_in_h_b_order", "[(b, h) for b in range(B) for h in range(H)]",
     "[(b, h) for h in range(H) for b in range(B)]"),
    # bands that excuse GPU/oracle differences
    ("band_value_tol_doubled", "if (r < row.k_star and s <= s_next + tol) or (r >= row.k_star and s >= s_last - tol):",
     "if (r < row.k_star and s <= s_next + 2 * tol) or (r >= row.k_star and s >= s_last - 2 * tol):"),
    ("band_cumulative_rank_off", "band.add(int(row.ranked[r - 1]))", "band.add(int(row.ranked[r - 2]))"),
    ("band_keeps_forced", "    return band - set(row.forced.tolist())\n\n\ndef top_p_from_mass",
     "    return band\n\n\ndef top_p_from_mass"),
    ("mass_band_off_by_one_rank", "band = {int(row.ranked[r - 1]) for r in range(2, n + 1) if abs(row.cumulative[r - 2] - p)",
     "band = {int(row.ranked[r - 2]) for r in range(2, n + 1) if abs(row.cumulative[r - 2] - p)"),
    # Top-p over block masses (narrowing)
    ("mass_share_unnormalised", "cum = np.cumsum(m[order]) / total", "cum = np.cumsum(m[order])"),
    ("mass_ties_to_higher_id", "order = np.lexsort((ent, -m))", "order = np.lexsort((-ent, -m))"),
    ("mass_negative_kept", "m = np.where(m > 0, m, 0.0)", "m = np.nan_to_num(m)"),
    ("narrow_keeps_bad_ids", "ok = (ent >= 0) & (ent < nb)", "ok = ent >= 0"),
    # token permutation
    ("gather_as_scatter", "        y[:, ok] = x[:, perm[ok]]\n", "        y[:, perm[ok]] = x[:, ok]\n"),
    # structured masks
    ("temporal_uses_frames", "ok = bool(spots[i] & spots[j])", "ok = bool(frames[i] & frames[j])"),
    ("text_keys_dropped", "if has_text[i] or has_text[j] or kind == PATTERN_DENSE:",
     "if has_text[i] or kind == PATTERN_DENSE:"),
    ("multi_diagonal_strict", "ok = any(abs(i - j - k * period) <= band for k in range(-nb, nb + 1))",
     "ok = any(abs(i - j - k * period) < band for k in range(-nb, nb + 1))"),
    # sparse attention forward
    ("attention_drops_scale", "S = float(scale) * (q_blk @ keys.T)", "S = q_blk @ keys.T"),
    ("empty_row_lse_zero", "np.full(nq, -np.inf)", "np.zeros(nq)"),
    ("lse_drops_max", "lse = (m + np.log(l))[:, 0]", "lse = np.log(l)[:, 0]"),
    ("mass_summed_over_queries", "mass = np.array([P[:, a:b].sum(axis=1).mean() for a, b in cols])",
     "mass = np.array([P[:, a:b].sum() for a, b in cols])"),
    ("mass_of_unnormalised_weights", "mass = np.array([P[:, a:b].sum(axis=1).mean() for a, b in cols])",
     "mass = np.array([E[:, a:b].sum(axis=1).mean() for a, b in cols])"),
    ("values_from_keys", "vals, _ = _gather(v, spans, key_blocks)", "vals, _ = _gather(k, spans, key_blocks)"),
    # backward
    ("backward_drops_delta", "                dS = P * (dP - delta)\n", "                dS = P * dP\n"),
    ("backward_delta_sign", "                dS = P * (dP - delta)\n", "                dS = P * (delta - dP)\n"),
    ("backward_dk_drops_scale", "np.add.at(dK[b, h], idx, float(scale) * (dS.T @ q[lo:hi]))",
     "np.add.at(dK[b, h], idx, dS.T @ q[lo:hi])"),
    ("backward_dq_from_values", "dQ[b, h, lo:hi] += float(scale) * (dS @ k[idx])",
     "dQ[b, h, lo:hi] += float(scale) * (dS @ v[idx])"),
    ("backward_dv_from_dp", "np.add.at(dV[b, h], idx, P.T @ g[lo:hi])", "np.add.at(dV[b, h], idx, dS.T @ g[lo:hi])"),
    # work count
    ("executed_pairs_full_blocks", "sizes = np.array([hi - lo for lo, hi in spans], dtype=np.int64)",
     "sizes = np.array([block for lo, hi in spans], dtype=np.int64)"),
]


def _mutant(monkeypatch, old, new):
    assert SRC.count(old) == 1, f"mutation site found {SRC.count(old)} times"
    name = "bsa_oracle_mutant"
    mod = types.ModuleType(name)
    monkeypatch.setitem(sys.modules, name, mod)      # dataclasses look their module up
    exec(compile(SRC.replace(old, new), name, "exec"), mod.__dict__)
    return mod


def _pin_cases():
    for name, fn in sorted(vars(pins).items()):
        if not name.startswith("test_") or not callable(fn):
            continue
        params = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
        if not params:
            yield name, fn, {}
            continue
        argname, values = params[0].args[:2]
        for v in values:
            yield f"{name}[{v}]", fn, {argname: v}


def test_pins_pass_on_the_unmodified_copy(monkeypatch):
    monkeypatch.setattr(pins, "O", _mutant(monkeypatch, "def num_blocks", "def num_blocks"))
    for name, fn, kw in _pin_cases():
        fn(**kw)


@pytest.mark.parametrize("old,new", [m[1:] for m in MUTATIONS], ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(monkeypatch, old, new):
    monkeypatch.setattr(pins, "O", _mutant(monkeypatch, old, new))
    caught = []
    for name, fn, kw in _pin_cases():
        try:
            fn(**kw)
        except (Exception, pytest.fail.Exception):   # an assertion, or the mutant failing outright
            caught.append(name)
    assert caught, "no pin fails with this mistake planted in the oracle"
