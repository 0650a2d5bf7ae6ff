"""Pins of the CPU oracle to things other than itself (CPU only).

Each test checks an oracle function against a hand-worked fixture, a brute
force, an exact-arithmetic special case, a closed form or an independent
construction (pure-Python loops, an explicit token-level mask, finite
differences), chosen so that a dropped term, a flipped comparison or a
transposed operand in the oracle fails at least one of them.
"""
import itertools
import math
import os

import numpy as np
import pytest

from oracle import bsa_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _ints(s):
    s = s.strip()
    return [] if s == "-" else [int(t) for t in s.split()]


# ----------------------------------------------------------------------------
# Top-p
# ----------------------------------------------------------------------------

def test_top_p_hand_worked_fixture():
    rows = [ln for ln in open(os.path.join(GOLDEN, "top_p_hand_worked.txt")) if ln.strip() and not ln.startswith("#")]
    assert len(rows) == 10
    for ln in rows:
        cand, weights, p, forced, expect = ln.split("|")
        cand = np.array(_ints(cand))
        logits = np.log(np.array([float(t) for t in weights.split()]))
        sel = O.top_p_select(cand, logits, float(p), np.array(_ints(forced), dtype=np.int64))
        assert sel.selected.tolist() == _ints(expect), ln


def _brute_force_top_p(logits, p):
    """Smallest subset with probability mass >= p; then largest mass; then lowest ids."""
    n = len(logits)
    w = [math.exp(s) for s in logits]
    z = sum(w)
    prob = [x / z for x in w]
    for size in range(1, n + 1):
        best = None
        for sub in itertools.combinations(range(n), size):
            m = sum(prob[j] for j in sub)
            if m >= p and (best is None or m > best[0] + 1e-12):
                best = (m, sub)
        if best is not None:
            return sorted(best[1]), prob
    return list(range(n)), prob


def _subset_margin(prob, p):
    n = len(prob)
    return min(abs(sum(prob[j] for j in sub) - p)
               for size in range(1, n + 1) for sub in itertools.combinations(range(n), size))


def test_top_p_brute_force_small_rows():
    rng = np.random.default_rng(11)
    checked = 0
    while checked < 200:
        n = int(rng.integers(1, 11))
        logits = rng.normal(0, 1.5, n)
        p = float(rng.uniform(0.05, 0.99))
        expect, prob = _brute_force_top_p(logits.tolist(), p)
        if _subset_margin(prob, p) < 1e-9:
            continue
        got = O.top_p_select(np.arange(n), logits, p)
        assert got.selected.tolist() == expect
        checked += 1


def test_top_p_coverage_invariant():
    rng = np.random.default_rng(12)
    for _ in range(300):
        n = int(rng.integers(2, 200))
        logits = rng.normal(0, 3, n)
        p = float(rng.uniform(0.1, 0.999))
        r = O.top_p_select(np.arange(n), logits, p)
        prob = np.exp(logits - logits.max())
        prob /= prob.sum()
        kept = prob[r.selected].sum()
        assert kept >= p - 1e-12
        # dropping the lowest-ranked kept block falls below p
        last = r.ranked[r.k_star - 1]
        assert kept - prob[last] < p
        # every kept block outranks every dropped one
        dropped = np.setdiff1d(np.arange(n), r.selected)
        if dropped.size:
            assert logits[r.selected].min() >= logits[dropped].max()


def test_top_p_exact_uniform_ties_and_inclusive_cut():
    # K = 0 makes every pooled logit exactly 0: probabilities are exactly 1/16.
    N, bs, D = 1024, 64, 64
    q = np.random.default_rng(3).normal(size=(N, D))
    k = np.zeros((N, D))
    rows = O.estimate_head(q, k, bs, float(np.float32(0.9)), 0.125)
    for r in rows:
        assert r.selected.tolist() == list(range(15))       # 14/16 < 0.9 <= 15/16
    rows = O.estimate_head(q, k, bs, 0.875, 0.125)
    for r in rows:
        assert r.selected.tolist() == list(range(14))       # C_14 = 14/16 == p: inclusive cut


def test_top_p_duplicated_key_block_resolves_to_lower_index():
    # Constant tokens per block: pooled logit of key block j is exactly c_j.
    D, bs = 16, 8
    u = np.zeros(D)
    u[0] = 1.0
    c = [2.0, 1.0, 0.0, 1.0]               # blocks 1 and 3 are identical
    k = np.concatenate([np.tile(cj * u, (bs, 1)) for cj in c])
    q = np.tile(4.0 * u, (4 * bs, 1))      # scale = 1/4 -> logit = c_j
    # probabilities e^2, e, 1, e over Z: C_1 = 0.534, C_2 = 0.731, C_3 = 0.928
    sel = O.estimate_head(q, k, bs, 0.6, 0.25)[0].selected.tolist()
    assert sel == [0, 1]
    sel = O.estimate_head(q, k, bs, 0.8, 0.25)[0].selected.tolist()
    assert sel == [0, 1, 3]
    sel = O.estimate_head(q, k, bs, 0.95, 0.25)[0].selected.tolist()
    assert sel == [0, 1, 2, 3]


def test_forced_prefix_blocks_join_after_the_cut():
    rng = np.random.default_rng(4)
    q = rng.normal(size=(300, 8))
    k = rng.normal(size=(300, 8))
    plain = O.estimate_head(q, k, 64, 0.5, 0.35)
    forced = O.estimate_head(q, k, 64, 0.5, 0.35, keep_prefix_tokens=70)   # tokens 0..69: blocks 0, 1
    for a, b in zip(plain, forced):
        assert b.k_star == a.k_star
        assert b.selected.tolist() == sorted(set(a.selected.tolist()) | {0, 1})
    assert O.forced_blocks(64, 64, 5).tolist() == [0]
    assert O.forced_blocks(65, 64, 5).tolist() == [0, 1]
    assert O.forced_blocks(0, 64, 5).tolist() == []


def test_candidate_restriction():
    rng = np.random.default_rng(5)
    N, bs = 700, 64
    q = rng.normal(size=(N, 16))
    k = rng.normal(size=(N, 16)) + q
    nb = O.num_blocks(N, bs)
    full = O.estimate_head(q, k, bs, 0.8, 0.25)
    same = O.estimate_head(q, k, bs, 0.8, 0.25, candidate_rows=[np.arange(nb)] * nb)
    assert [r.selected.tolist() for r in full] == [r.selected.tolist() for r in same]
    cands = [np.sort(rng.choice(nb, size=int(rng.integers(1, nb)), replace=False)) for _ in range(nb)]
    sub = O.estimate_head(q, k, bs, 0.8, 0.25, candidate_rows=cands, keep_prefix_tokens=10)
    qb, kb = O.pool_blocks(q, bs), O.pool_blocks(k, bs)
    for i, r in enumerate(sub):
        assert set(r.selected.tolist()) <= set(cands[i].tolist()) | {0}
        # same answer as a full-row softmax with non-candidates at -inf
        s = 0.25 * (qb[i] @ kb.T)
        s_masked = np.full(nb, -np.inf)
        s_masked[cands[i]] = s[cands[i]]
        e = np.exp(s_masked - s_masked.max())
        prob = e / e.sum()
        order = sorted(range(nb), key=lambda j: (-s_masked[j], j))
        acc, keep = 0.0, []
        for j in order:
            keep.append(j)
            acc += prob[j]
            if acc >= 0.8:
                break
        assert r.selected.tolist() == sorted(set(keep) | {0})
    empty = O.estimate_head(q, k, bs, 0.8, 0.25, candidate_rows=[np.zeros(0)] * nb)
    assert all(r.selected.size == 0 for r in empty)
    # repeated ids count once and ids outside [0, nb) are ignored (the CSR
    # convention): such rows select what their distinct valid ids select
    messy = [np.concatenate([[-3, -1], c, c[:2], [nb, nb + 7]]) for c in cands]
    got = O.estimate_head(q, k, bs, 0.8, 0.25, candidate_rows=messy, keep_prefix_tokens=10)
    assert [r.selected.tolist() for r in got] == [r.selected.tolist() for r in sub]
    assert [r.candidates.tolist() for r in got] == [c.tolist() for c in cands]


def _dominant_block_heads(B, H, nb, bs, D, j_star):
    """Q, K [B, H, nb*bs, D] whose pooled logits make block j_star(b, h) take
    all but ~1e-8 of every row's probability: every query is e_0, and the keys
    are zero except block j_star(b, h), whose keys are 40 e_0 (logit 40 * scale
    against 0 for every other block)."""
    N = nb * bs
    q = np.zeros((B, H, N, D))
    q[..., 0] = 1.0
    k = np.zeros((B, H, N, D))
    for b in range(B):
        for h in range(H):
            j = j_star(b, h)
            k[b, h, j * bs:(j + 1) * bs, 0] = 40.0
    return q, k


def test_estimate_mask_rows_follow_b_h_i_order_at_b_above_1():
    """Closed form at B = 2, H = 3: every row of head (b, h) selects exactly the
    dominant block j*(b, h) = (3b + h) mod nb, and the CSR lists rows in
    (b, h, i) order -- so a head order of (h, b) or a head's rows read from
    another head shows up as a wrong block."""
    B, H, nb, bs, D = 2, 3, 5, 16, 4
    j_star = lambda b, h: (3 * b + h) % nb
    q, k = _dominant_block_heads(B, H, nb, bs, D, j_star)
    rp, ci, sels = O.estimate_mask(q, k, bs, 0.5, 0.5)
    assert rp.tolist() == list(range(B * H * nb + 1))
    assert ci.tolist() == [j_star(b, h) for b in range(B) for h in range(H) for _ in range(nb)]
    assert sorted(sels) == [(b, h) for b in range(B) for h in range(H)]


def test_estimate_mask_candidate_rows_are_taken_from_their_own_head():
    """B = 2, H = 3 with single-block candidate rows: a row whose only candidate
    is c keeps exactly c (k* >= 1), whatever the logits.  The candidate of row
    r = (b*H + h)*nb + i is c(b, h, i) = (7(bH + h) + 2i) mod nb, different for
    the two b of one h, so reading head (b, h)'s candidates from any other
    head's rows changes the output."""
    B, H, nb, bs, D = 2, 3, 5, 16, 4
    rng = np.random.default_rng(61)
    q = rng.normal(size=(B, H, nb * bs, D))
    k = rng.normal(size=(B, H, nb * bs, D))
    c = lambda b, h, i: (7 * (b * H + h) + 2 * i) % nb
    want = [c(b, h, i) for b in range(B) for h in range(H) for i in range(nb)]
    cand = (np.arange(B * H * nb + 1), np.array(want))
    rp, ci, _ = O.estimate_mask(q, k, bs, 0.9, 0.5, candidate=cand)
    assert rp.tolist() == list(range(B * H * nb + 1))
    assert ci.tolist() == want
    # with the same dominant-block inputs as above, a two-block candidate row
    # {c, j*} keeps j* alone (probability ~1 - 1e-8 >= p), and {c} alone when
    # c == j* -- rows again read from their own head only
    j_star = lambda b, h: (3 * b + h) % nb
    q2, k2 = _dominant_block_heads(B, H, nb, bs, D, j_star)
    rows = [np.unique([c(b, h, i), j_star(b, h)]) for b in range(B) for h in range(H) for i in range(nb)]
    rp2, ci2, _ = O.estimate_mask(q2, k2, bs, 0.5, 0.5, candidate=O.rows_to_csr(rows))
    assert ci2.tolist() == [j_star(b, h) for b in range(B) for h in range(H) for _ in range(nb)]


def test_estimate_mask_random_candidates_equal_per_head_rows():
    """B = 2, H = 3, random candidate CSR: every row r = (b*H + h)*nb + i of the
    whole-tensor estimator equals the single-head estimator run on head (b, h)
    with that head's candidate rows, sliced out here by explicit row index."""
    B, H, N, bs, D = 2, 3, 300, 64, 8
    rng = np.random.default_rng(62)
    q = rng.normal(size=(B, H, N, D))
    k = rng.normal(size=(B, H, N, D)) + 0.5 * q
    nb = O.num_blocks(N, bs)
    cand_rows = [np.sort(rng.choice(nb, size=int(rng.integers(1, nb + 1)), replace=False))
                 for _ in range(B * H * nb)]
    rp, ci, _ = O.estimate_mask(q, k, bs, 0.7, 0.3, candidate=O.rows_to_csr(cand_rows), keep_prefix_tokens=5)
    for b in range(B):
        for h in range(H):
            mine = [cand_rows[(b * H + h) * nb + i] for i in range(nb)]
            ref = O.estimate_head(q[b, h], k[b, h], bs, 0.7, 0.3, mine, keep_prefix_tokens=5)
            for i in range(nb):
                r = (b * H + h) * nb + i
                assert ci[rp[r]:rp[r + 1]].tolist() == ref[i].selected.tolist(), (b, h, i)


# ----------------------------------------------------------------------------
# pooling
# ----------------------------------------------------------------------------

# ----------------------------------------------------------------------------
# mask narrowing: Top-p over exact block masses
# ----------------------------------------------------------------------------

def test_mass_top_p_hand_worked_fixture():
    rows = [ln for ln in open(os.path.join(GOLDEN, "mass_top_p_hand_worked.txt"))
            if ln.strip() and not ln.startswith("#")]
    assert len(rows) == 12
    for ln in rows:
        ent, masses, p, forced, expect = ln.split("|")
        ent = np.array(_ints(ent), dtype=np.int64)
        m = np.array([float(t) for t in masses.split()] if masses.strip() != "-" else [], dtype=np.float64)
        sel = O.top_p_from_mass(ent, m, float(p), np.array(_ints(forced), dtype=np.int64))
        assert sel.selected.tolist() == _ints(expect), ln


def _brute_force_mass(m, p):
    """Smallest subset whose share of the total reaches p; then largest mass; then lowest ids."""
    n = len(m)
    z = sum(m)
    for size in range(1, n + 1):
        best = None
        for sub in itertools.combinations(range(n), size):
            s = sum(m[j] for j in sub) / z
            if s >= p and (best is None or s > best[0] + 1e-12):
                best = (s, sub)
        if best is not None:
            return sorted(best[1])
    return list(range(n))


def test_mass_top_p_brute_force_small_rows():
    rng = np.random.default_rng(21)
    checked = 0
    while checked < 200:
        n = int(rng.integers(1, 10))
        m = rng.dirichlet(np.full(n, 0.7)) * float(rng.uniform(0.5, 2.0))
        p = float(rng.uniform(0.05, 0.99))
        shares = [x / m.sum() for x in m]
        if _subset_margin(shares, p) < 1e-9:
            continue
        ent = np.sort(rng.choice(64, n, replace=False))
        expect = ent[_brute_force_mass(m.tolist(), p)].tolist()
        got = O.top_p_from_mass(ent, m, p)
        assert got.selected.tolist() == expect
        checked += 1


def test_mass_top_p_equals_estimator_rule_on_softmax_weights():
    # Masses equal to the softmax of some logits must select what the
    # estimator's rule selects from those logits (two independent code paths:
    # exp/normalise there, given shares here).
    rng = np.random.default_rng(22)
    for _ in range(300):
        n = int(rng.integers(1, 120))
        logits = rng.normal(0, 2.5, n)
        p = float(rng.uniform(0.1, 0.99))
        ent = np.sort(rng.choice(4096, n, replace=False))
        a = O.top_p_select(ent, logits, p)
        w = np.exp(logits - logits.max())
        b = O.top_p_from_mass(ent, w / w.sum(), p)
        band = O.selection_band(a, p, tol=1e-9, mass_tol=1e-9)
        assert set(a.selected.tolist()) ^ set(b.selected.tolist()) <= band


def test_narrow_by_mass_on_forward_masses():
    # The forward's exact masses narrow a mask to a subset; p = 1 keeps it.
    rng = np.random.default_rng(23)
    B, H, N, D, bs = 1, 2, 700, 64, 64
    nb = O.num_blocks(N, bs)
    Q, K, V = (rng.normal(size=(B, H, N, D)) for _ in range(3))
    rp, ci = _random_mask(rng, B, H, nb, empty_rows=True)
    _, _, mass = O.sparse_forward(Q, K, V, bs, rp, ci, 0.125)
    rp1, ci1, _ = O.narrow_by_mass(rp, ci, mass, 1.0, 0, bs, nb)
    assert rp1.tolist() == list(rp) and ci1.tolist() == list(ci)
    rp2, ci2, sels = O.narrow_by_mass(rp, ci, mass, 0.8, 0, bs, nb)
    for r in range(rp.size - 1):
        before = set(ci[rp[r]:rp[r + 1]].tolist())
        after = set(ci2[rp2[r]:rp2[r + 1]].tolist())
        assert after <= before
        if before:
            kept = sum(mass[rp[r] + sorted(before).index(j)] for j in after)
            assert kept >= 0.8 * mass[rp[r]:rp[r + 1]].sum() - 1e-12


def test_mass_top_p_negative_and_nan_masses_count_as_zero():
    # entries 0, 1, 2, 3 with masses 0.6, -0.5, 0.4, NaN: the total is 1.0
    # (the negative and the NaN count as 0), the ranking is 0, 2, then the two
    # zero masses in ascending id, so C = 0.6, 1.0, 1.0, 1.0 and p = 0.9 keeps
    # {0, 2}.  (Taking -0.5 at face value would give a total of 0.5 and keep
    # {0} alone.)
    sel = O.top_p_from_mass(np.array([0, 1, 2, 3]), np.array([0.6, -0.5, 0.4, np.nan]), 0.9)
    assert sel.ranked.tolist() == [0, 2, 1, 3]
    assert np.allclose(sel.cumulative, [0.6, 1.0, 1.0, 1.0], rtol=0, atol=1e-15)
    assert sel.selected.tolist() == [0, 2]
    # a row whose masses are all <= 0 has total 0 and keeps every entry
    assert O.top_p_from_mass(np.array([3, 5]), np.array([-1.0, 0.0]), 0.5).selected.tolist() == [3, 5]


def test_narrow_by_mass_ignores_ids_outside_the_grid():
    # nb = 4: the row lists blocks 0, 5 and 1 with masses 0.2, 0.7 and 0.1.
    # Block 5 does not exist, so the row is {0: 0.2, 1: 0.1}, total 0.3, and
    # p = 0.6 keeps block 0 alone (C_1 = 2/3).  Counting block 5 would keep
    # {5} instead.
    rp, ci, _ = O.narrow_by_mass(np.array([0, 3]), np.array([0, 5, 1]), np.array([0.2, 0.7, 0.1]), 0.6, 0, 64, 4)
    assert rp.tolist() == [0, 1] and ci.tolist() == [0]
    rp, ci, _ = O.narrow_by_mass(np.array([0, 2]), np.array([-1, 2]), np.array([0.9, 0.1]), 0.5, 0, 64, 4)
    assert rp.tolist() == [0, 1] and ci.tolist() == [2]


def test_selection_band_hand_worked():
    # The band excuses GPU/oracle differences: a block is in it when its
    # logit is within tol of the cut seen from the other side, or when its
    # inclusion hinges on a cumulative share within mass_tol of p; forced
    # blocks never are.  Logits 2.0, 1.0, 1.0 + g, 0.0 for blocks 0..3 rank
    # 0, 2, 1, 3; with e = exp: C_1 = e^2 / Z, C_2 = (e^2 + e^(1+g)) / Z.
    def row(g, p, forced=()):
        return O.top_p_select(np.arange(4), np.array([2.0, 1.0, 1.0 + g, 0.0]), p, np.array(forced, dtype=np.int64))

    # p midway between C_1 ~ 0.534 and C_2 ~ 0.731: k* = 2, the cut lies
    # between block 2 (kept) and block 1 (dropped), 5e-5 apart: both within
    # 1e-4 of the other side, nothing near a cumulative share.
    a = row(5e-5, 0.63)
    assert a.k_star == 2 and a.selected.tolist() == [0, 2]
    assert O.selection_band(a, 0.63) == {1, 2}
    # 1.5e-4 apart: neither is within 1e-4 of the other side.
    b = row(1.5e-4, 0.63)
    assert b.k_star == 2 and O.selection_band(b, 0.63) == set()
    # p just above C_2: k* = 3 (block 1 is kept because C_2 < p), and block 1
    # is the rank-3 block whose inclusion hinges on C_2 being within 1e-5 of
    # p; the value clause adds nothing (block 3 is 1.0 below block 1).
    z = np.exp([2.0, 1.0, 1.0 + 1.5e-4, 0.0]).sum()
    p = float((np.exp(2.0) + np.exp(1.0 + 1.5e-4)) / z + 1e-7)
    c = row(1.5e-4, p)
    assert c.k_star == 3 and O.selection_band(c, p) == {1}
    # the same with block 1 forced: forced blocks are never in the band
    assert O.selection_band(row(1.5e-4, p, forced=[1]), p) == set()
    # p = 1 keeps every block and has no band
    assert O.selection_band(row(5e-5, 1.0), 1.0) == set()


def test_mass_band_hand_worked():
    # entries 4, 7, 9 with masses 0.25, 0.5, 0.25 rank 7, 4, 9 (equal masses
    # in ascending id), C = 0.5, 0.75, 1.0 exactly.  At p = 0.75 the rank-3
    # block (9) is dropped only because C_2 reaches p exactly: it is the band.
    sel = O.top_p_from_mass(np.array([4, 7, 9]), np.array([0.25, 0.5, 0.25]), 0.75)
    assert sel.ranked.tolist() == [7, 4, 9] and sel.selected.tolist() == [4, 7]
    assert O.mass_band(sel, 0.75) == {9}
    assert O.mass_band(sel, 0.74) == set()
    forced = O.top_p_from_mass(np.array([4, 7, 9]), np.array([0.25, 0.5, 0.25]), 0.75, np.array([9]))
    assert O.mass_band(forced, 0.75) == set()


# ----------------------------------------------------------------------------
# token permutation
# ----------------------------------------------------------------------------

def test_permute_rows_by_hand_and_round_trip():
    x = np.arange(2 * 5 * 3, dtype=np.float64).reshape(2, 5, 3)
    perm = np.array([3, 0, 4, 1, 2])
    y = O.permute_rows(x, perm)
    assert y[0, 0].tolist() == x[0, 3].tolist() and y[1, 2].tolist() == x[1, 4].tolist()
    assert y[0, :, 0].tolist() == [9.0, 0.0, 12.0, 3.0, 6.0]                 # rows 3, 0, 4, 1, 2 of head 0
    assert (O.permute_rows(y, perm, inverse=True) == x).all()
    assert (O.permute_rows(x, np.arange(5)) == x).all()
    rng = np.random.default_rng(31)
    p1, p2 = rng.permutation(5), rng.permutation(5)
    assert (O.permute_rows(O.permute_rows(x, p1), p2) == O.permute_rows(x, p1[p2])).all()
    bad = np.array([0, 7, 1, -1, 2])
    z = O.permute_rows(x, bad)
    assert (z[:, 1] == 0).all() and (z[:, 3] == 0).all() and (z[:, 4] == x[:, 2]).all()
    w = O.permute_rows(x, bad, inverse=True)
    assert (w[:, 0] == x[:, 0]).all() and (w[:, 1] == x[:, 2]).all() and (w[:, 3] == 0).all()


# ----------------------------------------------------------------------------
# structured head masks
# ----------------------------------------------------------------------------

def _token_relation(kind, N, prefix, F, block, band, period, stripes):
    """Explicit N x N token relation (pattern definitions on token pairs), lifted
    to blocks by 'any pair related'; block patterns use block ids of tokens."""
    n = np.arange(N)
    text = n < prefix
    frame = np.where(text, -1, (n - prefix) // F)
    spot = np.where(text, -1, (n - prefix) % F)
    blk = n // block
    dq, dk = np.meshgrid(blk, blk, indexing="ij")
    d = dq - dk
    if kind == O.PATTERN_DENSE:
        tok = np.ones((N, N), dtype=bool)
    elif kind == O.PATTERN_SPATIAL:
        tok = frame[:, None] == frame[None, :]
    elif kind == O.PATTERN_TEMPORAL:
        tok = spot[:, None] == spot[None, :]
    elif kind == O.PATTERN_DIAGONAL:
        tok = np.abs(d) <= band
    elif kind == O.PATTERN_MULTI_DIAGONAL:
        r = np.mod(d, period)
        tok = np.minimum(r, period - r) <= band
    else:
        tok = np.isin(dk, list(stripes)) | (np.abs(d) <= band)
    tok = tok | text[:, None] | text[None, :]
    nb = O.num_blocks(N, block)
    out = np.zeros((nb, nb), dtype=bool)
    np.logical_or.at(out, (dq.ravel(), dk.ravel()), tok.ravel())
    return out


@pytest.mark.parametrize("kind", range(6))
def test_structured_mask_equals_token_level_lifting(kind):
    for N, prefix, F, block, band, period in [(700, 30, 50, 64, 1, 3), (1000, 0, 96, 64, 0, 4),
                                              (513, 200, 31, 128, 2, 2), (900, 77, 120, 64, 1, 5)]:
        stripes = (0, 5, 9)
        got = O.structured_block_mask(kind, N, block, prefix, F, band, period, stripes)
        ref = _token_relation(kind, N, prefix, F, block, band, period, stripes)
        assert (got == ref).all(), (kind, N, prefix, F, block)


def test_structured_mask_special_cases():
    N, bs = 1000, 64
    nb = O.num_blocks(N, bs)
    dense = np.ones((nb, nb), dtype=bool)
    assert (O.structured_block_mask(O.PATTERN_SPATIAL, N, bs, 0, N, 0, 0) == dense).all()       # one frame
    assert (O.structured_block_mask(O.PATTERN_TEMPORAL, N, bs, 0, 1, 0, 0) == dense).all()      # one position
    assert (O.structured_block_mask(O.PATTERN_DIAGONAL, N, bs, 0, 10, nb, 0) == dense).all()
    assert (O.structured_block_mask(O.PATTERN_MULTI_DIAGONAL, N, bs, 0, 10, 0, 1) == dense).all()
    eye = O.structured_block_mask(O.PATTERN_STRIPES, N, bs, 0, 10, 0, 0, ())
    assert (eye == np.eye(nb, dtype=bool)).all()
    far = O.structured_block_mask(O.PATTERN_MULTI_DIAGONAL, N, bs, 0, 10, 1, 3 * nb)
    assert (far == O.structured_block_mask(O.PATTERN_DIAGONAL, N, bs, 0, 10, 1, 0)).all()
    for kind in (O.PATTERN_SPATIAL, O.PATTERN_TEMPORAL, O.PATTERN_DIAGONAL, O.PATTERN_MULTI_DIAGONAL):
        m = O.structured_block_mask(kind, 1500, 64, 100, 130, 1, 4)
        assert (m == m.T).all()
        assert m[0].all() and m[:, 0].all()          # the text block is kept by and keeps everything


def test_pool_blocks_matches_loop_on_ragged_tail():
    rng = np.random.default_rng(6)
    x = rng.normal(size=(37, 3))
    got = O.pool_blocks(x, 8)
    assert got.shape == (5, 3)
    for i in range(5):
        toks = [t for t in range(37) if t // 8 == i]
        for d in range(3):
            assert got[i, d] == pytest.approx(sum(x[t, d] for t in toks) / len(toks), abs=1e-14)
    assert len(toks) == 5


# ----------------------------------------------------------------------------
# sparse attention
# ----------------------------------------------------------------------------

def _dense_reference(q, k, v, scale):
    s = scale * q @ k.T
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    lse = np.log(np.exp(s).sum(axis=1))
    return p @ v, lse, p


def test_all_blocks_equals_dense_softmax_attention():
    rng = np.random.default_rng(7)
    B, H, N, D, bs = 1, 2, 200, 16, 64
    Q, K, V = (rng.normal(size=(B, H, N, D)) for _ in range(3))
    scale = 1 / math.sqrt(D)
    row_ptr, col_idx, _ = O.estimate_mask(Q, K, bs, 1.0, scale)
    nb = O.num_blocks(N, bs)
    assert np.diff(row_ptr).tolist() == [nb] * (B * H * nb)
    Ob, L, M = O.sparse_forward(Q, K, V, bs, row_ptr, col_idx, scale)
    for h in range(H):
        o, lse, p = _dense_reference(Q[0, h], K[0, h], V[0, h], scale)
        assert np.abs(Ob[0, h] - o).max() < 1e-12
        assert np.abs(L[0, h] - lse).max() < 1e-12
        for i in range(nb):
            r = h * nb + i
            qs = slice(i * bs, min((i + 1) * bs, N))
            for e in range(row_ptr[r], row_ptr[r + 1]):
                j = col_idx[e]
                ks = slice(j * bs, min((j + 1) * bs, N))
                assert M[e] == pytest.approx(p[qs, ks].sum(axis=1).mean(), abs=1e-12)


def _random_mask(rng, B, H, nb, empty_rows=True):
    rows = []
    for _ in range(B * H * nb):
        if empty_rows and rng.random() < 0.1:
            rows.append(np.zeros(0, np.int64))
        else:
            rows.append(np.sort(rng.choice(nb, size=int(rng.integers(1, nb + 1)), replace=False)))
    return O.rows_to_csr(rows)


def test_block_mask_equals_explicit_token_mask():
    rng = np.random.default_rng(8)
    B, H, N, D, bs = 2, 2, 150, 8, 32        # 5 blocks, last one holds 22 tokens
    Q, K, V = (rng.normal(size=(B, H, N, D)) for _ in range(3))
    nb = O.num_blocks(N, bs)
    row_ptr, col_idx = _random_mask(rng, B, H, nb)
    scale = 0.3
    Ob, L, M = O.sparse_forward(Q, K, V, bs, row_ptr, col_idx, scale)
    for b in range(B):
        for h in range(H):
            allow = np.zeros((N, N), bool)
            for i in range(nb):
                r = (b * H + h) * nb + i
                for j in col_idx[row_ptr[r]:row_ptr[r + 1]]:
                    allow[i * bs:(i + 1) * bs, j * bs:(j + 1) * bs] = True
            s = np.where(allow, scale * Q[b, h] @ K[b, h].T, -np.inf)
            has = allow.any(axis=1)
            m = np.where(has, s.max(axis=1), 0.0)
            e = np.exp(s - m[:, None])
            z = e.sum(axis=1)
            p = np.divide(e, z[:, None], out=np.zeros_like(e), where=has[:, None])
            assert np.abs(Ob[b, h] - p @ V[b, h]).max() < 1e-12
            lse = np.where(has, m + np.log(np.where(has, z, 1.0)), -np.inf)
            assert np.array_equal(np.isinf(L[b, h]), ~has)
            assert np.abs(L[b, h][has] - lse[has]).max() < 1e-12
            for i in range(nb):
                r = (b * H + h) * nb + i
                for e_ in range(row_ptr[r], row_ptr[r + 1]):
                    j = col_idx[e_]
                    blk = p[i * bs:(i + 1) * bs, j * bs:(j + 1) * bs]
                    assert M[e_] == pytest.approx(blk.sum(axis=1).mean(), abs=1e-12)


def test_tiny_case_against_pure_python_loops():
    rng = np.random.default_rng(9)
    N, D, bs = 11, 3, 4                        # blocks of 4, 4, 3 tokens
    q, k, v = (rng.normal(size=(N, D)) for _ in range(3))
    rows = [np.array([0, 2]), np.array([1]), np.array([0, 1, 2])]
    row_ptr, col_idx = O.rows_to_csr(rows)
    scale = 0.7
    Ob, L, M = O.sparse_forward(q[None, None], k[None, None], v[None, None], bs, row_ptr, col_idx, scale)
    for t in range(N):
        i = t // bs
        keys = [u for j in rows[i] for u in range(j * bs, min(j * bs + bs, N))]
        logit = {u: scale * sum(q[t, d] * k[u, d] for d in range(D)) for u in keys}
        z = sum(math.exp(logit[u]) for u in keys)
        assert L[0, 0, t] == pytest.approx(math.log(z), abs=1e-13)
        for d in range(D):
            o = sum(math.exp(logit[u]) / z * v[u, d] for u in keys)
            assert Ob[0, 0, t, d] == pytest.approx(o, abs=1e-13)
    # mass of (block 0, key block 2): mean over 4 queries of the probability on tokens 8..10
    want = 0.0
    for t in range(4):
        keys = list(range(0, 4)) + list(range(8, 11))
        w = [math.exp(scale * sum(q[t, d] * k[u, d] for d in range(D))) for u in keys]
        want += sum(w[4:]) / sum(w) / 4
    assert M[1] == pytest.approx(want, abs=1e-13)


def test_mass_rows_sum_to_one_and_empty_rows():
    rng = np.random.default_rng(10)
    B, H, N, D, bs = 1, 3, 300, 8, 64
    Q, K, V = (rng.normal(size=(B, H, N, D)) for _ in range(3))
    nb = O.num_blocks(N, bs)
    row_ptr, col_idx = _random_mask(rng, B, H, nb)
    Ob, L, M = O.sparse_forward(Q, K, V, bs, row_ptr, col_idx, 0.4)
    assert (M >= 0).all()
    for r in range(B * H * nb):
        a, b = row_ptr[r], row_ptr[r + 1]
        h, i = divmod(r, nb)
        span = slice(i * bs, min(i * bs + bs, N))
        if a == b:
            assert (Ob[0, h, span] == 0).all() and np.isneginf(L[0, h, span]).all()
        else:
            assert M[a:b].sum() == pytest.approx(1.0, abs=1e-12)


def test_executed_pairs_counts_valid_token_pairs():
    rng = np.random.default_rng(13)
    N, bs, B, H = 150, 32, 1, 2
    nb = O.num_blocks(N, bs)
    row_ptr, col_idx = _random_mask(rng, B, H, nb)
    want = 0
    for r in range(B * H * nb):
        i = r % nb
        nq = min(bs, N - i * bs)
        want += sum(nq * min(bs, N - j * bs) for j in col_idx[row_ptr[r]:row_ptr[r + 1]])
    assert O.executed_pairs(N, bs, B, H, row_ptr, col_idx) == want


# ----------------------------------------------------------------------------
# backward
# ----------------------------------------------------------------------------

def test_backward_matches_central_finite_differences():
    rng = np.random.default_rng(14)
    B, H, N, D, bs = 1, 1, 10, 3, 4
    Q, K, V, G = (rng.normal(size=(B, H, N, D)) for _ in range(4))
    rows = [np.array([0, 2]), np.array([1, 2]), np.array([0, 1, 2])]
    row_ptr, col_idx = O.rows_to_csr(rows)
    scale = 0.6
    dQ, dK, dV = O.sparse_backward(Q, K, V, G, bs, row_ptr, col_idx, scale)

    def loss(q, k, v):
        o, _, _ = O.sparse_forward(q, k, v, bs, row_ptr, col_idx, scale)
        return float((o * G).sum())

    h = 1e-6
    for which, grad in ((0, dQ), (1, dK), (2, dV)):
        for t in range(N):
            for d in range(D):
                args = [Q.copy(), K.copy(), V.copy()]
                args[which][0, 0, t, d] += h
                up = loss(*args)
                args[which][0, 0, t, d] -= 2 * h
                dn = loss(*args)
                fd = (up - dn) / (2 * h)
                assert abs(fd - grad[0, 0, t, d]) <= 1e-6 * max(1.0, abs(fd)), (which, t, d)


def test_backward_dv_closed_form_and_zero_row_sums():
    rng = np.random.default_rng(15)
    B, H, N, D, bs = 1, 1, 90, 5, 32
    Q, K, V, G = (rng.normal(size=(B, H, N, D)) for _ in range(4))
    nb = O.num_blocks(N, bs)
    row_ptr, col_idx = _random_mask(rng, B, H, nb)
    scale = 0.5
    dQ, dK, dV = O.sparse_backward(Q, K, V, G, bs, row_ptr, col_idx, scale)
    allow = np.zeros((N, N), bool)
    for i in range(nb):
        for j in col_idx[row_ptr[i]:row_ptr[i + 1]]:
            allow[i * bs:(i + 1) * bs, j * bs:(j + 1) * bs] = True
    s = np.where(allow, scale * Q[0, 0] @ K[0, 0].T, -np.inf)
    has = allow.any(axis=1)
    e = np.exp(s - np.where(has, s.max(axis=1), 0.0)[:, None])
    p = np.divide(e, e.sum(axis=1)[:, None], out=np.zeros_like(e), where=has[:, None])
    assert np.abs(dV[0, 0] - p.T @ G[0, 0]).max() < 1e-12
    # dS rows sum to zero, so sum_k dS[q,k] * (K_k + c) is independent of c:
    # shifting every key by a constant vector leaves dQ unchanged.
    shift = rng.normal(size=D)
    dQ2, _, _ = O.sparse_backward(Q, K + shift, V, G, bs, row_ptr, col_idx, scale)
    # the shift changes the logits by scale*q.shift per query row, which the
    # softmax removes, so P (and dS) are unchanged and dQ moves by scale*dS@shift = 0
    assert np.abs(dQ2 - dQ).max() < 1e-10


# ----------------------------------------------------------------------------
# hierarchical block scoring (reading of the DFSAttn page, Abstract)
# ----------------------------------------------------------------------------

def test_hierarchical_hand_worked_fixture():
    rows, q, k = [], None, None
    with open(os.path.join(GOLDEN, "hier_stripe_hand_worked.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            head, rest = [x.strip() for x in line.split("|", 1)]
            if head in ("q", "k"):
                arr = np.array([[float(v) for v in t.split(",")] for t in rest.split()])
                if head == "q":
                    q = arr
                else:
                    k = arr
                continue
            p, sel = [x.strip() for x in rest.split("|")]
            rows.append((int(head), float(p), sorted(int(v) for v in sel.split())))
    assert q.shape == (12, 2) and k.shape == (12, 2) and len(rows) == 7
    for g, p, want in rows:
        for r in O.estimate_head(q, k, 4, p, 1.0, sub_blocks=g):
            assert sorted(r.selected.tolist()) == want, (g, p)


def test_hierarchical_g1_is_mean_pool_logit():
    rng = np.random.default_rng(11)
    q, k = rng.standard_normal((37, 8)), rng.standard_normal((37, 8))
    want = 0.3 * (O.pool_blocks(q, 8) @ O.pool_blocks(k, 8).T)
    np.testing.assert_allclose(O.hierarchical_logits(q, k, 8, 1, 0.3), want, rtol=0, atol=1e-14)


@pytest.mark.parametrize("g", [2, 4, 8])
def test_hierarchical_block_probability_is_sum_of_sub_block_probabilities(g):
    # pure-Python loops over tokens: sub-block means (ragged tail), a softmax
    # over every sub-block of the row, summed per key block
    rng = np.random.default_rng(20 + g)
    N, D, bs, scale = 37, 3, 16, 0.7
    q, k = rng.standard_normal((N, D)), rng.standard_normal((N, D))
    nb = -(-N // bs)
    w = bs // g
    qbar, parts = [], []
    for i in range(nb):
        toks = range(i * bs, min((i + 1) * bs, N))
        qbar.append([sum(q[t][d] for t in toks) / len(toks) for d in range(D)])
        for a in range(i * bs, i * bs + bs, w):
            toks = range(a, min(a + w, (i + 1) * bs, N))
            if len(toks):
                parts.append((i, [sum(k[t][d] for t in toks) / len(toks) for d in range(D)]))
    lg = O.hierarchical_logits(q, k, bs, g, scale)
    for i in range(nb):
        sub = [scale * sum(qbar[i][d] * kb[d] for d in range(D)) for _, kb in parts]
        m = max(sub)
        e = [math.exp(x - m) for x in sub]
        tot = sum(e)
        want = [0.0] * nb
        for (j, _), x in zip(parts, e):
            want[j] += x / tot
        got = np.exp(lg[i] - lg[i].max())
        got /= got.sum()
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
