"""Plain CPU float64 oracle for dynamic block-sparse attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The HIP product
path never calls it and shares no code with it.

What it computes, in the order the method runs:

* Block-importance estimator (the two-stage estimate-then-attend scheme of the
  DSV page, Abstract; Top-p selection of the GSRS page, Abstract; candidate
  restriction = "reduced search", GSRS page, Abstract and Figure 4 caption):
  mean-pool Q and K over each token block, score the pooled pairs
  scale * <Qbar_i, Kbar_j>, take a softmax over each query block's row (over
  the candidate blocks only when a candidate mask is given), rank the row by
  (logit descending, block index ascending) and keep the shortest prefix
  whose cumulative probability reaches p; blocks that hold prefix (text)
  tokens are added afterwards.
* Hierarchical block scoring (DFSAttn page, Abstract; named there without a
  definition -- the reading is stated at ``hierarchical_logits``): block
  logits as the log-sum-exp of the query block mean against the key block's
  sub-block means, then the same softmax, Top-p and forced blocks.
* Mask narrowing: Top-p over the exact block attention weights of an earlier
  step, restricted to that step's blocks (GSRS page, Abstract; Figure 4
  caption) -- the same ranking and cut as the estimator, applied to masses.
* Token permutation (gather into a space-filling-curve order, scatter back).
* Structured head masks: the SVG page's spatial and temporal heads and the
  Sparse-vDiT page's diagonal, multi-diagonal and vertical-stripe patterns
  (both Abstracts), lifted from token pairs to block pairs.
* Sparse attention over the selected key blocks, computed with whole rows
  (no online rescaling): O, the per-query log-sum-exp and the exact
  attention mass of every (query block, key block) pair -- the block-level
  attention map of the GSRS page, Figure 3 caption, whose exact weights the
  GSRS abstract obtains inside the attention computation.
* The gradients of sum(O * G) over the same mask (the DSV page trains with
  sparse attention, Abstract).

Inputs are the exact tensors the GPU consumes, upcast to float64, with the
same float32 ``top_p`` and ``scale``.  Everything here is float64 numpy; a
matrix product or a cumulative sum is the only library primitive used.

Pins (tests/test_oracle_pins.py) tie each function to something other than
itself: brute-force subset search for Top-p, uniform and duplicated-block
tie cases in exact arithmetic, the dense softmax special case, an explicit
token-level mask, pure-Python loops on tiny inputs, row sums of the mass and
central finite differences for the gradients.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


# ----------------------------------------------------------------------------
# blocks and pooling
# ----------------------------------------------------------------------------

def num_blocks(n_tokens: int, block: int) -> int:
    return -(-n_tokens // block)


def block_spans(n_tokens: int, block: int) -> list[tuple[int, int]]:
    """Token range [lo, hi) of every block; the last one may be partial."""
    return [(i * block, min((i + 1) * block, n_tokens)) for i in range(num_blocks(n_tokens, block))]


def pool_blocks(x: np.ndarray, block: int) -> np.ndarray:
    """Mean of the valid tokens of each block: x [N, D] -> [nb, D] (float64)."""
    x = np.asarray(x, dtype=np.float64)
    spans = block_spans(x.shape[0], block)
    return np.stack([x[lo:hi].mean(axis=0) for lo, hi in spans])


def sub_block_spans(n_tokens: int, block: int, sub_blocks: int) -> list[list[tuple[int, int]]]:
    """Token ranges of the sub-blocks of every block: block j splits into
    ``sub_blocks`` parts of block // sub_blocks tokens; parts that start past
    the last token are dropped, so a partial last block keeps its non-empty
    parts (the last of them possibly partial)."""
    w = block // sub_blocks
    return [[(a, min(a + w, hi)) for a in range(lo, lo + block, w) if a < hi]
            for lo, hi in block_spans(n_tokens, block)]


def hierarchical_logits(q: np.ndarray, k: np.ndarray, block: int, sub_blocks: int, scale: float) -> np.ndarray:
    """Block logits of hierarchical block scoring for one (b, h): [nb, nb].

    Reading of the DFSAttn page's hierarchical block scoring (Abstract; the
    page gives no definition): each query block's mean is scored against the
    means of the key block's sub-blocks, scale * <Qbar_i, Kbar_{j,m}>, and the
    key block's logit is the natural log-sum-exp over its non-empty sub-blocks.
    A block's softmax probability is then the sum of its sub-blocks'
    probabilities under a softmax over all sub-blocks, so one strongly matched
    sub-block is not averaged away.  sub_blocks = 1 is the mean-pool logit.
    """
    qbar = pool_blocks(q, block)
    k = np.asarray(k, dtype=np.float64)
    spans = sub_block_spans(k.shape[0], block, sub_blocks)
    out = np.empty((qbar.shape[0], len(spans)))
    for j, parts in enumerate(spans):
        ksub = np.stack([k[a:b].mean(axis=0) for a, b in parts])     # [parts, D]
        s = float(scale) * (qbar @ ksub.T)                            # [nb, parts]
        mx = s.max(axis=1)
        out[:, j] = mx + np.log(np.exp(s - mx[:, None]).sum(axis=1))
    return out


def forced_blocks(keep_prefix_tokens: int, block: int, nb: int) -> np.ndarray:
    """Key blocks that intersect the always-kept token prefix [0, keep_prefix_tokens)."""
    return np.array([j for j in range(nb) if j * block < keep_prefix_tokens], dtype=np.int64)


# ----------------------------------------------------------------------------
# Top-p over one row of pooled scores
# ----------------------------------------------------------------------------

@dataclass
class RowSelection:
    candidates: np.ndarray   # candidate block ids, ascending
    logits: np.ndarray       # their pooled logits, aligned with candidates
    ranked: np.ndarray       # candidate ids in rank order (logit desc, id asc)
    cumulative: np.ndarray   # C_r, cumulative probability of the top r, r = 1..n
    k_star: int              # number of ranked blocks Top-p keeps
    forced: np.ndarray       # blocks added regardless of score
    selected: np.ndarray     # final ascending block list


def top_p_select(candidates: np.ndarray, logits: np.ndarray, top_p: float,
                 forced: np.ndarray | None = None) -> RowSelection:
    """Top-p over the softmax of ``logits`` (GSRS page, Abstract: Top-p selection).

    The row is ranked by logit, larger first, the lower block index first on
    equal logits; k* is the smallest r with C_r >= p (all of them when p >= 1
    or when rounding keeps C_n below p).  Forced blocks join after the cut and
    do not change k*.
    """
    cand = np.asarray(candidates, dtype=np.int64)
    s = np.asarray(logits, dtype=np.float64)
    forced = np.zeros(0, dtype=np.int64) if forced is None else np.asarray(forced, dtype=np.int64)
    n = cand.size
    if n == 0:
        return RowSelection(cand, s, cand, np.zeros(0), 0, forced, np.unique(forced))
    order = np.lexsort((cand, -s))            # primary: -logit, secondary: id
    ranked = cand[order]
    e = np.exp(s - s.max())
    prob = e / e.sum()
    cum = np.cumsum(prob[order])
    p = float(top_p)
    if p >= 1.0:
        k_star = n
    else:
        hit = np.nonzero(cum >= p)[0]
        k_star = int(hit[0]) + 1 if hit.size else n
    sel = np.union1d(ranked[:k_star], forced).astype(np.int64)
    return RowSelection(cand, s, ranked, cum, k_star, forced, sel)


def selection_band(row: RowSelection, top_p: float, tol: float = 1e-4,
                   mass_tol: float = 1e-5) -> set[int]:
    """Blocks whose selection a rounding-level change of the scores could flip.

    The cut lies between the last kept logit s_last (rank k*) and the first
    dropped logit s_next (rank k*+1).  A block is in the band when
    (1) its logit lies within ``tol`` of the cut seen from the other side:
        a kept block with s <= s_next + tol, or a dropped block with
        s >= s_last - tol (such a block could trade places across the cut);
    (2) it sits at rank r >= 2 with |C_{r-1} - p| <= mass_tol, so that its
        inclusion hinges on the cumulative sum (float32 logits and sums on
        the GPU move C_r by about 1e-6; mass_tol leaves a tenfold margin).
    Forced blocks are never in the band.  Outside it the list is unique.
    """
    n = row.ranked.size
    if n == 0 or float(top_p) >= 1.0:
        return set()
    p = float(top_p)
    s_of = dict(zip(row.candidates.tolist(), row.logits.tolist()))
    band: set[int] = set()
    if row.k_star < n:
        s_last = s_of[int(row.ranked[row.k_star - 1])]
        s_next = s_of[int(row.ranked[row.k_star])]
        for r, j in enumerate(row.ranked.tolist()):
            s = s_of[j]
            if (r < row.k_star and s <= s_next + tol) or (r >= row.k_star and s >= s_last - tol):
                band.add(j)
    for r in range(2, n + 1):
        if abs(row.cumulative[r - 2] - p) <= mass_tol:
            band.add(int(row.ranked[r - 1]))
    return band - set(row.forced.tolist())


def top_p_from_mass(entries: np.ndarray, mass: np.ndarray, top_p: float,
                    forced: np.ndarray | None = None) -> RowSelection:
    """Top-p over a row's exact block attention weights (mask narrowing).

    The GSRS page (Abstract) evaluates exact attention weights inside the
    attention computation and restricts later search steps to the blocks an
    earlier step kept (Abstract; Figure 4 caption); its Figure 3 caption
    describes the block-level map those weights form.  Narrowing applies the
    same Top-p rule as ``top_p_select`` to those weights instead of to a
    softmax of pooled scores: the row's entries are ranked by mass, larger
    first, the lower block index first on equal masses, and k* is the smallest
    r whose cumulative share C_r = (sum of the top r masses) / (row total)
    reaches p.  A negative or NaN mass counts as 0; a row whose total is 0
    keeps every entry (C_n never reaches p); a block listed twice counts once,
    with its first mass.  Forced blocks join after the cut.  The result lists
    ascending block ids.
    """
    ent = np.asarray(entries, dtype=np.int64)
    m = np.asarray(mass, dtype=np.float64)
    m = np.where(m > 0, m, 0.0)               # NaN > 0 is False
    _, first = np.unique(ent, return_index=True)
    first = np.sort(first)
    ent, m = ent[first], m[first]
    forced = np.zeros(0, dtype=np.int64) if forced is None else np.asarray(forced, dtype=np.int64)
    n = ent.size
    if n == 0:
        return RowSelection(ent, m, ent, np.zeros(0), 0, forced, np.unique(forced))
    order = np.lexsort((ent, -m))             # primary: -mass, secondary: id
    ranked = ent[order]
    total = m.sum()
    p = float(top_p)
    if total <= 0.0:
        cum = np.zeros(n)
        k_star = n
    else:
        cum = np.cumsum(m[order]) / total
        if p >= 1.0:
            k_star = n
        else:
            hit = np.nonzero(cum >= p)[0]
            k_star = int(hit[0]) + 1 if hit.size else n
    sel = np.union1d(ranked[:k_star], forced).astype(np.int64)
    return RowSelection(ent, m, ranked, cum, k_star, forced, sel)


def narrow_by_mass(row_ptr: np.ndarray, col_idx: np.ndarray, mass: np.ndarray, top_p: float,
                   keep_prefix_tokens: int, block: int, nb: int):
    """Narrow a CSR mask with ``top_p_from_mass`` row by row.

    ``mass`` is aligned with ``col_idx`` (the forward's block mass).  Returns
    (row_ptr, col_idx, selections).  Entry ids outside [0, nb) are ignored.
    """
    forced = forced_blocks(keep_prefix_tokens, block, nb)
    rp = np.asarray(row_ptr, dtype=np.int64)
    ci = np.asarray(col_idx, dtype=np.int64)
    ms = np.asarray(mass, dtype=np.float64)
    sels = []
    for r in range(rp.size - 1):
        ent, m = ci[rp[r]:rp[r + 1]], ms[rp[r]:rp[r + 1]]
        ok = (ent >= 0) & (ent < nb)
        sels.append(top_p_from_mass(ent[ok], m[ok], top_p, forced))
    out_rp, out_ci = rows_to_csr([s.selected for s in sels])
    return out_rp, out_ci, sels


def mass_band(row: RowSelection, top_p: float, mass_tol: float = 1e-5) -> set[int]:
    """Blocks whose narrowing a rounding-level change of the cumulative share
    could flip: rank r >= 2 with |C_{r-1} - p| <= mass_tol.  The masses
    themselves are the same float32 values on both sides, so the ranking is
    exact; only the summation order differs (float32 on the GPU).
    """
    n = row.ranked.size
    if n == 0 or float(top_p) >= 1.0 or row.cumulative.size == 0 or row.cumulative[-1] == 0.0:
        return set()
    p = float(top_p)
    band = {int(row.ranked[r - 1]) for r in range(2, n + 1) if abs(row.cumulative[r - 2] - p) <= mass_tol}
    return band - set(row.forced.tolist())


# ----------------------------------------------------------------------------
# estimator over whole tensors
# ----------------------------------------------------------------------------

def estimate_head(q: np.ndarray, k: np.ndarray, block: int, top_p: float, scale: float,
                  candidate_rows: list[np.ndarray] | None = None,
                  keep_prefix_tokens: int = 0, sub_blocks: int = 1) -> list[RowSelection]:
    """Estimator for one (b, h): q, k [N, D] -> one RowSelection per query block.
    sub_blocks > 1 scores with ``hierarchical_logits``."""
    if sub_blocks == 1:
        qbar = pool_blocks(q, block)
        kbar = pool_blocks(k, block)
        logits = float(scale) * (qbar @ kbar.T)      # [nb, nb] pooled scores
    else:
        logits = hierarchical_logits(q, k, block, sub_blocks, scale)
    nb = logits.shape[0]
    forced = forced_blocks(keep_prefix_tokens, block, nb)
    rows = []
    for i in range(nb):
        if candidate_rows is None:
            cand = np.arange(nb, dtype=np.int64)
        else:                                # repeated ids count once; ids outside [0, nb) are ignored
            cand = np.unique(np.asarray(candidate_rows[i], dtype=np.int64))
            cand = cand[(cand >= 0) & (cand < nb)]
        rows.append(top_p_select(cand, logits[i, cand], top_p, forced))
    return rows


def csr_rows(row_ptr: np.ndarray, col_idx: np.ndarray) -> list[np.ndarray]:
    row_ptr = np.asarray(row_ptr, dtype=np.int64)
    col_idx = np.asarray(col_idx, dtype=np.int64)
    return [col_idx[row_ptr[r]:row_ptr[r + 1]] for r in range(row_ptr.size - 1)]


def rows_to_csr(rows: list[np.ndarray]) -> tuple[np.ndarray, np.ndarray]:
    counts = np.array([len(r) for r in rows], dtype=np.int64)
    row_ptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    col_idx = np.concatenate([np.asarray(r, dtype=np.int64) for r in rows]) if rows else np.zeros(0, np.int64)
    return row_ptr, col_idx.astype(np.int64)


def estimate_mask(Q: np.ndarray, K: np.ndarray, block: int, top_p: float, scale: float,
                  candidate: tuple[np.ndarray, np.ndarray] | None = None,
                  keep_prefix_tokens: int = 0, heads: list[tuple[int, int]] | None = None,
                  sub_blocks: int = 1):
    """Estimator over [B, H, N, D]; rows ordered (b, h, i).

    Returns (row_ptr, col_idx, selections) where selections maps (b, h) to the
    per-row RowSelection list.  With ``heads`` only those heads are evaluated
    and the CSR covers those rows only, in the order given.
    """
    B, H, N, _ = Q.shape
    nb = num_blocks(N, block)
    cand_rows = csr_rows(*candidate) if candidate is not None else None
    pairs = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    all_rows, sels = [], {}
    for b, h in pairs:
        base = (b * H + h) * nb
        cr = cand_rows[base:base + nb] if cand_rows is not None else None
        rs = estimate_head(Q[b, h], K[b, h], block, top_p, scale, cr, keep_prefix_tokens, sub_blocks)
        sels[(b, h)] = rs
        all_rows.extend(r.selected for r in rs)
    row_ptr, col_idx = rows_to_csr(all_rows)
    return row_ptr, col_idx, sels


# ----------------------------------------------------------------------------
# token permutation (layout transformation)
# ----------------------------------------------------------------------------

def permute_rows(x: np.ndarray, perm: np.ndarray, inverse: bool = False) -> np.ndarray:
    """Reorder the token axis (axis 1 of [heads, N, ...]) by ``perm``.

    Token reordering along a space-filling curve keeps space-time neighbours
    in the same block (DFSAttn page, Abstract; GSRS page, Figure 1, 3 and 6
    captions), and the SVG page (Abstract) pairs its kernels with a layout
    transformation of the tensors.  Gather: y[:, n] = x[:, perm[n]]; inverse
    (scatter, undoing the gather): y[:, perm[n]] = x[:, n].  An entry of perm
    outside [0, N) gives a zero row in a gather and is skipped in a scatter.
    """
    perm = np.asarray(perm, dtype=np.int64)
    N = x.shape[1]
    ok = (perm >= 0) & (perm < N)
    y = np.zeros_like(x)
    if not inverse:
        y[:, ok] = x[:, perm[ok]]
    else:
        y[:, perm[ok]] = x[:, ok]
    return y


# ----------------------------------------------------------------------------
# structured (static) head masks
# ----------------------------------------------------------------------------

# Head kinds of the structured-mask generator.
PATTERN_DENSE, PATTERN_SPATIAL, PATTERN_TEMPORAL, PATTERN_DIAGONAL, PATTERN_MULTI_DIAGONAL, PATTERN_STRIPES = range(6)


def _block_tokens(i: int, block: int, N: int) -> range:
    return range(i * block, min((i + 1) * block, N))


def structured_block_mask(kind: int, N: int, block: int, prefix: int, frame_tokens: int, band: int,
                          period: int, stripes=(), rows=None) -> np.ndarray:
    """Block-level mask [nb, nb] of one head for a structured pattern.

    Token geometry: tokens [0, prefix) are text; a video token n >= prefix sits
    in frame (n - prefix) // F at spatial index (n - prefix) % F, F =
    frame_tokens.  Patterns:
      spatial  (SVG page, Abstract: Spatial Head) -- a video query token
               attends to the video key tokens of its own frame;
      temporal (SVG page, Abstract: Temporal Head) -- to the video key tokens
               at its own spatial index in every frame;
      diagonal / multi-diagonal / vertical-stripe (Sparse-vDiT page,
               Abstract) -- block bands |i - j| <= band; bands around every
               multiple of `period` blocks, |i - j - k period| <= band; the
               listed key blocks for every row plus the band |i - j| <= band;
      dense    -- every pair.
    Every pattern also keeps text: pairs with a text query or text key token
    are related.  A block pair (i, j) is kept iff some token pair of it is
    related (for the block patterns, iff the block relation holds or a text
    token is involved).  With ``rows`` only those query blocks are evaluated
    (the result then has len(rows) rows).
    """
    nb = num_blocks(N, block)
    rows = list(range(nb)) if rows is None else [int(i) for i in rows]
    rel = np.zeros((len(rows), nb), dtype=bool)
    F = max(1, int(frame_tokens))
    stripes = set(int(j) for j in stripes)
    toks = [_block_tokens(i, block, N) for i in range(nb)]
    has_text = [any(n < prefix for n in t) for t in toks]
    frames = [{(n - prefix) // F for n in t if n >= prefix} for t in toks]
    spots = [{(n - prefix) % F for n in t if n >= prefix} for t in toks]
    for ri, i in enumerate(rows):
        for j in range(nb):
            if has_text[i] or has_text[j] or kind == PATTERN_DENSE:
                ok = True
            elif kind == PATTERN_SPATIAL:
                ok = bool(frames[i] & frames[j])
            elif kind == PATTERN_TEMPORAL:
                ok = bool(spots[i] & spots[j])
            elif kind == PATTERN_DIAGONAL:
                ok = abs(i - j) <= band
            elif kind == PATTERN_MULTI_DIAGONAL:
                ok = any(abs(i - j - k * period) <= band for k in range(-nb, nb + 1))
            elif kind == PATTERN_STRIPES:
                ok = j in stripes or abs(i - j) <= band
            else:
                raise ValueError(f"unknown pattern {kind}")
            rel[ri, j] = ok
    return rel


def structured_mask(B: int, H: int, N: int, block: int, kinds, prefix: int, frame_tokens: int, band: int,
                    period: int, stripes=()):
    """CSR over rows (b, h, i) with head (b, h) using pattern kinds[b*H + h]."""
    rows = []
    cache = {}
    for bh in range(B * H):
        kind = int(kinds[bh])
        if kind not in cache:
            cache[kind] = structured_block_mask(kind, N, block, prefix, frame_tokens, band, period, stripes)
        m = cache[kind]
        rows.extend(np.nonzero(m[i])[0].astype(np.int64) for i in range(m.shape[0]))
    return rows_to_csr(rows)


# ----------------------------------------------------------------------------
# sparse attention over selected key blocks
# ----------------------------------------------------------------------------

def _gather(x: np.ndarray, spans, key_blocks) -> tuple[np.ndarray, list[tuple[int, int]]]:
    parts, cols, at = [], [], 0
    for j in key_blocks:
        lo, hi = spans[int(j)]
        parts.append(x[lo:hi])
        cols.append((at, at + hi - lo))
        at += hi - lo
    if not parts:
        return np.zeros((0, x.shape[1])), cols
    return np.concatenate(parts, axis=0), cols


def attend_block(q_blk: np.ndarray, k: np.ndarray, v: np.ndarray, spans, key_blocks,
                 scale: float):
    """One query block against its selected key blocks, whole rows at once.

    Returns O [nq, D], LSE [nq] (natural log) and mass [len(key_blocks)]: the
    mean over the block's queries of the softmax probability that falls in
    each selected key block.  An empty selection gives O = 0, LSE = -inf.
    """
    nq, D = q_blk.shape
    keys, cols = _gather(k, spans, key_blocks)
    vals, _ = _gather(v, spans, key_blocks)
    if keys.shape[0] == 0:
        return np.zeros((nq, D)), np.full(nq, -np.inf), np.zeros(0)
    S = float(scale) * (q_blk @ keys.T)
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    l = E.sum(axis=1, keepdims=True)
    P = E / l
    O = P @ vals
    lse = (m + np.log(l))[:, 0]
    mass = np.array([P[:, a:b].sum(axis=1).mean() for a, b in cols])
    return O, lse, mass


def sparse_forward(Q, K, V, block: int, row_ptr, col_idx, scale: float,
                   rows: list[int] | None = None):
    """O [B,H,N,D], LSE [B,H,N] and mass [nnz] aligned with col_idx.

    With ``rows`` only those CSR rows (r = (b*H + h)*nb + i) are computed; the
    outputs of the other rows are NaN.
    """
    B, H, N, D = Q.shape
    nb = num_blocks(N, block)
    spans = block_spans(N, block)
    row_ptr = np.asarray(row_ptr, dtype=np.int64)
    col_idx = np.asarray(col_idx, dtype=np.int64)
    O = np.full((B, H, N, D), np.nan)
    LSE = np.full((B, H, N), np.nan)
    mass = np.full(col_idx.size, np.nan)
    todo = range(B * H * nb) if rows is None else rows
    for r in todo:
        bh, i = divmod(int(r), nb)
        b, h = divmod(bh, H)
        lo, hi = spans[i]
        kb = col_idx[row_ptr[r]:row_ptr[r + 1]]
        o, lse, ms = attend_block(np.asarray(Q[b, h, lo:hi], np.float64), np.asarray(K[b, h], np.float64),
                                  np.asarray(V[b, h], np.float64), spans, kb, scale)
        O[b, h, lo:hi] = o
        LSE[b, h, lo:hi] = lse
        mass[row_ptr[r]:row_ptr[r + 1]] = ms
    return O, LSE, mass


def sparse_backward(Q, K, V, G, block: int, row_ptr, col_idx, scale: float):
    """Gradients of L = sum(O * G) w.r.t. Q, K, V for a fixed block mask.

    Per query block i with selected keys K_S, V_S and P = softmax(scale Q_i K_S^T):
    dV_S += P^T G_i;  dP = G_i V_S^T;  delta = rowsum(P * dP);
    dS = P * (dP - delta);  dQ_i = scale dS K_S;  dK_S += scale dS^T Q_i.
    """
    B, H, N, D = Q.shape
    nb = num_blocks(N, block)
    spans = block_spans(N, block)
    row_ptr = np.asarray(row_ptr, dtype=np.int64)
    col_idx = np.asarray(col_idx, dtype=np.int64)
    dQ = np.zeros((B, H, N, D))
    dK = np.zeros((B, H, N, D))
    dV = np.zeros((B, H, N, D))
    for b in range(B):
        for h in range(H):
            q = np.asarray(Q[b, h], np.float64)
            k = np.asarray(K[b, h], np.float64)
            v = np.asarray(V[b, h], np.float64)
            g = np.asarray(G[b, h], np.float64)
            for i in range(nb):
                r = (b * H + h) * nb + i
                kb = col_idx[row_ptr[r]:row_ptr[r + 1]]
                if kb.size == 0:
                    continue
                lo, hi = spans[i]
                idx = np.concatenate([np.arange(*spans[int(j)]) for j in kb])
                S = float(scale) * (q[lo:hi] @ k[idx].T)
                E = np.exp(S - S.max(axis=1, keepdims=True))
                P = E / E.sum(axis=1, keepdims=True)
                dP = g[lo:hi] @ v[idx].T
                delta = (P * dP).sum(axis=1, keepdims=True)
                dS = P * (dP - delta)
                dQ[b, h, lo:hi] += float(scale) * (dS @ k[idx])
                np.add.at(dK[b, h], idx, float(scale) * (dS.T @ q[lo:hi]))
                np.add.at(dV[b, h], idx, P.T @ g[lo:hi])
    return dQ, dK, dV


# ----------------------------------------------------------------------------
# work counts used by the measurements
# ----------------------------------------------------------------------------

def executed_pairs(N: int, block: int, B: int, H: int, row_ptr, col_idx) -> int:
    """Sum over selected (i, j) of |Q_i| * |K_j| (valid query-key token pairs)."""
    spans = block_spans(N, block)
    sizes = np.array([hi - lo for lo, hi in spans], dtype=np.int64)
    nb = len(spans)
    row_ptr = np.asarray(row_ptr, dtype=np.int64)
    col_idx = np.asarray(col_idx, dtype=np.int64)
    qsz = np.tile(sizes, B * H)
    csum = np.concatenate([[0], np.cumsum(sizes[col_idx])])
    ksum = csum[row_ptr[1:]] - csum[row_ptr[:-1]]     # valid keys per row
    assert ksum.size == B * H * nb
    return int((qsz * ksum).sum())
