"""GPU parity of mask narrowing (Top-p over exact block masses, GSRS reduced
search) against the CPU oracle.  Inputs are seeded; the masses given to the
GPU are the same float32 values the oracle reads, so the ranking is exact and
only the cumulative-share cut can move by float32 summation (the band)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import bsa_oracle as O
from workloads import get, make_inputs
from tests.gpu_helpers import default_scale, f32, messy_rows, to_device, to_host

pytestmark = pytest.mark.gpu

CUM_TOL = 1e-5       # cumulative-share band (float32 sums move C_r by ~1e-6)


@pytest.fixture(scope="module")
def bsa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_16_amd as m
    m.load()
    return m


def _random_csr(rng, R, nb, density, empty_frac=0.05):
    rows = []
    for _ in range(R):
        if rng.random() < empty_frac:
            rows.append(np.zeros(0, np.int64))
            continue
        k = int(min(nb, max(1, rng.binomial(nb, density))))
        rows.append(np.sort(rng.choice(nb, k, replace=False)))
    return O.rows_to_csr(rows)


def _random_masses(rng, rp, ci):
    """Per-row shares with exact ties, all-zero rows, negative and NaN entries."""
    m = np.zeros(ci.size, dtype=np.float32)
    for r in range(rp.size - 1):
        a, b = int(rp[r]), int(rp[r + 1])
        n = b - a
        if n == 0:
            continue
        u = rng.random()
        if u < 0.05:
            continue                                        # zero total
        w = rng.dirichlet(np.full(n, 0.6)) * rng.uniform(0.5, 1.5)
        if u < 0.25 and n >= 3:                             # exact ties
            t = rng.choice(n, size=min(n, 4), replace=False)
            w[t] = w[t[0]]
        if u > 0.95:
            w[rng.integers(n)] = -0.25
            w[rng.integers(n)] = np.nan
        m[a:b] = w.astype(np.float32)
    return m


def _narrow_gpu(bsa, rp, ci, mass, top_p, keep, B, H, N, bs):
    q = torch.empty((B, H, N, 64), dtype=torch.bfloat16, device="cuda")    # shape only
    mask = bsa.csr_from_host(rp.astype(np.int32), ci.astype(np.int32), "cuda")
    dm = torch.from_numpy(np.ascontiguousarray(mass, dtype=np.float32)).cuda()
    out = bsa.bsa_select_from_mass(q, mask, dm, top_p, bs, keep_prefix_tokens=keep)
    torch.cuda.synchronize()
    return out.to_host()


def _compare(grp, gci, rp, ci, sels, nb, top_p, value_tol=0.0):
    bad, band_total = [], 0
    for r, row in enumerate(sels):
        g = gci[grp[r]:grp[r + 1]]
        assert np.all(np.diff(g) > 0), f"row {r} not strictly ascending"
        allowed = set(ci[rp[r]:rp[r + 1]].tolist()) | set(row.forced.tolist())
        assert set(g.tolist()) <= allowed, f"row {r} keeps a block outside its row"
        band = O.mass_band(row, top_p, CUM_TOL)
        if value_tol > 0:
            band |= O.selection_band(row, top_p, tol=value_tol, mass_tol=CUM_TOL)
        band_total += len(band)
        if set(g.tolist()) - band != set(row.selected.tolist()) - band:
            bad.append(r)
    return bad, band_total


@pytest.mark.parametrize("nb", [16, 139, 500, 1500])
@pytest.mark.parametrize("top_p", [0.3, 0.9, 0.99, 1.0])
def test_narrowing_random_masks(bsa, nb, top_p):
    rng = np.random.default_rng(1000 + nb)
    bs, H = 64, 2
    N = nb * bs - 13                                       # ragged last block
    R = H * nb
    rp, ci = _random_csr(rng, R, nb, density=min(0.5, 60.0 / nb + 0.1))
    mass = _random_masses(rng, rp, ci)
    p = f32(top_p)
    keep = 0 if nb != 139 else 200                          # forced prefix blocks on one size
    grp, gci = _narrow_gpu(bsa, rp, ci, mass, p, keep, 1, H, N, bs)
    _, _, sels = O.narrow_by_mass(rp, ci, mass.astype(np.float64), p, keep, bs, nb)
    bad, band = _compare(grp, gci, rp, ci, sels, nb, p)
    assert not bad, f"{len(bad)} of {R} rows differ outside the band ({band} band blocks), first {bad[:5]}"
    if top_p == 1.0 and keep == 0:
        assert grp.tolist() == rp.tolist() and gci[:grp[-1]].tolist() == ci.tolist()


def test_narrowing_empty_and_tiny_rows(bsa):
    nb, bs, H = 8, 64, 1
    rows = [[], [3], [0, 7], [1, 2, 3, 4], [], [5], [0, 1, 2, 3, 4, 5, 6, 7], [6]]
    rp, ci = O.rows_to_csr([np.array(r, dtype=np.int64) for r in rows])
    mass = np.array([1.0, 0.2, 0.8, 0.25, 0.25, 0.25, 0.25, 0.0, 0.1, 0.2, 0.3, 0.4, 0.0, 0.0, 0.0, 0.0, 2.0],
                    dtype=np.float32)
    for p, keep in ((0.5, 0), (0.75, 0), (0.5, 64)):
        grp, gci = _narrow_gpu(bsa, rp, ci, mass, f32(p), keep, 1, H, nb * bs, bs)
        _, _, sels = O.narrow_by_mass(rp, ci, mass.astype(np.float64), f32(p), keep, bs, nb)
        got = [gci[grp[r]:grp[r + 1]].tolist() for r in range(nb)]
        assert got == [s.selected.tolist() for s in sels], (p, keep)


def test_narrowing_repeated_ids_and_long_rows(bsa):
    """Rows that repeat ids (the first listing's mass counts, also when both
    listings fall in one 64-entry chunk, and in shuffled rows) or list ids
    outside [0, nb) (ignored), including rows longer than the kernel's 256
    block slots."""
    nb, bs, H = 100, 64, 2
    rng = np.random.default_rng(43)
    rp, ci = O.rows_to_csr(messy_rows(rng, H * nb, nb))
    mass = rng.random(ci.size).astype(np.float32)
    for p in (0.5, 0.9):
        grp, gci = _narrow_gpu(bsa, rp, ci, mass, f32(p), 0, 1, H, nb * bs - 5, bs)
        _, _, sels = O.narrow_by_mass(rp, ci, mass.astype(np.float64), f32(p), 0, bs, nb)
        bad, band = _compare(grp, gci, rp, ci, sels, nb, f32(p))
        assert not bad, f"p={p}: {len(bad)} rows differ outside the band ({band} band blocks), first {bad[:5]}"


@pytest.mark.parametrize("wl", ["tiny", "small128"])
def test_reduced_search_loop_against_oracle_chain(bsa, wl):
    """Step 1 mask (oracle) -> forward with exact block mass -> narrowing, on the
    GPU and in the oracle; masses differ by float32 rounding, so blocks whose
    mass lies within 1e-5 of the cut are also in the band."""
    if wl == "tiny":
        w = get("tiny")
        x = make_inputs(w, dtype="bf16")
        B, H, N, D, bs = w.B, w.H, w.N, w.D, w.block
        p1 = f32(w.top_p[0])
    else:
        rng = np.random.default_rng(77)
        B, H, N, D, bs = 1, 2, 3000, 128, 128
        from workloads import round_to_bf16
        x = {n: round_to_bf16(rng.normal(size=(B, H, N, D)).astype(np.float32)) for n in "qkv"}
        x["q"] = round_to_bf16(x["q"] * 2.0)
        p1 = f32(0.95)
    scale = default_scale(D)
    nb = O.num_blocks(N, bs)
    rp, ci, _ = O.estimate_mask(x["q"], x["k"], bs, p1, scale)
    q, k, v = (to_device(x[n], "bf16") for n in "qkv")
    mask = bsa.csr_from_host(rp.astype(np.int32), ci.astype(np.int32), "cuda")
    _, _, gmass = bsa.bsa_forward(q, k, v, mask, bs)
    p2 = f32(0.8)
    out = bsa.bsa_select_from_mass(q, mask, gmass, p2, bs)
    torch.cuda.synchronize()
    grp, gci = out.to_host()
    _, _, omass = O.sparse_forward(x["q"], x["k"], x["v"], bs, rp, ci, scale)
    assert np.abs(to_host(gmass)[:ci.size] - omass).max() < 1e-4
    _, _, sels = O.narrow_by_mass(rp, ci, omass, p2, 0, bs, nb)
    bad, band = _compare(grp, gci, rp, ci, sels, nb, p2, value_tol=1e-5)
    assert not bad, f"{len(bad)} rows differ outside the band ({band} band blocks)"
    kept = grp[-1] / max(1, rp[-1])
    assert 0.0 < kept <= 1.0
