"""GPU parity at B > 1 (B = 2, H = 3): the row order r = (b*H + h)*nb + i of
every mask, candidate rows read from their own head, and the forward, the
narrowing and hierarchical scoring over batched tensors, against the oracle.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import bsa_oracle as O
from workloads import round_to_bf16
from tests.gpu_helpers import (assert_forward_within, compare_forward, compare_masks, default_scale, f32,
                               to_device, to_host)

pytestmark = pytest.mark.gpu

B, H = 2, 3


@pytest.fixture(scope="module")
def bsa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_16_amd as m
    m.load()
    return m


def _qkv(rng, N, D, dtype):
    q = rng.normal(size=(B, H, N, D)).astype(np.float32) * 0.4
    k = rng.normal(size=(B, H, N, D)).astype(np.float32) + q
    v = rng.normal(size=(B, H, N, D)).astype(np.float32)
    if dtype == "bf16":
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    return q, k, v


def _random_rows(rng, R, nb, empty_every=7):
    rows = []
    for r in range(R):
        if r % empty_every == 5:
            rows.append(np.zeros(0, np.int64))
        else:
            rows.append(np.sort(rng.choice(nb, size=int(rng.integers(1, nb + 1)), replace=False)))
    return rows


def test_dominant_block_per_head(bsa):
    """Closed form: every query is e_0, and head (b, h) has keys 40 e_0 only in
    block j*(b, h) = (3b + h) mod nb, so every row of that head selects exactly
    j*(b, h).  With single-block candidate rows c(b, h, i) every row keeps
    exactly its own candidate."""
    nb, bs, D = 5, 64, 64
    N = nb * bs
    q = np.zeros((B, H, N, D), np.float32)
    q[..., 0] = 1.0
    k = np.zeros((B, H, N, D), np.float32)
    j_star = lambda b, h: (3 * b + h) % nb
    for b in range(B):
        for h in range(H):
            k[b, h, j_star(b, h) * bs:(j_star(b, h) + 1) * bs, 0] = 40.0
    qd, kd = to_device(q, "bf16"), to_device(k, "bf16")
    m = bsa.bsa_estimate_mask(qd, kd, 0.5, bs)
    rp, ci = m.to_host()
    assert rp.tolist() == list(range(B * H * nb + 1))
    assert ci.tolist() == [j_star(b, h) for b in range(B) for h in range(H) for _ in range(nb)]
    c = lambda b, h, i: (7 * (b * H + h) + 2 * i) % nb
    want = [c(b, h, i) for b in range(B) for h in range(H) for i in range(nb)]
    cand = bsa.csr_from_host(np.arange(B * H * nb + 1), np.array(want), "cuda")
    rng = np.random.default_rng(3)
    qr = to_device(round_to_bf16(rng.normal(size=(B, H, N, D)).astype(np.float32)), "bf16")
    kr = to_device(round_to_bf16(rng.normal(size=(B, H, N, D)).astype(np.float32)), "bf16")
    m2 = bsa.bsa_estimate_mask(qr, kr, 0.9, bs, candidate=cand)
    rp2, ci2 = m2.to_host()
    assert rp2.tolist() == list(range(B * H * nb + 1))
    assert ci2.tolist() == want


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("D,bs", [(64, 128), (128, 64), (128, 128)])
def test_candidate_path_batched(bsa, dtype, D, bs):
    rng = np.random.default_rng(700 + D + bs)
    N = 9 * bs - 21                                          # ragged last block
    q, k, _ = _qkv(rng, N, D, dtype)
    nb = O.num_blocks(N, bs)
    rows = _random_rows(rng, B * H * nb, nb)
    crp, cci = O.rows_to_csr(rows)
    cand = bsa.csr_from_host(crp, cci, "cuda")
    p = f32(0.8)
    m = bsa.bsa_estimate_mask(to_device(q, dtype), to_device(k, dtype), p, bs, candidate=cand,
                              keep_prefix_tokens=bs + 3)
    rp, ci = m.to_host()
    _, _, sels = O.estimate_mask(q, k, bs, p, default_scale(D), candidate=(crp, cci), keep_prefix_tokens=bs + 3)
    nrows, bad, band = compare_masks(rp, ci, sels, H, nb, p)
    assert nrows == B * H * nb
    assert not bad, f"{len(bad)} of {nrows} rows differ outside the band ({band} band blocks): {bad[:8]}"


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("g", [2, 4])
def test_hierarchical_batched_with_candidates(bsa, dtype, g):
    rng = np.random.default_rng(800 + g)
    D, bs = 128, 128
    N = 11 * bs - 40
    q, k, _ = _qkv(rng, N, D, dtype)
    nb = O.num_blocks(N, bs)
    p = f32(0.85)
    qd, kd = to_device(q, dtype), to_device(k, dtype)
    m = bsa.bsa_estimate_mask(qd, kd, p, bs, sub_blocks=g)
    rp, ci = m.to_host()
    _, _, sels = O.estimate_mask(q, k, bs, p, default_scale(D), sub_blocks=g)
    nrows, bad, band = compare_masks(rp, ci, sels, H, nb, p)
    assert not bad, f"no candidates: {len(bad)} of {nrows} rows differ outside the band"
    rows = _random_rows(rng, B * H * nb, nb)
    crp, cci = O.rows_to_csr(rows)
    m2 = bsa.bsa_estimate_mask(qd, kd, p, bs, sub_blocks=g, candidate=bsa.csr_from_host(crp, cci, "cuda"))
    rp2, ci2 = m2.to_host()
    _, _, sels2 = O.estimate_mask(q, k, bs, p, default_scale(D), candidate=(crp, cci), sub_blocks=g)
    nrows, bad, band = compare_masks(rp2, ci2, sels2, H, nb, p)
    assert not bad, f"candidates: {len(bad)} of {nrows} rows differ outside the band"


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("D,bs", [(64, 64), (128, 128)])
def test_forward_and_narrowing_batched(bsa, dtype, D, bs):
    """Random block mask over B = 2, H = 3: every row of O, LSE and block mass
    against the oracle; then narrowing of that mask by the GPU's own masses
    against the oracle's narrowing of the same float32 masses."""
    rng = np.random.default_rng(900 + D + bs)
    N = 6 * bs - 9
    q, k, v = _qkv(rng, N, D, dtype)
    nb = O.num_blocks(N, bs)
    R = B * H * nb
    rp, ci = O.rows_to_csr(_random_rows(rng, R, nb))
    mask = bsa.csr_from_host(rp, ci, "cuda")
    qd, kd, vd = (to_device(t, dtype) for t in (q, k, v))
    o, lse, mass = bsa.bsa_forward(qd, kd, vd, mask, bs)
    torch.cuda.synchronize()
    scale = default_scale(D)
    gm = mass[:ci.size].cpu().numpy()
    err = compare_forward(q, k, v, bs, rp, ci, scale, list(range(R)), to_host(o), to_host(lse),
                          gm.astype(np.float64), dtype)
    assert_forward_within(err, dtype, f"B=2 D={D} bs={bs}")
    p = f32(0.7)
    out = bsa.bsa_select_from_mass(qd, mask, mass, p, bs, keep_prefix_tokens=1)
    grp, gci = out.to_host()
    _, _, sels = O.narrow_by_mass(rp, ci, gm.astype(np.float64), p, 1, bs, nb)
    bad = []
    for r, row in enumerate(sels):
        g = set(gci[grp[r]:grp[r + 1]].tolist())
        band = O.mass_band(row, p, 1e-5)
        if g - band != set(row.selected.tolist()) - band:
            bad.append(r)
    assert not bad, f"narrowing: {len(bad)} of {R} rows differ outside the band: {bad[:8]}"
