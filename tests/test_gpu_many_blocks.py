"""GPU parity with more than 1024 key blocks per row (up to the 4096 limit):
the widest instantiation of the selection kernels (64 blocks per lane) on the
full search, candidate rows and hierarchical scoring, and the forward on a
sample of rows of the estimated mask."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import bsa_oracle as O
from workloads import round_to_bf16
from tests.gpu_helpers import (assert_forward_within, compare_forward, compare_masks, default_scale, f32,
                               sample_rows, to_device, to_host)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bsa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_16_amd as m
    m.load()
    return m


def _qkv(seed, N, D=64):
    rng = np.random.default_rng(seed)
    q = round_to_bf16(rng.normal(size=(1, 1, N, D)).astype(np.float32) * 0.3)
    k = round_to_bf16(rng.normal(size=(1, 1, N, D)).astype(np.float32) + q)
    v = round_to_bf16(rng.normal(size=(1, 1, N, D)).astype(np.float32))
    return q, k, v


@pytest.mark.parametrize("N", [1100 * 64 - 23, 4096 * 64])
def test_full_search_and_forward_many_blocks(bsa, N):
    bs, D, p = 64, 64, f32(0.9)
    q, k, v = _qkv(N, N, D)
    qd, kd, vd = (to_device(t, "bf16") for t in (q, k, v))
    mask = bsa.bsa_estimate_mask(qd, kd, p, bs, keep_prefix_tokens=100)
    o, lse, mass = bsa.bsa_forward(qd, kd, vd, mask, bs)
    torch.cuda.synchronize()
    rp, ci = mask.to_host()
    nb = O.num_blocks(N, bs)
    _, _, sels = O.estimate_mask(q, k, bs, p, default_scale(D), keep_prefix_tokens=100)
    rows, bad, band = compare_masks(rp, ci, sels, 1, nb, p)
    assert not bad, f"{len(bad)} of {rows} rows differ outside the band"
    sel = sample_rows(nb, nb, 12, seed=N)
    err = compare_forward(q, k, v, bs, rp, ci, default_scale(D), sel, to_host(o), to_host(lse),
                          to_host(mass[:ci.size]), "bf16")
    assert_forward_within(err, "bf16", f"nb={nb}")


def test_candidate_rows_many_blocks(bsa):
    bs, D, N, p = 64, 64, 1100 * 64 - 23, f32(0.8)
    q, k, _ = _qkv(7, N, D)
    nb = O.num_blocks(N, bs)
    rng = np.random.default_rng(8)
    cand_rows = [np.sort(rng.choice(nb, size=int(rng.integers(1, nb + 1)), replace=False)) for _ in range(nb)]
    crp, cci = O.rows_to_csr(cand_rows)
    cand = bsa.csr_from_host(crp, cci, "cuda")
    m = bsa.bsa_estimate_mask(to_device(q, "bf16"), to_device(k, "bf16"), p, bs, candidate=cand)
    rp, ci = m.to_host()
    _, _, sels = O.estimate_mask(q, k, bs, p, default_scale(D), candidate=(crp, cci))
    rows, bad, band = compare_masks(rp, ci, sels, 1, nb, p)
    assert not bad, f"{len(bad)} of {rows} rows differ outside the band"


def test_hierarchical_many_blocks(bsa):
    bs, D, N, p, g = 64, 64, 1100 * 64 - 23, f32(0.85), 2
    q, k, _ = _qkv(9, N, D)
    m = bsa.bsa_estimate_mask(to_device(q, "bf16"), to_device(k, "bf16"), p, bs, sub_blocks=g)
    rp, ci = m.to_host()
    _, _, sels = O.estimate_mask(q, k, bs, p, default_scale(D), sub_blocks=g)
    rows, bad, band = compare_masks(rp, ci, sels, 1, O.num_blocks(N, bs), p)
    assert not bad, f"{len(bad)} of {rows} rows differ outside the band"


@pytest.mark.parametrize("delta", ["exact", "o32"])
def test_backward_many_blocks(bsa, delta):
    # 1100 key blocks per head: the CSC transpose and the dK/dV grid's
    # longest-first tail at a wide mask; a sparse random mask keeps the
    # oracle's gradients quick
    from tests.gpu_helpers import compare_backward
    bs, D, N = 64, 64, 1100 * 64 - 23
    nb = O.num_blocks(N, bs)
    q, k, v = _qkv(11, N, D)
    rng = np.random.default_rng(12)
    g = round_to_bf16(rng.normal(size=q.shape).astype(np.float32))
    rows = [np.zeros(0, np.int64) if r % 9 == 4 else
            np.sort(rng.choice(nb, size=int(rng.integers(1, 40)), replace=False)) for r in range(nb)]
    rows[nb - 1] = np.arange(nb - 30, nb)                  # the ragged last block in its own row
    rp, ci = O.rows_to_csr(rows)
    mask = bsa.csr_from_host(rp, ci, "cuda")
    qd, kd, vd, gd = (to_device(t, "bf16") for t in (q, k, v, g))
    o32 = torch.empty(qd.shape, dtype=torch.float32, device="cuda") if delta == "o32" else None
    o, lse, _ = bsa.bsa_forward(qd, kd, vd, mask, bs, want_mass=False, o32=o32)
    dq, dk, dv = bsa.bsa_backward(qd, kd, vd, o, gd, lse, mask, bs, o32=o32)
    torch.cuda.synchronize()
    err = compare_backward({"q": q, "k": k, "v": v, "g": g}, bs, rp, ci, default_scale(D), [(0, 0)],
                           {"dq": to_host(dq), "dk": to_host(dk), "dv": to_host(dv)}, "bf16")
    assert err["excess"] <= 0.0, f"gradient errors {err}"
