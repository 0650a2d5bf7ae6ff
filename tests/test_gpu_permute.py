"""GPU parity of the token permutation (gather into a new token order, scatter
back) against the oracle.  Pure data movement: results must match bit for bit."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import bsa_oracle as O

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bsa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_16_amd as m
    m.load()
    return m


def _bits(t: torch.Tensor) -> np.ndarray:
    """Raw element bits on the host (exact comparison of any dtype)."""
    view = {2: torch.int16, 4: torch.int32}[t.element_size()]
    return t.contiguous().view(view).cpu().numpy()


@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 64), (torch.bfloat16, 128), (torch.float32, 128),
                                     (torch.float32, None), (torch.bfloat16, 6)])
@pytest.mark.parametrize("N", [1, 7, 1000])
def test_gather_scatter_round_trip(bsa, dtype, D, N):
    rng = np.random.default_rng(N + (D or 1))
    B, H = 2, 3
    shape = (B, H, N) if D is None else (B, H, N, D)
    x = torch.from_numpy(rng.normal(size=shape).astype(np.float32)).to(dtype).cuda()
    perm = rng.permutation(N).astype(np.int32)
    p = torch.from_numpy(perm).cuda()
    y = bsa.bsa_permute_tokens(x, p)
    z = bsa.bsa_permute_tokens(y, p, inverse=True)
    torch.cuda.synchronize()
    xb = _bits(x).reshape(B * H, N, -1)
    assert (_bits(y).reshape(B * H, N, -1) == O.permute_rows(xb, perm)).all()
    assert (_bits(z) == _bits(x)).all()


def test_out_of_range_entries(bsa):
    rng = np.random.default_rng(5)
    B, H, N, D = 1, 2, 50, 64
    x = torch.from_numpy(rng.normal(size=(B, H, N, D)).astype(np.float32)).to(torch.bfloat16).cuda()
    perm = rng.permutation(N).astype(np.int32)
    perm[[3, 17]] = [-1, N + 4]
    p = torch.from_numpy(perm).cuda()
    xb = _bits(x).reshape(B * H, N, D)
    y = bsa.bsa_permute_tokens(x, p)
    dst = torch.full_like(x, 7.0)
    z = bsa.bsa_permute_tokens(x, p, inverse=True, out=dst)
    torch.cuda.synchronize()
    assert (_bits(y).reshape(B * H, N, D) == O.permute_rows(xb, perm)).all()
    zb = _bits(z).reshape(B * H, N, D)
    ref = O.permute_rows(xb, perm, inverse=True)
    written = np.zeros(N, dtype=bool)
    written[perm[(perm >= 0) & (perm < N)]] = True
    assert (zb[:, written] == ref[:, written]).all()
    assert (zb[:, ~written] == _bits(torch.full_like(x, 7.0)).reshape(B * H, N, D)[:, ~written]).all()


def test_hilbert_order_at_video_geometry(bsa):
    from workloads import get
    from workloads.hilbert import hilbert_order
    w = get("cogvideox")
    T, Hg, Wg = w.grid
    order = hilbert_order((T, Hg, Wg))                        # video tokens in curve order
    perm = np.concatenate([np.arange(w.text_prefix), w.text_prefix + np.asarray(order)]).astype(np.int32)
    assert np.array_equal(np.sort(perm), np.arange(w.N))
    rng = np.random.default_rng(8)
    x = torch.from_numpy(rng.normal(size=(1, 4, w.N, w.D)).astype(np.float32)).to(torch.bfloat16).cuda()
    p = torch.from_numpy(perm).cuda()
    y = bsa.bsa_permute_tokens(x, p)
    torch.cuda.synchronize()
    assert (_bits(y).reshape(4, w.N, w.D) == O.permute_rows(_bits(x).reshape(4, w.N, w.D), perm)).all()
