"""GPU parity of the structured head masks (SVG spatial/temporal heads,
Sparse-vDiT diagonal / multi-diagonal / vertical-stripe) against the oracle.
Integer work: the CSR must match exactly."""
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


def _gpu_mask(bsa, B, H, N, bs, kinds, prefix, F, band, period, stripes):
    q = torch.empty((B, H, N, 64), dtype=torch.bfloat16, device="cuda")   # shape only
    hk = torch.tensor(kinds, dtype=torch.int32, device="cuda")
    st = torch.tensor(list(stripes), dtype=torch.int32, device="cuda") if len(stripes) else None
    out = bsa.bsa_structured_mask(q, hk, bs, prefix_tokens=prefix, frame_tokens=F, band=band, period=period,
                                  stripes=st)
    torch.cuda.synchronize()
    return out.to_host()


GEOMS = [  # N, bs, prefix, frame tokens, band, period
    (1000, 64, 0, 96, 1, 3),
    (1000, 64, 40, 96, 0, 4),
    (2077, 128, 226, 150, 2, 5),
    (513, 64, 200, 31, 1, 2),
    (4000, 128, 0, 4000, 0, 1),
]


@pytest.mark.parametrize("geom", GEOMS)
@pytest.mark.parametrize("kind", range(6))
def test_structured_mask_matches_oracle(bsa, kind, geom):
    N, bs, prefix, F, band, period = geom
    nb = O.num_blocks(N, bs)
    stripes = [0, 3, nb - 1, nb + 5, -2]                    # out-of-range ids are ignored
    grp, gci = _gpu_mask(bsa, 1, 1, N, bs, [kind], prefix, F, band, period, stripes)
    orp, oci = O.structured_mask(1, 1, N, bs, [kind], prefix, F, band, period, stripes)
    assert grp.tolist() == orp.tolist()
    assert gci[:grp[-1]].tolist() == oci.tolist()


def test_mixed_heads_and_unknown_kind(bsa):
    N, bs, prefix, F = 1500, 64, 100, 130
    kinds = [1, 2, 3, 4, 5, 0, 9, 1]                         # 9: unknown -> dense rows
    B, H = 2, 4
    grp, gci = _gpu_mask(bsa, B, H, N, bs, kinds, prefix, F, 1, 4, [2, 7])
    orp, oci = O.structured_mask(B, H, N, bs, [k if k <= 5 else 0 for k in kinds], prefix, F, 1, 4, [2, 7])
    assert grp.tolist() == orp.tolist()
    assert gci[:grp[-1]].tolist() == oci.tolist()


@pytest.mark.parametrize("wl", ["cogvideox", "hunyuan"])
@pytest.mark.parametrize("kind", [O.PATTERN_SPATIAL, O.PATTERN_TEMPORAL, O.PATTERN_MULTI_DIAGONAL])
def test_structured_mask_at_workload_geometry_sampled_rows(bsa, wl, kind):
    from workloads import get
    w = get(wl)
    T, Hg, Wg = w.grid
    F = Hg * Wg
    N, bs, prefix = w.N, w.block, w.text_prefix
    nb = w.nb
    period = max(1, F // bs)
    grp, gci = _gpu_mask(bsa, 1, 1, N, bs, [kind], prefix, F, 1, period, [])
    rows = sorted(set(np.linspace(0, nb - 1, 24).astype(int).tolist()))
    ref = O.structured_block_mask(kind, N, bs, prefix, F, 1, period, (), rows=rows)
    for ri, i in enumerate(rows):
        assert gci[grp[i]:grp[i + 1]].tolist() == np.nonzero(ref[ri])[0].tolist(), (wl, kind, i)
