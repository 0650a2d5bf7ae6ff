"""GPU parity of hierarchical block scoring (bsa_estimate_mask_hierarchical).

Reading of the DFSAttn page's hierarchical block scoring (Abstract): block
logits are the log-sum-exp of the query block mean against the key block's
sub-block means.  Masks are compared with the oracle row by row outside the
selection band; a stripe case checks the selections a hand calculation fixes.
"""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import bsa_oracle as O
from workloads import get, make_inputs, round_to_bf16
from tests.gpu_helpers import compare_masks, default_scale, f32, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bsa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_16_amd as m
    m.load()
    return m


def _qk(rng, B, H, N, D, dtype):
    q = rng.normal(size=(B, H, N, D)).astype(np.float32) * 0.3
    k = rng.normal(size=(B, H, N, D)).astype(np.float32) + q
    if dtype == "bf16":
        q, k = round_to_bf16(q), round_to_bf16(k)
    return q, k


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("D,bs", [(64, 64), (64, 128), (128, 64), (128, 128)])
@pytest.mark.parametrize("N", [37, 1000])
@pytest.mark.parametrize("g", [2, 4, 8])
def test_hierarchical_masks_ragged(bsa, dtype, D, bs, N, g):
    rng = np.random.default_rng(N + 10 * D + bs + 1000 * g)
    B, H = 1, 2
    q, k = _qk(rng, B, H, N, D, dtype)
    p = f32(0.8)
    m = bsa.bsa_estimate_mask(to_device(q, dtype), to_device(k, dtype), p, bs, sub_blocks=g)
    rp, ci = m.to_host()
    _, _, sels = O.estimate_mask(q, k, bs, p, default_scale(D), sub_blocks=g)
    rows, bad, band = compare_masks(rp, ci, sels, H, O.num_blocks(N, bs), p)
    assert not bad, f"{len(bad)} of {rows} rows differ outside the band"


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_hierarchical_candidates_and_forced_prefix(bsa, dtype):
    rng = np.random.default_rng(5)
    B, H, N, D, bs, g = 1, 2, 2000, 128, 128, 4
    q, k = _qk(rng, B, H, N, D, dtype)
    nb = O.num_blocks(N, bs)
    cand_rows = [np.zeros(0, np.int64) if r % 7 == 2 else
                 np.sort(rng.choice(nb, size=int(rng.integers(1, nb + 1)), replace=False))
                 for r in range(B * H * nb)]
    crp, cci = O.rows_to_csr(cand_rows)
    cand = bsa.csr_from_host(crp, cci, "cuda")
    p = f32(0.85)
    m = bsa.bsa_estimate_mask(to_device(q, dtype), to_device(k, dtype), p, bs, candidate=cand,
                              keep_prefix_tokens=130, sub_blocks=g)
    rp, ci = m.to_host()
    _, _, sels = O.estimate_mask(q, k, bs, p, default_scale(D), candidate=(crp, cci), keep_prefix_tokens=130,
                                 sub_blocks=g)
    rows, bad, band = compare_masks(rp, ci, sels, H, nb, p)
    assert not bad, f"{len(bad)} of {rows} rows differ"
    assert ci[rp[2]:rp[3]].tolist() == [0, 1]      # empty candidate row: the forced blocks only


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_hierarchical_stripe_block(bsa, dtype):
    # the hand-worked stripe case, at D = 64, block 64 (scale 1/8): query
    # tokens e0; key block 0 = 0, block 1 = +80 e0 then -80 e0 (half each),
    # block 2 = 8 e0.  Mean-pool logits 0, 0, 1; sub-block logits of block 1
    # are +-10, so hierarchical scoring ranks block 1 first.
    D, bs, N = 64, 64, 192
    u = np.zeros(D, np.float32)
    u[0] = 1.0
    q = np.tile(u, (N, 1))[None, None]
    k = np.concatenate([np.zeros((bs, D), np.float32), np.tile(80 * u, (32, 1)), np.tile(-80 * u, (32, 1)),
                        np.tile(8 * u, (bs, 1))])[None, None]
    qd, kd = to_device(q, dtype), to_device(k, dtype)
    cases = [(1, 0.5, [2]), (1, 0.7, [0, 2]), (1, 0.8, [0, 1, 2]),
             (2, 0.5, [1]), (2, 0.9998, [1, 2]), (4, 0.5, [1]), (4, 0.9998, [1, 2]), (8, 0.9998, [1, 2])]
    for g, p, want in cases:
        m = bsa.bsa_estimate_mask(qd, kd, f32(p), bs, sub_blocks=g)
        rp, ci = m.to_host()
        for r in range(3):
            assert ci[rp[r]:rp[r + 1]].tolist() == want, (g, p, r)


def test_hierarchical_one_sub_block_is_the_plain_estimator(bsa):
    w = get("tiny")
    x = make_inputs(w, dtype="bf16")
    q, k = to_device(x["q"], "bf16"), to_device(x["k"], "bf16")
    plain = bsa.bsa_estimate_mask(q, k, 0.9, w.block)
    L = bsa.load()
    shape = bsa.make_shape(w.B, w.H, w.N, w.D, w.block, 0)
    ws = torch.empty(bsa.bsa_workspace_size(shape, 5, 0), dtype=torch.uint8, device="cuda")
    out = bsa.Csr(torch.empty_like(plain.row_ptr), torch.empty_like(plain.col_idx))
    oc = out.c()
    st = L.bsa_estimate_mask_hierarchical(ctypes.byref(shape), q.data_ptr(), k.data_ptr(), 0.9, 0.0, None, 0, 1,
                                          ctypes.byref(oc), ws.data_ptr(), ws.numel(),
                                          torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    a, b = plain.to_host(), out.to_host()
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("g", [4])
def test_hierarchical_cogvideox_workload(bsa, g):
    w = get("cogvideox")
    x = make_inputs(w, dtype="bf16")
    p = f32(w.top_p[0])
    m = bsa.bsa_estimate_mask(to_device(x["q"], "bf16"), to_device(x["k"], "bf16"), p, w.block,
                              keep_prefix_tokens=w.keep_prefix_tokens, sub_blocks=g)
    rp, ci = m.to_host()
    _, _, sels = O.estimate_mask(x["q"], x["k"], w.block, p, default_scale(w.D),
                                 keep_prefix_tokens=w.keep_prefix_tokens, sub_blocks=g)
    rows, bad, band = compare_masks(rp, ci, sels, w.H, w.nb, p)
    plain = ci.size
    print(f"[cogvideox hierarchical g={g}] rows={rows} nnz={plain} band={band} mismatched={len(bad)}", flush=True)
    assert not bad, f"{len(bad)} of {rows} rows differ outside the band: {bad[:10]}"
