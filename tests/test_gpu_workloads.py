"""GPU parity at the full workload sizes, in the launch configuration the benchmark times.

Masks: every row against the oracle (outside the selection band).  Forward:
a seeded sample of rows, the first/last block of the first/last head and, in
every head, its longest row, its shortest non-empty row and one random row,
each recomputed by the oracle on the GPU's own mask.  The bf16 O is held to
1e-2 plus the rounding of its bf16 store; the fp32 O of the same forward
(before that rounding) to a flat 1e-2.
"""
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import bsa_oracle as O
from workloads import get, make_inputs
from tests.gpu_helpers import (assert_forward_within, compare_forward, compare_masks, default_scale, f32,
                               sample_rows, to_device, to_host)

pytestmark = pytest.mark.gpu

SAMPLE = int(os.environ.get("BSA_PARITY_SAMPLE_ROWS", "24"))


@pytest.fixture(scope="module")
def bsa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_16_amd as m
    m.load()
    return m


def _run_step(bsa, w, x, top_p, candidate=None, cand_host=None):
    q, k, v = (to_device(x[n], "bf16") for n in "qkv")
    mask = bsa.bsa_estimate_mask(q, k, top_p, w.block, candidate=candidate,
                                 keep_prefix_tokens=w.keep_prefix_tokens)
    o, lse, mass = bsa.bsa_forward(q, k, v, mask, w.block)
    # the same forward with the fp32 O kept: the arithmetic alone, before the
    # bf16 store, is held to the flat O tolerance
    o32 = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    o_b, lse_b, _ = bsa.bsa_forward(q, k, v, mask, w.block, want_mass=False, o32=o32)
    torch.cuda.synchronize()
    assert torch.equal(o, o_b) and torch.equal(lse, lse_b), "the fp32-O instantiation changed O or LSE"
    del o_b, lse_b
    rp, ci = mask.to_host()
    _, _, sels = O.estimate_mask(x["q"], x["k"], w.block, top_p, default_scale(w.D), candidate=cand_host,
                                 keep_prefix_tokens=w.keep_prefix_tokens)
    rows, bad, band = compare_masks(rp, ci, sels, w.H, w.nb, top_p)
    print(f"[{w.name}] p={top_p:.4f} rows={rows} nnz={ci.size} density={ci.size / rows / w.nb:.3f} "
          f"band={band} mismatched={len(bad)}", flush=True)
    assert not bad, f"{len(bad)} of {rows} rows differ outside the band: {bad[:10]}"
    R = w.B * w.H * w.nb
    sel_rows = sample_rows(R, w.nb, SAMPLE, seed=w.cfg_id, row_ptr=rp)
    err = compare_forward(x["q"], x["k"], x["v"], w.block, rp, ci, default_scale(w.D), sel_rows,
                          to_host(o), to_host(lse), to_host(mass[:ci.size]), "bf16", o32_gpu=o32.cpu().numpy())
    lens = np.diff(rp)
    print(f"[{w.name}] forward errors on {len(sel_rows)} rows (longest row {int(lens.max())} entries, "
          f"sampled max {int(max(lens[r] for r in sel_rows))}): {err}", flush=True)
    assert_forward_within(err, "bf16", w.name)
    del o32
    return mask, (rp, ci)


@pytest.mark.parametrize("name", ["cogvideox", "hunyuan"])
def test_single_step_workload(bsa, name):
    w = get(name)
    x = make_inputs(w, dtype="bf16")
    _run_step(bsa, w, x, f32(w.top_p[0]))


def test_wan_reduced_search_steps(bsa):
    w = get("wan")
    first, first_host = None, None
    for s, p in enumerate(w.top_p, start=1):
        x = make_inputs(w, step=s, dtype="bf16")
        mask, host = _run_step(bsa, w, x, f32(p), candidate=first, cand_host=first_host)
        if s == 1:
            first, first_host = mask, host
        else:
            # every later mask lies inside step 1's blocks
            rp, ci = host
            frp, fci = first_host
            for r in range(0, w.B * w.H * w.nb, 97):
                assert set(ci[rp[r]:rp[r + 1]].tolist()) <= set(fci[frp[r]:frp[r + 1]].tolist())


@pytest.mark.parametrize("delta", ["exact", "o32"])
def test_dsv_training_forward_and_backward(bsa, delta):
    from tests.gpu_helpers import compare_backward
    w = get("dsv_train")
    x = make_inputs(w, dtype="bf16", want_grad=True)
    mask, (rp, ci) = _run_step(bsa, w, x, f32(w.top_p[0]))
    q, k, v, g = (to_device(x[n], "bf16") for n in "qkvg")
    o32 = torch.empty(q.shape, dtype=torch.float32, device="cuda") if delta == "o32" else None
    o, lse, _ = bsa.bsa_forward(q, k, v, mask, w.block, want_mass=False, o32=o32)
    dq, dk, dv = bsa.bsa_backward(q, k, v, o, g, lse, mask, w.block, o32=o32)
    torch.cuda.synchronize()
    heads = [(0, 0), (1, w.H - 1)]
    grads = {"dq": to_host(dq), "dk": to_host(dk), "dv": to_host(dv)}
    err = compare_backward(x, w.block, rp, ci, default_scale(w.D), heads, grads, "bf16")
    print(f"[{w.name} delta={delta}] gradient errors on heads {heads}: {err}", flush=True)
    assert err["excess"] <= 0.0, f"gradient errors {err}"
