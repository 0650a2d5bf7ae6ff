"""Shared pieces of the GPU parity tests: moving seeded inputs to the device and
comparing the HIP path's outputs with the CPU oracle."""
from __future__ import annotations

import numpy as np
import torch

from oracle import bsa_oracle as O
from workloads import bf16_bits

# Tolerances.  bf16: 1e-2 on O (2e-2 on gradients) for the arithmetic, plus the
# rounding of the bf16 store itself (at most 2^-9 |x| with ties to even).
TOL = {
    "bf16": {"o": 1e-2, "grad": 2e-2, "lse": 1e-3, "mass": 1e-4, "store_rel": 2.0 ** -9},
    "fp32": {"o": 1e-5, "grad": 1e-5, "lse": 1e-5, "mass": 1e-5, "store_rel": 0.0},
}


def to_device(x: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(bf16_bits(x).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)


def to_host(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def f32(x: float) -> float:
    return float(np.float32(x))


def default_scale(D: int) -> float:
    return f32(1.0 / np.sqrt(D))


def compare_masks(rp_gpu, ci_gpu, sels: dict, H: int, nb: int, top_p: float, candidate_rows=None):
    """Checks every oracle row against the GPU CSR outside the selection band.

    Returns (rows, mismatched rows, band blocks).  Also checks that each GPU row
    is strictly ascending, in range and inside candidates + forced blocks.
    """
    bad, band_total, rows = [], 0, 0
    for (b, h), sel_rows in sels.items():
        for i, row in enumerate(sel_rows):
            r = (b * H + h) * nb + i
            g = ci_gpu[rp_gpu[r]:rp_gpu[r + 1]]
            assert np.all(np.diff(g) > 0), f"row {r} not strictly ascending"
            assert g.size == 0 or (g.min() >= 0 and g.max() < nb)
            allowed = set(row.candidates.tolist()) | set(row.forced.tolist())
            assert set(g.tolist()) <= allowed, f"row {r} selects outside candidates"
            band = O.selection_band(row, top_p)
            band_total += len(band)
            if set(g.tolist()) - band != set(row.selected.tolist()) - band:
                bad.append(r)
            rows += 1
    return rows, bad, band_total


def compare_forward(Qh, Kh, Vh, block, rp, ci, scale, rows, o_gpu, lse_gpu, mass_gpu, dtype: str, o32_gpu=None):
    """Oracle on the GPU's own mask for the listed rows; returns the max errors.
    ``o32_gpu``: the forward's fp32 O (before its rounding to bf16), compared
    with the oracle at the flat O tolerance, no store allowance ("o32")."""
    tol = TOL[dtype]
    Oo, Lo, Mo = O.sparse_forward(Qh, Kh, Vh, block, rp, ci, scale, rows=rows)
    B, H, N, D = Qh.shape
    nb = O.num_blocks(N, block)
    err = {"o": 0.0, "o_excess": 0.0, "lse": 0.0, "mass": 0.0}
    if o32_gpu is not None:
        err["o32"] = 0.0
    for r in rows:
        bh, i = divmod(r, nb)
        b, h = divmod(bh, H)
        lo, hi = i * block, min(i * block + block, N)
        og, oo = o_gpu[b, h, lo:hi], Oo[b, h, lo:hi]
        diff = np.abs(og - oo)
        err["o"] = max(err["o"], float(diff.max()))
        err["o_excess"] = max(err["o_excess"], float((diff - tol["o"] - tol["store_rel"] * np.abs(oo)).max()))
        if o32_gpu is not None:
            err["o32"] = max(err["o32"], float(np.abs(o32_gpu[b, h, lo:hi].astype(np.float64) - oo).max()))
        lg, lo_ = lse_gpu[b, h, lo:hi], Lo[b, h, lo:hi]
        fin = np.isfinite(lo_)
        assert np.array_equal(np.isfinite(lg), fin), f"row {r}: -inf pattern of LSE differs"
        if fin.any():
            err["lse"] = max(err["lse"], float(np.abs(lg[fin] - lo_[fin]).max()))
        a, z = rp[r], min(rp[r + 1], ci.size)
        if mass_gpu is not None and z > a:
            assert np.isfinite(mass_gpu[a:z]).all(), f"row {r}: non-finite block mass"
            err["mass"] = max(err["mass"], float(np.abs(mass_gpu[a:z] - Mo[a:z]).max()))
    return err


def assert_forward_within(err: dict, dtype: str, what: str = ""):
    tol = TOL[dtype]
    assert err["o_excess"] <= 0.0, f"{what} O error {err['o']:.3g} beyond {tol['o']} (+ bf16 store rounding)"
    if "o32" in err:
        assert err["o32"] <= tol["o"], f"{what} fp32 O error {err['o32']:.3g} > {tol['o']}"
    assert err["lse"] <= tol["lse"], f"{what} LSE error {err['lse']:.3g} > {tol['lse']}"
    assert err["mass"] <= tol["mass"], f"{what} mass error {err['mass']:.3g} > {tol['mass']}"


def sample_rows(R: int, nb: int, count: int, seed: int = 0, row_ptr=None) -> list[int]:
    """Rows to check against the oracle: the first and last block of the first
    and last head (ragged tail), plus a seeded random sample.  With the CSR's
    ``row_ptr``, also every head's longest row, its shortest non-empty row and
    one seeded random row of it."""
    rng = np.random.default_rng(seed)
    fixed = {0, nb - 1, R - nb, R - 1}
    extra = rng.choice(R, size=min(count, R), replace=False).tolist()
    if row_ptr is not None:
        lens = np.diff(np.asarray(row_ptr, dtype=np.int64)[:R + 1])
        for r0 in range(0, R, nb):
            ln = lens[r0:r0 + nb]
            fixed.add(r0 + int(np.argmax(ln)))
            nz = np.nonzero(ln > 0)[0]
            if nz.size:
                fixed.add(r0 + int(nz[np.argmin(ln[nz])]))
            fixed.add(r0 + int(rng.integers(nb)))
    return sorted(fixed | set(extra))


def head_csr(rp, ci, H: int, nb: int, b: int, h: int):
    """CSR rows of one head, rebased to start at 0."""
    r0 = (b * H + h) * nb
    sub_rp = rp[r0:r0 + nb + 1] - rp[r0]
    sub_ci = ci[rp[r0]:rp[r0 + nb]]
    return sub_rp, sub_ci


def compare_backward(x, block, rp, ci, scale, heads, grads_gpu, dtype: str):
    """Oracle gradients of sum(O * G) for the listed heads vs the GPU's; max errors."""
    tol = TOL[dtype]
    B, H, N, D = x["q"].shape
    nb = O.num_blocks(N, block)
    err = {"dq": 0.0, "dk": 0.0, "dv": 0.0, "excess": -1.0}
    for b, h in heads:
        srp, sci = head_csr(rp, ci, H, nb, b, h)
        sl = (slice(b, b + 1), slice(h, h + 1))
        dQ, dK, dV = O.sparse_backward(x["q"][sl], x["k"][sl], x["v"][sl], x["g"][sl], block, srp, sci, scale)
        for name, want in (("dq", dQ), ("dk", dK), ("dv", dV)):
            got = grads_gpu[name][b, h]
            diff = np.abs(got - want[0, 0])
            err[name] = max(err[name], float(diff.max()))
            err["excess"] = max(err["excess"],
                                float((diff - tol["grad"] - tol["store_rel"] * np.abs(want[0, 0])).max()))
    return err


def messy_rows(rng, R: int, nb: int) -> list:
    """Candidate / mask rows outside the strictly ascending form, for a grid of
    65 <= nb <= 200 blocks (the selection kernels then hold 256 block slots):
      r % 6 == 0  repeats inside one 64-entry chunk (the first 10 ids twice);
      r % 6 == 1  repeats across chunks, negative ids between the listings;
      r % 6 == 2  ascending, 300 leading negative ids and 3 ids >= nb, so the
                  row is longer than 256 entries;
      r % 6 == 3  strictly ascending;
      r % 6 == 4  non-decreasing, every id listed 3 times (86 or more ids, so
                  the row is longer than 256 entries);
      r % 6 == 5  unordered: a shuffled row with repeats and bad ids mixed in."""
    assert 65 <= nb <= 200
    rows = []
    for r in range(R):
        kind = r % 6
        lo, hi = (86, nb) if kind == 4 else (1, 60 if kind < 2 else nb)
        c = np.sort(rng.choice(nb, size=int(rng.integers(lo, hi + 1)), replace=False))
        if kind == 0:
            rows.append(np.concatenate([c[:10], c[:10], c[10:]]))
        elif kind == 1:
            rows.append(np.concatenate([c, np.full(64 - c.size, -1), c]))
        elif kind == 2:
            rows.append(np.concatenate([np.arange(-300, 0), c, np.arange(nb, nb + 3)]))
        elif kind == 4:
            rows.append(np.repeat(c, 3))
        elif kind == 5:
            x = np.concatenate([c, c[: c.size // 2], [-1, nb, -7]])
            rows.append(x[rng.permutation(x.size)])
        else:
            rows.append(c)
    return rows
