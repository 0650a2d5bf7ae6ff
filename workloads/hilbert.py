"""3-D Hilbert-curve ordering of a (t, h, w) token grid.

Token layout only: video tokens are reordered along a Hilbert curve before they
are cut into blocks, so that a block of consecutive tokens is a compact
space-time region (DFSAttn abstract: Hilbert curve-based token reordering; GSRS
page, Figure 1, Figure 3 and Figure 6 captions: tokens reordered via Hilbert /
Gilbert curves before blocking).

The index is computed with Skilling's transpose method (J. Skilling,
"Programming the Hilbert curve", AIP Conf. Proc. 707, 381 (2004)): the
coordinates of a point in a 2^b cube are turned in place into the "transposed"
Hilbert index, whose bits, read most-significant first and interleaved across
the axes, form the index along the curve.  Written here from the published
description, vectorised over numpy arrays.
"""
from __future__ import annotations

import numpy as np


def _axes_to_transpose(coords: list[np.ndarray], bits: int) -> list[np.ndarray]:
    """Skilling's AxesToTranspose, applied elementwise to uint64 arrays."""
    x = [c.astype(np.uint64).copy() for c in coords]
    n = len(x)
    top = np.uint64(1) << np.uint64(bits - 1)
    # Undo the excess work of the recursive construction, from the top bit down.
    q = top
    while q > 1:
        p = q - np.uint64(1)
        for i in range(n):
            hit = (x[i] & q) != 0
            # where the bit is set, invert the low bits of axis 0
            x0_inv = x[0] ^ p
            # elsewhere, exchange the low bits of axis 0 and axis i
            t = (x[0] ^ x[i]) & p
            x0_swp = x[0] ^ t
            xi_swp = x[i] ^ t
            if i == 0:
                # exchange with itself is a no-op; only the inversion applies
                x[0] = np.where(hit, x0_inv, x[0])
            else:
                new0 = np.where(hit, x0_inv, x0_swp)
                x[i] = np.where(hit, x[i], xi_swp)
                x[0] = new0
        q >>= np.uint64(1)
    # Gray encode.
    for i in range(1, n):
        x[i] ^= x[i - 1]
    t = np.zeros_like(x[0])
    q = top
    while q > 1:
        t = np.where((x[n - 1] & q) != 0, t ^ (q - np.uint64(1)), t)
        q >>= np.uint64(1)
    for i in range(n):
        x[i] ^= t
    return x


def hilbert_index(coords: list[np.ndarray], bits: int) -> np.ndarray:
    """Hilbert-curve index of integer points in the cube [0, 2^bits)^n.

    The transposed form is read bit plane by bit plane from the most
    significant bit, axis 0 first, which yields the index along the curve.
    """
    n = len(coords)
    for c in coords:
        if np.any(c < 0) or np.any(c >= (1 << bits)):
            raise ValueError("coordinate outside the 2^bits cube")
    x = _axes_to_transpose(coords, bits)
    h = np.zeros_like(x[0])
    for j in range(bits - 1, -1, -1):
        for i in range(n):
            h = (h << np.uint64(1)) | ((x[i] >> np.uint64(j)) & np.uint64(1))
    return h


def hilbert_order(grid: tuple[int, int, int]) -> np.ndarray:
    """Permutation of frame-major token ids n = (t*Hg + h)*Wg + w into Hilbert order.

    Returns ``perm`` such that token ``perm[r]`` (frame-major id) sits at row r
    of the reordered sequence.  The curve is taken over the smallest
    power-of-two cube that encloses the grid; grid points are sorted by their
    index on it.
    """
    T, Hg, Wg = grid
    bits = max(1, int(np.ceil(np.log2(max(T, Hg, Wg)))))
    t, h, w = np.meshgrid(np.arange(T), np.arange(Hg), np.arange(Wg), indexing="ij")
    idx = hilbert_index([t.ravel(), h.ravel(), w.ravel()], bits)
    return np.argsort(idx, kind="stable").astype(np.int64)
