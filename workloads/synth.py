"""Seeded synthetic video-token Q/K/V (and loss-gradient G) for the workloads.

Holds none of the method's arithmetic: it only draws the input tensors that
both the HIP path and the CPU oracle consume.

Recipe, per (b, h) with independent numpy streams
``default_rng([seed, cfg_id, b, h, stream])``:

1. Positions: video token (t, y, x) of a T x Hg x Wg grid, frame-major id
   n = (t*Hg + y)*Wg + x, normalised u = (t/(T-1), y/(Hg-1), x/(Wg-1)).
   With ``hilbert`` the video rows are permuted into 3-D Hilbert order.
2. Random Fourier features (stream 0, fixed across denoising steps):
   Omega ~ N(0, sigma^2)^{16x3}, beta ~ U[0, 2pi)^16,
   phi(u) = sqrt(2/16) cos(Omega u + beta).
3. Projections (stream 0): W ~ N(0,1)^{16xD} shared by Q and K, so that the
   expected q.k follows a Gaussian kernel of the position difference
   (space-time locality); a separate W_V for V.
4. Tensors (stream = step): Q = 0.5 eps_Q + alpha phi W, K = 0.5 eps_K + alpha phi W,
   V = 0.5 eps_V + phi W_V with eps ~ N(0,1); alpha = 1 + 0.125 (step-1) on
   multi-step workloads (attention grows more concentrated over denoising),
   else 1.
5. Additions: a text prefix of N(0,1) rows for Q, K, V (drawn after eps);
   vertical stripes: ceil(frac*N) key rows drawn without replacement get
   4 sqrt(D) e added and every query gets e added, e a per-head unit vector
   (stream 0), so stripe keys earn a +4 logit bonus from every query.
6. G ~ N(0,1) (stream 1000) for the training workload.

Values are formed in float32 (the Fourier product in float64) and, for the
bf16 dtype, rounded to bfloat16 with round-to-nearest-even.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .configs import Workload
from .hilbert import hilbert_order

N_FEATURES = 16


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), kept as float32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (r & np.uint32(0xFFFF0000)).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float32 values that are already exact bfloat16."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    if np.any(u & np.uint32(0xFFFF)):
        raise ValueError("values are not exact bfloat16")
    return (u >> np.uint32(16)).astype(np.uint16)


_POS_CACHE: dict[tuple, np.ndarray] = {}


def video_positions(w: Workload) -> np.ndarray:
    """Normalised (t, y, x) of every video token in sequence order, [Nv, 3] float64."""
    key = (w.grid, w.hilbert)
    if key not in _POS_CACHE:
        T, Hg, Wg = w.grid
        t, y, x = np.meshgrid(np.arange(T), np.arange(Hg), np.arange(Wg), indexing="ij")
        pos = np.stack([t.ravel(), y.ravel(), x.ravel()], axis=1).astype(np.float64)
        pos /= np.array([max(T - 1, 1), max(Hg - 1, 1), max(Wg - 1, 1)], dtype=np.float64)
        if w.hilbert:
            pos = pos[hilbert_order(w.grid)]
        _POS_CACHE[key] = pos
    return _POS_CACHE[key]


def head_tensors(w: Workload, b: int, h: int, step: int = 1, seed: int = 0,
                 want_grad: bool | None = None) -> dict[str, np.ndarray]:
    """float32 [N, D] arrays q, k, v (and g) of one (b, h), before any dtype rounding."""
    N, D = w.N, w.D
    prm = np.random.default_rng([seed, w.cfg_id, b, h, 0])
    omega = prm.normal(0.0, w.sigma, size=(N_FEATURES, 3))
    beta = prm.uniform(0.0, 2.0 * math.pi, size=N_FEATURES)
    W = prm.standard_normal((N_FEATURES, D))
    WV = prm.standard_normal((N_FEATURES, D))
    stripes = None
    if w.stripe_frac > 0.0:
        n_stripes = int(math.ceil(w.stripe_frac * N))
        stripes = prm.choice(N, size=n_stripes, replace=False)
        e = prm.standard_normal(D)
        e /= np.linalg.norm(e)

    u = video_positions(w)
    phi = math.sqrt(2.0 / N_FEATURES) * np.cos(u @ omega.T + beta)
    base_qk = (phi @ W).astype(np.float32)
    base_v = (phi @ WV).astype(np.float32)

    alpha = np.float32(1.0 + 0.125 * (step - 1)) if w.reduced_search else np.float32(1.0)
    nz = np.random.default_rng([seed, w.cfg_id, b, h, step])
    eq = nz.standard_normal((N, D), dtype=np.float32)
    ek = nz.standard_normal((N, D), dtype=np.float32)
    ev = nz.standard_normal((N, D), dtype=np.float32)
    P = w.text_prefix
    half = np.float32(0.5)
    q = half * eq
    k = half * ek
    v = half * ev
    q[P:] += alpha * base_qk
    k[P:] += alpha * base_qk
    v[P:] += base_v
    if P:
        q[:P] = nz.standard_normal((P, D), dtype=np.float32)
        k[:P] = nz.standard_normal((P, D), dtype=np.float32)
        v[:P] = nz.standard_normal((P, D), dtype=np.float32)
    if stripes is not None:
        k[stripes] += (4.0 * math.sqrt(D) * e).astype(np.float32)
        q += e.astype(np.float32)
    out = {"q": q, "k": k, "v": v}
    if want_grad if want_grad is not None else w.backward:
        out["g"] = np.random.default_rng([seed, w.cfg_id, b, h, 1000]).standard_normal(
            (N, D), dtype=np.float32)
    return out


def make_inputs(w: Workload, step: int = 1, dtype: str = "bf16", seed: int = 0,
                heads: list[tuple[int, int]] | None = None, threads: int = 8,
                want_grad: bool | None = None) -> dict[str, np.ndarray]:
    """float32 arrays [B, H, N, D] (exact bf16 values when dtype == "bf16").

    ``heads`` restricts generation to a list of (b, h); other heads stay zero.
    Every (b, h) has its own streams, so a subset equals the same heads of the
    full tensor.
    """
    if dtype not in ("bf16", "fp32"):
        raise ValueError(dtype)
    pairs = heads if heads is not None else [(b, h) for b in range(w.B) for h in range(w.H)]
    names = ["q", "k", "v"] + (["g"] if (want_grad if want_grad is not None else w.backward) else [])
    out = {n: np.zeros((w.B, w.H, w.N, w.D), dtype=np.float32) for n in names}

    def one(bh):
        b, h = bh
        t = head_tensors(w, b, h, step=step, seed=seed, want_grad=want_grad)
        for n in names:
            out[n][b, h] = round_to_bf16(t[n]) if dtype == "bf16" else t[n]

    video_positions(w)  # fill the cache before the threads start
    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        list(ex.map(one, pairs))
    return out
