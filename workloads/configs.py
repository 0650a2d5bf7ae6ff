"""The five seeded synthetic workloads of this library's test and benchmark suite.

Each entry names a video-DiT attention layer shape (B, H, N, D), the token
block size, the Top-p threshold(s) and the structure the generator gives the
tokens.  The shapes stand in for the models the pages evaluate (CogVideoX,
Wan 2.1, HunyuanVideo, DSV-style DiT training); no model weights or prompts
are involved.
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int
    B: int
    H: int
    D: int
    grid: tuple[int, int, int]        # (T, Hg, Wg) latent video grid
    block: int
    top_p: tuple[float, ...]          # one threshold per denoising step
    sigma: float = 3.0                # Fourier-feature frequency scale
    text_prefix: int = 0              # leading N(0,1) text tokens, always kept
    hilbert: bool = False             # reorder video tokens along a 3-D Hilbert curve
    stripe_frac: float = 0.0          # fraction of key positions given a shared component
    reduced_search: bool = False      # steps >= 2 search only step 1's blocks
    backward: bool = False            # forward + backward with loss sum(O * G)
    note: str = field(default="", compare=False)

    @property
    def video_tokens(self) -> int:
        T, Hg, Wg = self.grid
        return T * Hg * Wg

    @property
    def N(self) -> int:
        return self.text_prefix + self.video_tokens

    @property
    def nb(self) -> int:
        return -(-self.N // self.block)

    @property
    def steps(self) -> int:
        return len(self.top_p)

    @property
    def keep_prefix_tokens(self) -> int:
        return self.text_prefix

    def dense_fwd_flop(self) -> float:
        return 4.0 * self.B * self.H * self.N * self.N * self.D


def _growing(p0: float, p1: float, n: int) -> tuple[float, ...]:
    return tuple(p0 + (p1 - p0) * s / (n - 1) for s in range(n))


WORKLOADS: dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("tiny", 1, B=1, H=2, D=64, grid=(4, 16, 16), block=64, top_p=(0.9,),
                 note="tiny reference case, fp32 and bf16"),
        Workload("cogvideox", 2, B=1, H=48, D=64, grid=(13, 30, 45), block=128, top_p=(0.9,),
                 sigma=4.0, text_prefix=226,
                 note="CogVideoX-like layer with a 226-token text prefix every query keeps"),
        Workload("wan", 3, B=1, H=40, D=128, grid=(21, 30, 52), block=128,
                 top_p=_growing(0.80, 0.95, 5), reduced_search=True,
                 note="Wan2.1-like layer over 5 denoising steps; steps 2-5 search step 1's blocks"),
        Workload("hunyuan", 4, B=1, H=24, D=128, grid=(33, 45, 80), block=128, top_p=(0.95,),
                 sigma=6.0, hilbert=True, stripe_frac=0.02,
                 note="HunyuanVideo-like long sequence, Hilbert order, vertical stripes"),
        Workload("dsv_train", 5, B=2, H=24, D=128, grid=(16, 32, 32), block=64, top_p=(0.9,),
                 backward=True, note="DSV-style training step: forward + backward"),
    ]
}


def get(name: str) -> Workload:
    return WORKLOADS[name]
