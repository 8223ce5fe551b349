"""Synthetic workloads for distilled sparse attention over video-DiT latents.

The pages (Veda, "Technical Summary", §4 Experimental Results) run Waver-T2V-12B and
Wan2.1-T2V-14B at up to 720P and 241 frames; their latent grids, head counts and
weights are not available here.  The five workloads below stand in for them: synthetic
Q/K/V with the attention shapes of 1.3B-, 14B- and 720P-10 s-scale DiTs, a randomly
initialised per-head estimator, and a fixed fraction of kept key tiles.

This module is data only.  It holds no step of the method.
"""
from dataclasses import dataclass, field, replace
from typing import List, Optional, Tuple

Shape3 = Tuple[int, int, int]

#: candidate per-head tile factorisations (p_t, p_h, p_w) of a 128-token tile
SHAPES_128 = [(2, 8, 8), (4, 4, 8), (1, 8, 16), (8, 4, 4)]


@dataclass(frozen=True)
class Config:
    name: str
    index: int
    batch: int
    heads: int
    head_dim: int
    dtype: str                      # "f32" or "bf16": storage type of Q, K, V
    grid: Shape3                    # latent (T, H, W)
    tile: int                       # tokens per tile P
    shape_list: Tuple[Shape3, ...]  # candidate tile shapes, in order
    topk: Tuple[int, ...]           # kept key tiles per query tile; first entry is the headline
    n_sink: int                     # keys whose norm is scaled x4
    seed: int
    sampled_q_tiles: Optional[int]  # query tiles per head checked by the oracle (None: all)
    mlp_hidden: int = 256
    mlp_out: int = 64
    score_scale: float = 1.0 / 8.0
    unit_axis_scale: bool = False   # per-head (t,h,w) position-code scales all 1.0
    padded: bool = False            # cycle every listed shape, also those that do not divide the grid

    @property
    def n_tokens(self) -> int:
        t, h, w = self.grid
        return t * h * w

    @property
    def n_tiles(self) -> int:
        return self.n_tokens // self.tile

    def valid_shapes(self) -> List[Shape3]:
        """Shapes of the list that divide the grid on every axis, in list order."""
        t, h, w = self.grid
        out = [s for s in self.shape_list if t % s[0] == 0 and h % s[1] == 0 and w % s[2] == 0]
        for s in out:
            assert s[0] * s[1] * s[2] == self.tile
        return out

    def head_shapes(self) -> List[Shape3]:
        """Tile shape of each head: the valid shapes cycled by head index (every listed
        shape when the workload is padded)."""
        v = list(self.shape_list) if self.padded else self.valid_shapes()
        return [v[h % len(v)] for h in range(self.heads)]

    def head_tiles(self, h: int) -> int:
        """Tiles of head h on the grid padded up to whole tiles of its shape."""
        (t, hh, w), (pt, ph, pw) = self.grid, self.head_shapes()[h]
        return (-(-t // pt)) * (-(-hh // ph)) * (-(-w // pw))

    def kept_flops(self, k: int) -> float:
        """4 * N * N * d * (k / n_t) * heads * batch: the QK^T and PV products on kept tiles."""
        n = self.n_tokens
        return 4.0 * n * n * self.head_dim * (k / self.n_tiles) * self.heads * self.batch


def padded_variant(cfg: Config, name: Optional[str] = None, **changes) -> Config:
    """The same workload with the full shape list cycled over the heads, so that heads whose
    shape does not divide the grid get a padded tiling."""
    return replace(cfg, name=name or cfg.name + "-padded", padded=True, **changes)


CONFIGS = [
    Config("tiny", 0, 1, 1, 64, "f32", (4, 8, 8), 64, ((4, 4, 4),), (2,), 0, 0, None,
           unit_axis_scale=True),
    Config("small", 1, 1, 12, 128, "bf16", (8, 16, 32), 128,
           ((2, 8, 8), (8, 4, 4), (1, 8, 16), (4, 4, 8)), (6,), 4, 1, None),
    Config("mid", 2, 1, 12, 128, "bf16", (20, 32, 48), 128, tuple(SHAPES_128), (24,), 4, 2, None),
    Config("large", 3, 1, 40, 128, "bf16", (20, 48, 80), 128, tuple(SHAPES_128), (60, 600), 8, 3, 64),
    Config("long", 4, 1, 48, 128, "bf16", (40, 48, 80), 128, tuple(SHAPES_128) + ((16, 2, 4),),
           (120, 240, 60, 1200), 8, 4, 64),
]

BY_NAME = {c.name: c for c in CONFIGS}


def get(name_or_index) -> Config:
    if isinstance(name_or_index, int):
        return CONFIGS[name_or_index]
    return BY_NAME[name_or_index]
