"""Batch entries are independent: a batch-2 step gives, per entry, what a batch-1 step of
that entry gives, bit for bit.

The large workload is generated with two batch entries (different data, the same per-head
tile shapes and estimator weights).  The default step (scoring with K's and V's tiled
copies and the key-tile bounds, attention and the tile map with raster Q and O) runs once
on both entries together and once on each entry alone; every kernel computes each (batch,
head) item on its own, so the kept lists, bounds, output and tile map must agree exactly.
A kernel that read one entry's data, bounds or list for the other, or mis-strided the
batch axis of a raster tensor or a workspace, fails."""
from dataclasses import replace

import numpy as np
import pytest
import torch

from workloads import get, make

pytestmark = pytest.mark.gpu

V = pytest.importorskip("video_dit_block_head_amd")
from video_dit_block_head_amd.pipeline import SparseAttention  # noqa: E402


def say(*a):
    print(*a, flush=True)


def test_batch_entries_independent():
    cfg = replace(get("large"), batch=2)
    say("[gpu-batch] large, batch 2: generating")
    wl = make(cfg)
    B, H, nt, kk = cfg.batch, cfg.heads, cfg.n_tiles, cfg.topk[0]
    n_sel = 8
    up = lambda a: torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16).permute(0, 2, 1, 3).contiguous()
    q, k, v = up(wl.q), up(wl.k), up(wl.v)                           # [2, N, H, d]
    qtl = np.stack([wl.sample_tiles(h)[:n_sel] for h in range(H)]).astype(np.int32)[None].repeat(B, 0)
    w1, w2 = torch.from_numpy(wl.w1), torch.from_numpy(wl.w2)

    def step(nb, q, k, v, qtl):
        geom = V.Geom(nb, H, cfg.head_dim, cfg.grid, cfg.tile, wl.shapes)
        sa = SparseAttention(geom, torch.bfloat16, w1, w2, score_scale=cfg.score_scale)
        idx = sa.score_raster(q, kk, k=k, tile_k=True, v=v)
        out = torch.empty_like(q)
        sa.attend_raster(q, idx, out)
        tmap = torch.empty((nb, H, n_sel, nt), dtype=torch.float32, device="cuda")
        sa.tilemap_raster(q, torch.from_numpy(np.ascontiguousarray(qtl)).cuda(), n_sel, tmap)
        torch.cuda.synchronize()
        return idx.clone(), sa.k_bound.clone(), out, tmap

    say("[gpu-batch] both entries together")
    both = step(B, q, k, v, qtl)
    for b in range(B):
        say(f"[gpu-batch] entry {b} alone")
        one = step(1, q[b:b + 1].contiguous(), k[b:b + 1].contiguous(), v[b:b + 1].contiguous(), qtl[b:b + 1])
        for name, x2, x1 in zip(("kept lists", "key-tile bounds", "output", "tile map"), both, one):
            a, c = x2[b:b + 1], x1
            if a.dtype == torch.bfloat16:
                a, c = a.view(torch.int16), c.view(torch.int16)
            assert torch.equal(a, c), (b, name)
        say(f"[gpu-batch] entry {b}: lists, bounds, output and tile map equal to the batch-2 step's, bit for bit")
