"""Heads are independent: reversing their order reverses every result, bit for bit.

The default step (scoring on raster Q and K, whose launch also writes K's and V's tiled
copies and the key-tile bounds; attention and the tile map with raster Q and O) runs on the
large workload twice: once as generated, once with the heads in reverse order (Q, K, V,
the per-head tile shapes, the estimator weights and the sampled query tiles all reversed).
Every kernel computes each (batch, head) item on its own, deterministically, so the kept
lists, the bounds, the output and the tile map of the second run must be those of the first
with the head axis reversed.  A kernel that paired one head's data with another head's tile
shape, bounds, weights or list fails, on any of the 40 heads."""
import numpy as np
import pytest
import torch

from workloads import get, make

pytestmark = pytest.mark.gpu

V = pytest.importorskip("video_dit_block_head_amd")
from video_dit_block_head_amd.pipeline import SparseAttention  # noqa: E402


def say(*a):
    print(*a, flush=True)


def test_reversed_heads_give_reversed_results():
    cfg = get("large")
    say("[gpu-head-order] large: generating")
    wl = make(cfg)
    B, H, N, nt, kk = cfg.batch, cfg.heads, cfg.n_tokens, cfg.n_tiles, cfg.topk[0]
    n_sel = 8
    up = lambda a: torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16).permute(0, 2, 1, 3).contiguous()
    q0, k0, v0 = up(wl.q), up(wl.k), up(wl.v)                       # [B, N, H, d]
    qtl0 = np.stack([wl.sample_tiles(h)[:n_sel] for h in range(H)]).astype(np.int32)[None].repeat(B, 0)
    w1, w2 = torch.from_numpy(wl.w1), torch.from_numpy(wl.w2)
    rev = list(range(H - 1, -1, -1))

    def step(shapes, q, k, v, w1, w2, qtl):
        geom = V.Geom(B, H, cfg.head_dim, cfg.grid, cfg.tile, shapes)
        sa = SparseAttention(geom, torch.bfloat16, w1, w2, score_scale=cfg.score_scale)
        idx = sa.score_raster(q, kk, k=k, tile_k=True, v=v)
        out = torch.empty_like(q)
        sa.attend_raster(q, idx, out)
        tmap = torch.empty((B, H, n_sel, nt), dtype=torch.float32, device="cuda")
        sa.tilemap_raster(q, torch.from_numpy(np.ascontiguousarray(qtl)).cuda(), n_sel, tmap)
        torch.cuda.synchronize()
        return idx.clone(), sa.k_bound.clone(), out, tmap

    say("[gpu-head-order] heads in order")
    a = step(list(wl.shapes), q0, k0, v0, w1, w2, qtl0)
    say("[gpu-head-order] heads reversed")
    r = step([wl.shapes[h] for h in rev], q0[:, :, rev].contiguous(), k0[:, :, rev].contiguous(),
             v0[:, :, rev].contiguous(), w1[rev].contiguous(), w2[rev].contiguous(), qtl0[:, rev])
    idx_a, kb_a, out_a, tm_a = a
    idx_r, kb_r, out_r, tm_r = r
    assert torch.equal(idx_r, idx_a[:, rev]), "kept lists"
    assert torch.equal(kb_r, kb_a[:, rev]), "key-tile bounds"
    assert torch.equal(out_r.view(torch.int16), out_a[:, :, rev].contiguous().view(torch.int16)), "attention output"
    assert torch.equal(tm_r, tm_a[:, rev]), "tile map"
    say("[gpu-head-order] large: lists, bounds, output and tile map reversed bit for bit")
