"""Out-of-range tile indices are clamped, as include/veda.h states, and nothing else changes.

The attention calls clamp each kept-list entry into [0, n_t) before they use it (for the
copy of the key tile and for its norm bound), and the tile map clamps its query-tile list
the same way.  So a list with entries below 0 and at or past n_t must give, bit for bit, the
output of the same list with those entries replaced by 0 and n_t - 1 beforehand.  (Both
results are "not meaningful" as attention: a clamped list can repeat a tile.  What is
checked is that the kernels read only the clamped tiles.)"""
import numpy as np
import pytest
import torch

from workloads import get, make

pytestmark = pytest.mark.gpu

V = pytest.importorskip("video_dit_block_head_amd")
from video_dit_block_head_amd.pipeline import SparseAttention  # noqa: E402


def say(*a):
    print(*a, flush=True)


def setup(name):
    cfg = get(name)
    say(f"[gpu-clamp] {name}: generating")
    wl = make(cfg)
    geom = V.Geom(cfg.batch, cfg.heads, cfg.head_dim, cfg.grid, cfg.tile, wl.shapes)
    up = lambda a: torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16).permute(0, 2, 1, 3).contiguous()
    q, k, v = up(wl.q), up(wl.k), up(wl.v)
    sa = SparseAttention(geom, torch.bfloat16, torch.from_numpy(wl.w1), torch.from_numpy(wl.w2),
                         score_scale=cfg.score_scale)
    return cfg, wl, geom, sa, q, k, v


def plant(idx, nt, seed):
    """A copy of idx with about a quarter of its entries moved out of range, and the same
    list clamped."""
    g = torch.Generator().manual_seed(seed)
    raw = idx.cpu().clone()
    sel = torch.rand(raw.shape, generator=g) < 0.25
    bad = torch.tensor([-1, -7, nt, nt + 13, 1 << 30, -(1 << 30)], dtype=torch.int32)
    pick = bad[torch.randint(0, len(bad), raw.shape, generator=g)]
    raw[sel] = pick[sel]
    return raw.cuda(), raw.clamp(0, nt - 1).cuda()


@pytest.mark.parametrize("name", ["small", "large"])
def test_attention_clamps_kept_list(name):
    cfg, wl, geom, sa, q, k, v = setup(name)
    kk, nt = cfg.topk[0], cfg.n_tiles
    idx = sa.score_raster(q, kk, k=k, tile_k=True, v=v)
    raw, clamped = plant(idx, nt, seed=5)
    assert int(raw.min()) < 0 and int(raw.max()) >= nt
    for bound in (True, False):
        outs = []
        for lst in (raw, clamped):
            out = torch.empty_like(q)
            V.veda_sparse_attn_fwd_raster(geom, q, sa.k_t, sa.v_t, lst, kk, sa.softmax_scale, out, k_layout=V.ROWS,
                                          v_layout=V.ROWS, k_bound=sa.k_bound if bound else None)
            outs.append(out)
        torch.cuda.synchronize()
        assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16)), (name, bound)
        say(f"[gpu-clamp] {name}: attention, bounds {'given' if bound else 'absent'}: out-of-range entries "
            f"give the clamped list's output bit for bit")


def test_tilemap_clamps_query_tiles():
    cfg, wl, geom, sa, q, k, v = setup("small")
    B, H, nt = cfg.batch, cfg.heads, cfg.n_tiles
    sa.gather_kv(k, v)
    n_sel = 6
    g = torch.Generator().manual_seed(9)
    raw = torch.randint(0, nt, (B, H, n_sel), generator=g, dtype=torch.int32)
    raw[..., 0] = -4
    raw[..., 1] = nt + 2
    raw[..., 2] = 1 << 30
    clamped = raw.clamp(0, nt - 1)
    maps = []
    for lst in (raw.cuda(), clamped.cuda()):
        out = torch.empty((B, H, n_sel, nt), dtype=torch.float32, device="cuda")
        sa.tilemap_raster(q, lst, n_sel, out)
        maps.append(out)
    torch.cuda.synchronize()
    assert torch.equal(maps[0], maps[1])
    say("[gpu-clamp] small: tile map: out-of-range query tiles give the clamped list's map bit for bit")
