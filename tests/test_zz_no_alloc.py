"""The no-allocation scoring call (veda_trippool_score_raster_noalloc, static scratch) through
the C ABI against the workspace call it mirrors (veda_trippool_score_raster), which the
parity tests check against the oracle: scores, probabilities, descriptors, key-tile bounds
and the top-k lists must be bit-identical.  Two calls in a row on one GPU, the second with a smaller
problem (so the shared scratch holds the first call's values when the second starts)."""
import numpy as np
import pytest
import torch

from workloads import get, make

pytestmark = pytest.mark.gpu

V = pytest.importorskip("video_dit_block_head_amd")


def say(*a):
    print(*a, flush=True)


def run_case(name, topk, k_layout):
    cfg = get(name)
    wl = make(cfg)
    B, H, d, P, nt = cfg.batch, cfg.heads, cfg.head_dim, cfg.tile, cfg.n_tiles
    geom = V.Geom(B, H, d, cfg.grid, P, wl.shapes)
    up = lambda a: torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16).permute(0, 2, 1, 3).contiguous()
    q, k, v = up(wl.q), up(wl.k), up(wl.v)
    if k_layout == V.ROWS:
        kt = torch.empty((B, H, geom.n_tiled, d), dtype=torch.bfloat16, device="cuda")
        V.veda_tile_gather(geom, k, kt, V.ROWS)
        k = kt
    w1, w2 = torch.from_numpy(wl.w1).cuda(), torch.from_numpy(wl.w2).cuda()

    def outputs():
        return dict(scores=torch.full((B, H, nt, nt), float("nan"), device="cuda"),
                    probs=torch.full((B, H, nt, nt), float("nan"), device="cuda"),
                    q_desc=torch.full((B, H, nt, 3 * d), float("nan"), device="cuda"),
                    k_desc=torch.full((B, H, nt, 3 * d), float("nan"), device="cuda"),
                    k_bound=torch.full((B, H, nt), float("nan"), device="cuda"),
                    idx=torch.full((B, H, nt, topk), -1, dtype=torch.int32, device="cuda"))

    ref, got = outputs(), outputs()
    vin = {}
    if k_layout == V.RASTER:   # with a raster K, both calls also write K's and V's tile-major copies
        for key in ("k_tiled_out", "v_tiled_out"):
            ref[key] = torch.zeros((B, H, geom.n_tiled, d), dtype=torch.bfloat16, device="cuda")
            got[key] = torch.ones_like(ref[key])
        vin = dict(v=v)
    ws = torch.empty(V.veda_trippool_workspace_bytes(geom, 256, 64), dtype=torch.uint8, device="cuda")
    V.veda_trippool_score_raster(geom, q, k, w1, w2, score_scale=cfg.score_scale, topk=topk, workspace=ws,
                                 k_layout=k_layout, **vin, **ref)
    V.veda_trippool_score_raster_noalloc(geom, q, k, w1, w2, score_scale=cfg.score_scale, topk=topk,
                                         k_layout=k_layout, **vin, **got)
    torch.cuda.synchronize()
    for key in ref:
        a, b = ref[key], got[key]
        if a.dtype == torch.bfloat16:
            a, b = a.view(torch.int16), b.view(torch.int16)
        assert torch.equal(a, b), (name, key)
    say(f"[no-alloc] {name}: k={topk} layout={k_layout}: " + ", ".join(ref) + " identical")


def test_noalloc_matches_workspace_call_twice():
    run_case("mid", 24, V.RASTER)       # 12 heads x 240 tiles
    run_case("small", 6, V.ROWS)        # then a smaller problem on the same scratch


def test_noalloc_largest_workloads():
    run_case("large", 60, V.ROWS)       # 40 x 600 tiles
    run_case("long", 120, V.ROWS)       # 48 x 1200 tiles = 57600 <= 65536 (29.5 MB of 32 MiB)
    run_case("small", 6, V.RASTER)
