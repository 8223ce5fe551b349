"""The library as a DiT block would call it, on one MI355X.

- A fused QKV projection emits one [B, N, 3, H, d] tensor; the raster calls take Q, K and V as
  strided views of it (token stride 3*H*d) and give bit for bit what contiguous copies give,
  with the output a view of a packed tensor as well, a contiguous tensor, or head-major
  storage (the output has strides of its own).
- The default step (scoring through the no-allocation call, its launch also writing K's and
  V's tiled copies; attention and tile map with raster Q and O) captured into a HIP graph:
  every replay, with eager work and synchronisations between them, gives the eager step's
  results bit for bit.
  The no-allocation call is there for exactly such callers: nothing in the captured step
  allocates or clears memory.
Both compare against the calls that test_gpu_parity checks against the oracle."""
import numpy as np
import pytest
import torch

from workloads import get, make

pytestmark = pytest.mark.gpu

V = pytest.importorskip("video_dit_block_head_amd")
from video_dit_block_head_amd.pipeline import SparseAttention  # noqa: E402


def say(*a):
    print(*a, flush=True)


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def setup(name):
    cfg = get(name)
    wl = make(cfg)
    geom = V.Geom(cfg.batch, cfg.heads, cfg.head_dim, cfg.grid, cfg.tile, wl.shapes)
    up = lambda a: torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16).permute(0, 2, 1, 3).contiguous()
    q, k, v = up(wl.q), up(wl.k), up(wl.v)
    sa = SparseAttention(geom, torch.bfloat16, torch.from_numpy(wl.w1), torch.from_numpy(wl.w2),
                         score_scale=cfg.score_scale)
    return cfg, wl, geom, sa, q, k, v


@pytest.mark.parametrize("name", ["small", "mid"])
def test_packed_qkv_views(name):
    cfg, wl, geom, sa, q, k, v = setup(name)
    kk = cfg.topk[0]
    say(f"[gpu-usage] {name}: packed QKV views")
    ref = torch.empty_like(q)
    sa.forward_raster(q, k, v, kk, ref)
    idx_ref = sa.idx_buffer(kk).clone()
    qkv = torch.stack([q, k, v], dim=2).contiguous()           # [B, N, 3, H, d]
    out_packed = torch.zeros_like(qkv)
    qv, kv_, vv, ov = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2], out_packed[:, :, 0]
    assert qv.stride(1) == 3 * cfg.heads * cfg.head_dim and not qv.is_contiguous()
    sa.forward_raster(qv, kv_, vv, kk, ov)
    torch.cuda.synchronize()
    assert torch.equal(sa.idx_buffer(kk), idx_ref), name
    assert torch.equal(bits(ov), bits(ref)), name
    assert not out_packed[:, :, 1:].any(), "the output view wrote outside its slots"
    # the output with strides of its own: a contiguous [B, N, H, d] tensor, and a head-major
    # [B, H, N, d] storage seen as [B, N, H, d]
    out_c = torch.zeros_like(ref)
    sa.forward_raster(qv, kv_, vv, kk, out_c)
    hm = torch.zeros((q.shape[0], q.shape[2], q.shape[1], q.shape[3]), dtype=q.dtype, device="cuda")
    out_h = hm.permute(0, 2, 1, 3)
    assert out_h.stride(1) != ov.stride(1) and out_h.stride(2) != ov.stride(2)
    sa.forward_raster(qv, kv_, vv, kk, out_h)
    torch.cuda.synchronize()
    assert torch.equal(bits(out_c), bits(ref)) and torch.equal(bits(out_h), bits(ref)), name


def test_graph_capture_noalloc_step():
    cfg, wl, geom, sa, q, k, v = setup("small")
    B, H, nt, kk, P = cfg.batch, cfg.heads, cfg.n_tiles, cfg.topk[0], cfg.tile
    n_sel = 8
    qtl = torch.from_numpy(np.stack([wl.sample_tiles(h)[:n_sel] for h in range(H)]).astype(np.int32)[None]
                           .repeat(B, 0)).cuda().contiguous()
    idx = torch.empty((B, H, nt, kk), dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    tmap = torch.empty((B, H, n_sel, nt), dtype=torch.float32, device="cuda")
    tm_ws = torch.empty(V.veda_oracle_tilemap_workspace_bytes(geom, n_sel), dtype=torch.uint8, device="cuda")

    def step():
        V.veda_trippool_score_raster_noalloc(geom, q, k, sa.w1, sa.w2, score_scale=cfg.score_scale, topk=kk,
                                             idx=idx, k_layout=V.RASTER, k_tiled_out=sa.k_t, v=v,
                                             v_tiled_out=sa.v_t, k_bound=sa.k_bound)
        V.veda_sparse_attn_fwd_raster(geom, q, sa.k_t, sa.v_t, idx, kk, sa.softmax_scale, out, k_layout=V.ROWS,
                                      k_bound=sa.k_bound)
        V.veda_oracle_tilemap_raster(geom, q, sa.k_t, sa.softmax_scale, qtl, n_sel, tmap, workspace=tm_ws,
                                     k_layout=V.ROWS)

    say("[gpu-usage] eager step (also looks up the static scratch before any capture)")
    step()
    torch.cuda.synchronize()
    want = [t.clone() for t in (idx, out, tmap, sa.k_t, sa.v_t, sa.k_bound)]
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                                   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    say("[gpu-usage] capturing the step")
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (idx, out, tmap, sa.k_t, sa.v_t, sa.k_bound):   # eager work between replays
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, ref in zip((idx, out, tmap, sa.k_t, sa.v_t, sa.k_bound), want):
            assert torch.equal(bits(got), bits(ref)), rep
        say(f"[gpu-usage] replay {rep}: identical to the eager step")
