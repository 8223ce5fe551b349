"""Attention is positively homogeneous in V, and the kernel keeps that exactly.

Scaling V by 2^e changes no exponent of P and no normaliser, and every product and fp32
partial sum of P V scales by 2^e exactly while nothing overflows; so the bf16 output of the
scaled V must equal 2^e times the output of V, bit for bit, and the LSE must not move.

- the running softmax offset (no key-tile bounds) at e = 60: its exponentials stay at or
  below 2^8, far from the fp32 range even for V times 2^60;
- the fixed offset (key-tile bounds given) at e = 20: its exponentials can reach 2^64, so
  the range it leaves V is smaller (include/veda.h states it); 2^20 stays well inside.

A mistake that mixed V into the exponent or the normaliser, or an overflow, breaks it.
(A product below the fp32 normal range, flushed in one run and kept in the other, could in
principle move a last bit; such terms are 2^-100 below the sums here.)"""
import numpy as np
import pytest
import torch

from workloads import get, make

pytestmark = pytest.mark.gpu

V = pytest.importorskip("video_dit_block_head_amd")
from video_dit_block_head_amd.pipeline import SparseAttention  # noqa: E402


def say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("name", ["small", "large"])
def test_attention_homogeneous_in_v(name):
    cfg = get(name)
    say(f"[gpu-vscale] {name}: generating")
    wl = make(cfg)
    geom = V.Geom(cfg.batch, cfg.heads, cfg.head_dim, cfg.grid, cfg.tile, wl.shapes)
    up = lambda a: torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16).permute(0, 2, 1, 3).contiguous()
    q, k, v = up(wl.q), up(wl.k), up(wl.v)
    sa = SparseAttention(geom, torch.bfloat16, torch.from_numpy(wl.w1), torch.from_numpy(wl.w2),
                         score_scale=cfg.score_scale)
    kk = cfg.topk[0]
    idx = sa.score_raster(q, kk, k=k, tile_k=True, v=v)  # writes K's and V's tiled copies and the bounds
    torch.cuda.synchronize()
    vmax = float(sa.v_t.float().abs().max())
    B, N, H = cfg.batch, cfg.n_tokens, cfg.heads

    def attend(vt, bound):
        out = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
        V.veda_sparse_attn_fwd_raster(geom, q, sa.k_t, vt, idx, kk, sa.softmax_scale, out, lse, k_layout=V.ROWS,
                                      v_layout=V.ROWS, k_bound=sa.k_bound if bound else None)
        return out, lse

    for e, bound in ((60, False), (20, True)):
        say(f"[gpu-vscale] {name}: V x 2^{e}, key-tile bounds {'given' if bound else 'absent'} (max|v| {vmax:.3g})")
        vs = sa.v_t * float(2.0 ** e)  # exact: a power of two, far from the bf16 range
        assert torch.isfinite(vs).all()
        out, lse = attend(sa.v_t, bound)
        out_s, lse_s = attend(vs, bound)
        torch.cuda.synchronize()
        assert torch.isfinite(out_s.float()).all(), (name, e)
        want = (out.float() * float(2.0 ** e)).to(torch.bfloat16)
        assert torch.equal(out_s.view(torch.int16), want.view(torch.int16)), (name, e)
        assert torch.equal(lse_s, lse), (name, e)
        say(f"[gpu-vscale] {name}: e={e} output scaled bit for bit, LSE unchanged")


@pytest.mark.parametrize("name", ["small", "large"])
def test_attention_weights_sum_to_one(name):
    """Every key of a head carrying the same V row c: each output row is a convex combination
    of copies of c, so it must be c, and in bf16 exactly (the normaliser and the P V sums of
    the same rounded weights differ by a few fp32 ulps, far below half a bf16 ulp of c).  A
    normaliser that missed or double-counted terms, or weights not rounded alike on both
    sides, moves it.  Both softmax offsets; every row of every head at full size."""
    cfg = get(name)
    say(f"[gpu-vscale] {name}: generating")
    wl = make(cfg)
    geom = V.Geom(cfg.batch, cfg.heads, cfg.head_dim, cfg.grid, cfg.tile, wl.shapes)
    up = lambda a: torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16).permute(0, 2, 1, 3).contiguous()
    q, k, v = up(wl.q), up(wl.k), up(wl.v)
    sa = SparseAttention(geom, torch.bfloat16, torch.from_numpy(wl.w1), torch.from_numpy(wl.w2),
                         score_scale=cfg.score_scale)
    kk = cfg.topk[0]
    idx = sa.score_raster(q, kk, k=k, tile_k=True, v=v)
    B, N, H, d = cfg.batch, cfg.n_tokens, cfg.heads, cfg.head_dim
    # c[h]: head h's first V row (bf16 values), the same for every key of the head
    c = v[:, 0, :, :].clone()                                   # [B, H, d]
    vt = c[:, :, None, :].expand(B, H, geom.n_tiled, d).contiguous()
    want = c[:, None, :, :].expand(B, N, H, d)
    for bound in (True, False):
        out = torch.empty_like(q)
        V.veda_sparse_attn_fwd_raster(geom, q, sa.k_t, vt, idx, kk, sa.softmax_scale, out, k_layout=V.ROWS,
                                      v_layout=V.ROWS, k_bound=sa.k_bound if bound else None)
        torch.cuda.synchronize()
        same = out.view(torch.int16) == want.reshape(B, N, H, d).contiguous().view(torch.int16)
        say(f"[gpu-vscale] {name}: constant V per head, bounds {'given' if bound else 'absent'}: "
            f"{int(same.sum())} of {same.numel()} output values equal to c")
        assert bool(same.all()), (name, bound)
