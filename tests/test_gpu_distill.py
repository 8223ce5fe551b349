"""GPU parity of the estimator's distillation step (veda_distill_step) against the CPU
oracle's loss and chain-rule gradients.

Tolerances: loss within 1e-5 relative; gradients within 1e-4 relative Frobenius and 1e-3 of
their largest entry (fp32 arithmetic on the GPU, float64 in the oracle, the same inputs:
descriptors differ only by the fp32 accumulation of the tile means).  The in-place update
is checked against w - lr * dw in fp32 to 1 ulp-scale tolerance; repeated calls are
bit-identical."""
import math

import numpy as np
import pytest
import torch

import oracle.veda_oracle as O
from conftest import record_measure
from workloads import get, make

pytestmark = pytest.mark.gpu

V = pytest.importorskip("video_dit_block_head_amd")
from video_dit_block_head_amd.pipeline import SparseAttention  # noqa: E402


def say(*a):
    print(*a, flush=True)


def to_dev_raster(arr_hm, bf16):
    t = torch.from_numpy(arr_hm.view(np.int16) if bf16 else arr_hm).cuda()
    if bf16:
        t = t.view(torch.bfloat16)
    return t.permute(0, 2, 1, 3).contiguous()


# "dup": sampled with replacement and with a repeated tile in every (b, h) list (a tile
# sampled twice counts twice: two KL rows, two gradient contributions).  Rows of up to 64,
# 256, 640 and 1280 key tiles take different instantiations of the row kernel (tiny/small,
# mid, large, long).
CASES = [("tiny", 2, "map"), ("small", 8, "map"), ("mid", 16, "random"), ("small", 8, "dup"),
         ("large", 64, "random"), ("long", 64, "dup")]


@pytest.mark.parametrize("name,n_sel,target_kind", CASES, ids=[f"{c[0]}-{c[2]}" for c in CASES])
def test_distill_step_vs_oracle(name, n_sel, target_kind):
    cfg = get(name)
    say(f"[gpu-distill] {name}: generating")
    wl = make(cfg)
    B, H, d, P, nt = cfg.batch, cfg.heads, cfg.head_dim, cfg.tile, cfg.n_tiles
    bf16 = wl.is_bf16
    geom = V.Geom(B, H, d, cfg.grid, P, wl.shapes)
    sa = SparseAttention(geom, torch.bfloat16 if bf16 else torch.float32, torch.from_numpy(wl.w1),
                         torch.from_numpy(wl.w2), score_scale=cfg.score_scale)
    q, k, v = (to_dev_raster(a, bf16) for a in (wl.q, wl.k, wl.v))
    sa.gather(q, k, v)
    rng = np.random.default_rng(cfg.seed + 500)
    if target_kind == "dup":
        def pick():
            x = rng.choice(nt, n_sel, replace=True)
            x[-1] = x[0]  # at least one repeat
            return np.sort(x)
    else:
        def pick():
            return np.sort(rng.choice(nt, n_sel, replace=False))
    sel = np.stack([np.stack([pick() for _ in range(H)]) for _ in range(B)])
    # oracle side: descriptors of the tiled inputs, targets
    descs, q_tiles, targets = {}, {}, {}
    for b in range(B):
        for h in range(H):
            perm = O.tile_permutation(cfg.grid, wl.shapes[h])
            qt, kt = O.to_tiles(wl.head("q", b, h), perm), O.to_tiles(wl.head("k", b, h), perm)
            bh = b * H + h
            descs[(bh, h)] = (O.trippool(qt, P), O.trippool(kt, P))
            q_tiles[bh] = sel[b, h]
            if target_kind == "map":
                targets[bh] = O.tilemap(qt, kt, P, 1 / math.sqrt(d), q_tiles=sel[b, h])
            else:
                targets[bh] = rng.random((n_sel, nt)) ** 4 + 1e-3
    say(f"[gpu-distill] {name}: oracle gradients")
    loss_o, g1_o, g2_o = O.distill_grads(descs, wl.w1, wl.w2, q_tiles, targets, cfg.score_scale)
    tgt = np.stack([np.stack([targets[b * H + h] for h in range(H)]) for b in range(B)]).astype(np.float32)
    say(f"[gpu-distill] {name}: GPU step")
    qtl = torch.from_numpy(sel.astype(np.int32)).cuda()
    tgt_d = torch.from_numpy(tgt).cuda()
    loss, dw1, dw2 = sa.distill_step(qtl, tgt_d)
    torch.cuda.synchronize()
    loss_err = abs(float(loss.item()) - loss_o) / abs(loss_o)
    rel = []
    for got, want in ((dw1, g1_o), (dw2, g2_o)):
        got = got.cpu().numpy().astype(np.float64)
        rel.append((np.linalg.norm(got - want) / np.linalg.norm(want),
                    np.abs(got - want).max() / np.abs(want).max()))
    msg = (f"[gpu-distill] {name} ({target_kind}, {H} heads x {n_sel} rows of {nt} tiles): loss rel err {loss_err:.2g}; "
           f"dw1 relFro {rel[0][0]:.2g} max/max {rel[0][1]:.2g}; dw2 relFro {rel[1][0]:.2g} max/max {rel[1][1]:.2g}")
    say(msg)
    record_measure(msg)
    assert loss_err <= 1e-5, (float(loss.item()), loss_o)
    for fro, mx in rel:
        assert fro <= 1e-4 and mx <= 1e-3
    # deterministic, then the in-place update
    loss2, dw1b, dw2b = sa.distill_step(qtl, tgt_d)
    assert torch.equal(dw1, dw1b) and torch.equal(dw2, dw2b) and torch.equal(loss, loss2)
    w1_before, w2_before = sa.w1.clone(), sa.w2.clone()
    lr = 0.05
    sa.distill_step(qtl, tgt_d, lr=lr)
    torch.cuda.synchronize()
    assert torch.allclose(sa.w1, w1_before - lr * dw1, rtol=1e-6, atol=1e-7)
    assert torch.allclose(sa.w2, w2_before - lr * dw2, rtol=1e-6, atol=1e-7)


def test_distill_training_lowers_the_loss():
    """A few plain gradient steps on the small workload's sampled rows, against the tile
    map of the same rows computed by the library."""
    cfg = get("small")
    wl = make(cfg)
    B, H, d, P, nt = cfg.batch, cfg.heads, cfg.head_dim, cfg.tile, cfg.n_tiles
    geom = V.Geom(B, H, d, cfg.grid, P, wl.shapes)
    sa = SparseAttention(geom, torch.bfloat16, torch.from_numpy(wl.w1), torch.from_numpy(wl.w2),
                         score_scale=cfg.score_scale)
    sa.gather(*(to_dev_raster(a, True) for a in (wl.q, wl.k, wl.v)))
    rng = np.random.default_rng(7)
    sel = torch.from_numpy(np.stack([np.stack([np.sort(rng.choice(nt, 8, replace=False)) for _ in range(H)])
                                     for _ in range(B)]).astype(np.int32)).cuda()
    tmap = torch.empty((B, H, 8, nt), dtype=torch.float32, device="cuda")
    sa.tilemap(sel, 8, tmap)
    losses = []
    for _ in range(15):
        loss, _, _ = sa.distill_step(sel, tmap, lr=0.05)
        losses.append(float(loss.item()))
    say(f"[gpu-distill] loss over 15 steps: {[round(x, 4) for x in losses]}")
    assert all(math.isfinite(x) for x in losses)
    assert losses[-1] < 0.5 * losses[0]
