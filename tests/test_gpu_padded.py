"""GPU parity on padded tilings: per-head tile shapes that do not divide the latent grid,
so that the grid is padded up to whole tiles per head (n_t(h) tiles, some of them partial).

Each check compares the tiled path of the C ABI with the oracle's padded tiling
(tile_slots, TripPool over real rows, attention and tile map with padding keys masked),
on the workloads' own shape cycles: (8,4,4) on T = 20 (mid, large) and (16,2,4) on T = 40
(long), plus a small grid on which every listed shape but two divides.  Tolerances as in
test_gpu_parity: layout bit-exact; max/min bit-exact, mean 1e-6; scores 1.25e-5 and indices
exact outside the 1e-5 near-tie band; attention max-abs 2e-2 and relative Frobenius 1e-2;
tile map 1e-4 in log space.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle.veda_oracle as O
from conftest import record_measure
from workloads import SHAPES_128, get, make, padded_variant

pytestmark = pytest.mark.gpu

V = pytest.importorskip("video_dit_block_head_amd")
from video_dit_block_head_amd.pipeline import SparseAttention  # noqa: E402

CASES = {
    # 20 x 16 x 32: (8,4,4) gives 3*4*8 = 96 tiles and (16,2,4) 2*8*8 = 128, the others 80
    "small-padded": (padded_variant(get(1), name="small-padded", grid=(20, 16, 32), heads=5,
                                    shape_list=tuple(SHAPES_128) + ((16, 2, 4),), topk=(16,), seed=11,
                                    sampled_q_tiles=24), None, None),
    # batch 2 and k at its bound (the smallest n_t(h) = 80): every tile of the dividing heads
    "small-padded-b2-kmax": (padded_variant(get(1), name="small-padded-b2-kmax", batch=2, grid=(20, 16, 32), heads=3,
                                            shape_list=((8, 4, 4), (2, 8, 8), (16, 2, 4)), topk=(80,), seed=12,
                                            sampled_q_tiles=8), None, None),
    "mid-padded": (padded_variant(get(2), sampled_q_tiles=32), 3, 16),
    "large-padded": (padded_variant(get(3), topk=(60,)), 4, 16),
    "long-padded": (padded_variant(get(4), topk=(120,)), 4, 8),
}
# Position -> key order inside a channel-major tile: groups of 16 ordered 0-3, 8-11, 4-7, 12-15
COLS_KEY = np.array([16 * (p // 16) + [0, 1, 2, 3, 8, 9, 10, 11, 4, 5, 6, 7, 12, 13, 14, 15][p % 16]
                     for p in range(128)])


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def measure(line):
    say(line)
    record_measure(line)


def to_dev_raster(arr_hm):
    t = torch.from_numpy(arr_hm.view(np.int16)).cuda().view(torch.bfloat16)
    return t.permute(0, 2, 1, 3).contiguous()


def host(t):
    return t.float().cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


def bitwise_equal(a, b):
    return np.array_equal(np.asarray(a, np.float32).view(np.uint32), np.asarray(b, np.float32).view(np.uint32))


class PaddedRun:
    def __init__(self, name):
        cfg, self.n_heads, self.n_tiles_checked = CASES[name]
        self.cfg = cfg
        say(f"[gpu-padded] {name}: generating")
        wl = self.wl = make(cfg)
        B, H, d, P = cfg.batch, cfg.heads, cfg.head_dim, cfg.tile
        self.geom = V.Geom(B, H, d, cfg.grid, P, wl.shapes)
        assert self.geom.padded
        self.nt = nt = self.geom.n_tiles
        self.kk = cfg.topk[0]
        say(f"[gpu-padded] {name}: n_t per head {sorted(set(self.geom.head_tiles(h) for h in range(H)))}, "
            f"k={self.kk}")
        self.sa = SparseAttention(self.geom, torch.bfloat16, torch.from_numpy(wl.w1), torch.from_numpy(wl.w2),
                                  score_scale=cfg.score_scale)
        self.q, self.k, self.v = (to_dev_raster(a) for a in (wl.q, wl.k, wl.v))
        self.sa.gather(self.q, self.k, self.v)
        self.scores = torch.empty((B, H, nt, nt), dtype=torch.float32, device="cuda")
        self.qd = torch.empty((B, H, nt, 3 * d), dtype=torch.float32, device="cuda")
        self.kd = torch.empty_like(self.qd)
        self.idx = self.sa.score(self.kk, scores=self.scores, q_desc=self.qd, k_desc=self.kd)
        self.lse = torch.empty((B, H, self.geom.n_tiled), dtype=torch.float32, device="cuda")
        self.sa.attend(self.idx, self.lse)
        self.out = torch.empty_like(self.q)
        self.sa.scatter(self.out)
        torch.cuda.synchronize()
        say(f"[gpu-padded] {name}: GPU path done")
        self._oh = {}

    def heads(self):
        """The heads whose shape does not divide the grid, and the first one whose shape does."""
        T, Hh, W = self.cfg.grid
        pad = [h for h, (pt, ph, pw) in enumerate(self.wl.shapes) if T % pt or Hh % ph or W % pw]
        div = [h for h in range(self.cfg.heads) if h not in pad][:1]
        return sorted(div + (pad if self.n_heads is None else pad[:self.n_heads - 1]))

    def pairs(self):
        """(batch, head) pairs checked against the oracle."""
        return [(b, h) for b in range(self.cfg.batch) for h in self.heads()]

    def oracle_head(self, b, h):
        if (b, h) not in self._oh:
            self._oh.clear()
            slots = O.tile_slots(self.cfg.grid, self.wl.shapes[h])
            self._oh[(b, h)] = tuple(O.to_tiles(self.wl.head(w, b, h), slots) for w in ("q", "k", "v")) + (slots,)
        return self._oh[(b, h)]

    def v_cols(self):
        """V gathered channel-major (VEDA_TILE_COLS), made once."""
        if not hasattr(self, "_v_cols"):
            self._v_cols = torch.empty_like(self.sa.v_t)
            V.veda_tile_gather(self.geom, self.v, self._v_cols, V.COLS)
            torch.cuda.synchronize()
        return self._v_cols

    def q_tiles(self, h):
        t = self.wl.sample_tiles(h)
        if self.n_tiles_checked is not None:
            t = t[np.linspace(0, len(t) - 1, self.n_tiles_checked).astype(int)]
        return t


@pytest.fixture(scope="module", params=list(CASES))
def r(request):
    run = PaddedRun(request.param)
    yield run
    del run
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_padded_gather(r):
    cfg, P, d = r.cfg, r.cfg.tile, r.cfg.head_dim
    for b, h in r.pairs():
        qt, kt, vt, slots = r.oracle_head(b, h)
        n = len(slots)
        gq, gk = host(r.sa.q_t[b, h]), host(r.sa.k_t[b, h])
        assert bitwise_equal(gq[:n], qt) and bitwise_equal(gk[:n], kt), (cfg.name, h)
        assert not gq[n:].any() and not gk[n:].any(), (cfg.name, h, "rows past the head's tiles")
        gv = host(r.sa.v_t[b, h])
        assert bitwise_equal(gv[:n], vt) and not gv[n:].any(), (cfg.name, h, "v")
        ntile = n // P
        vcols = host(r.v_cols()[b, h]).reshape(r.nt, d, P).transpose(0, 2, 1)[:ntile]
        assert bitwise_equal(vcols, vt.reshape(ntile, P, d)[:, COLS_KEY[:P], :]), (cfg.name, h, "v channel-major")
    back = torch.empty_like(r.q)
    V.veda_tile_gather(r.geom, back, r.sa.q_t, V.ROWS, inverse=True)
    torch.cuda.synchronize()
    assert torch.equal(back.view(torch.int16), r.q.view(torch.int16))


def test_padded_descriptors(r):
    cfg, P, d = r.cfg, r.cfg.tile, r.cfg.head_dim
    for b, h in r.pairs():
        qt, kt, _, slots = r.oracle_head(b, h)
        ntile = len(slots) // P
        for x, gd in ((qt, r.qd), (kt, r.kd)):
            ref = O.trippool(x, P, valid=slots >= 0)
            got = host(gd[b, h])[:ntile]
            assert bitwise_equal(got[:, d:], ref[:, d:]), (cfg.name, h)
            err = np.abs(got[:, :d] - ref[:, :d]) / np.maximum(np.abs(ref[:, :d]), 1.0)
            assert err.max() <= 1e-6, (cfg.name, h, err.max())


def test_padded_key_tile_bounds(r):
    """Each key tile's row-norm bound, sqrt(sum_c max(max_c^2, min_c^2)) over the oracle's
    padded max and min descriptors (real rows only), 0 past a head's own tiles; and the
    attention's running-maximum softmax (no bounds) against the oracle, beside the fixed
    offset that test_padded_attention checks."""
    cfg, P, d = r.cfg, r.cfg.tile, r.cfg.head_dim
    kb = host(r.sa.k_bound)
    o_run = torch.empty_like(r.sa.o_t)
    V.veda_sparse_attn_fwd(r.geom, r.sa.q_t, r.sa.k_t, r.sa.v_t, r.idx, r.kk, r.sa.softmax_scale, o_run)
    torch.cuda.synchronize()
    worst = mx = 0.0
    for b, h in r.pairs():
        qt, kt, vt, slots = r.oracle_head(b, h)
        ntile = len(slots) // P
        desc = O.trippool(kt, P, valid=slots >= 0)
        ref = np.sqrt((np.maximum(np.abs(desc[:, d:2 * d]), np.abs(desc[:, 2 * d:])) ** 2).sum(1))
        worst = max(worst, float(np.abs(kb[b, h, :ntile] / ref - 1).max()))
        assert not kb[b, h, ntile:].any(), (cfg.name, h, "bounds past the head's tiles")
        tiles = r.q_tiles(h)
        ref_o = O.sparse_attention(qt, kt, vt, host(r.idx[b, h]).astype(np.int64), P, 1 / math.sqrt(d),
                                   q_tiles=tiles, key_valid=slots >= 0)
        rows = (tiles[:, None] * P + np.arange(P)[None]).ravel()
        real = slots[rows] >= 0
        mx = max(mx, float(np.abs(host(o_run[b, h])[rows][real] - ref_o[real]).max()))
    measure(f"[gpu-padded] {cfg.name}: key-tile bounds max rel err {worst:.3g}; running-maximum attention "
            f"max|dO| {mx:.3g}")
    assert worst <= 1e-5 and mx <= 2e-2


def test_padded_scores_topk(r):
    cfg, P = r.cfg, r.cfg.tile
    worst, exempt, rows = 0.0, 0, 0
    for b, h in r.pairs():
        qt, kt, _, slots = r.oracle_head(b, h)
        valid = slots >= 0
        ntile = len(slots) // P
        yq = O.mlp(O.trippool(qt, P, valid=valid), r.wl.w1[h], r.wl.w2[h])
        yk = O.mlp(O.trippool(kt, P, valid=valid), r.wl.w1[h], r.wl.w2[h])
        s = O.tile_scores(yq, yk, cfg.score_scale)
        gs = host(r.scores[b, h])
        worst = max(worst, float(np.abs(gs[:ntile, :ntile] - s).max()))
        assert np.all(np.isneginf(gs[:ntile, ntile:])), (cfg.name, h, "columns past the head's tiles")
        idx = host(r.idx[b, h]).astype(np.int64)
        s32 = s.astype(np.float32)
        for i in range(ntile):
            ok, ex = O.topk_agrees(s32[i], idx[i], r.kk)
            assert ok, (cfg.name, h, i, idx[i])
            exempt += ex
            rows += 1
    measure(f"[gpu-padded] {cfg.name}: score max|err| {worst:.3g} over {rows} rows of {len(r.pairs())} heads, "
            f"{exempt} rows in the near-tie band")
    assert worst <= 1.25e-5   # as for dividing shapes (measured <= 8e-6 on these padded cases)


def test_padded_attention(r):
    cfg, P = r.cfg, r.cfg.tile
    scale = 1 / math.sqrt(cfg.head_dim)
    num = den = mx = lse_err = 0.0
    for b, h in r.pairs():
        qt, kt, vt, slots = r.oracle_head(b, h)
        tiles = r.q_tiles(h)
        idx = host(r.idx[b, h]).astype(np.int64)
        ref, ref_lse = O.sparse_attention(qt, kt, vt, idx, P, scale, q_tiles=tiles, return_lse=True,
                                          key_valid=slots >= 0)
        rows = (tiles[:, None] * P + np.arange(P)[None]).ravel()
        real = slots[rows] >= 0                               # padding query rows carry no token
        got = host(r.sa.o_t[b, h])[rows][real]
        ref = ref[real]
        num += float(((got - ref) ** 2).sum())
        den += float((ref ** 2).sum())
        mx = max(mx, float(np.abs(got - ref).max()))
        lse_err = max(lse_err, float(np.abs(host(r.lse[b, h])[rows][real] - ref_lse[real]).max()))
        # the raster output is the tiled output scattered through the slots
        sl = slots[slots >= 0]
        assert bitwise_equal(host(r.out[b, :, h])[sl], host(r.sa.o_t[b, h])[:len(slots)][slots >= 0]), (cfg.name, h)
    rel = math.sqrt(num / den)
    measure(f"[gpu-padded] {cfg.name} k={r.kk}: {len(r.pairs())} heads: max|dO| {mx:.3g}  relFro {rel:.3g}  "
            f"max|dLSE| {lse_err:.3g}")
    assert mx <= 2e-2 and rel <= 1e-2 and lse_err <= 4e-3


def test_padded_tilemap(r):
    cfg, P = r.cfg, r.cfg.tile
    B, H = cfg.batch, cfg.heads
    n_sel = cfg.sampled_q_tiles
    qtl = torch.from_numpy(np.stack([r.wl.sample_tiles(h) for h in range(H)]).astype(np.int32)[None]
                           .repeat(B, 0)).cuda()
    tm = torch.empty((B, H, n_sel, r.nt), dtype=torch.float32, device="cuda")
    say(f"[gpu-padded] {cfg.name}: tile map, {n_sel} query tiles per head")
    r.sa.tilemap(qtl, n_sel, tm)
    torch.cuda.synchronize()
    tmh = host(tm)
    worst = 0.0
    n_check = 8 if r.n_tiles_checked is not None else n_sel
    for b, h in r.pairs():
        qt, kt, _, slots = r.oracle_head(b, h)
        ntile = len(slots) // P
        sel = np.linspace(0, n_sel - 1, n_check).astype(int)
        ref = O.tilemap(qt, kt, P, 1 / math.sqrt(cfg.head_dim), q_tiles=r.wl.sample_tiles(h)[sel],
                        key_valid=slots >= 0, query_valid=slots >= 0)
        got = tmh[b, h, sel]
        assert not got[:, ntile:].any(), (cfg.name, h, "columns past the head's tiles")
        got = got[:, :ntile]
        keep = ref >= 1e-30
        assert np.all(got[~keep] < 1e-25)
        worst = max(worst, float(np.abs(np.log(got[keep]) - np.log(ref[keep])).max()))
    measure(f"[gpu-padded] {cfg.name}: tile map {n_check} rows x {len(r.pairs())} heads: max|dlog M| {worst:.3g}")
    assert worst <= 1e-4      # as for dividing shapes (measured <= 9.4e-6 on these padded cases)


def test_padded_raster_path(r):
    """The raster calls on a padded tiling (Q and O raster, K tiled for attention and the
    tile map) give bit-identical results to the tiled calls above, which are checked
    against the oracle; the scoring pass that also tiles K writes the gather's copy,
    zero rows included."""
    cfg, sa, g = r.cfg, r.sa, r.geom
    B, H, nt, P, d = cfg.batch, cfg.heads, r.nt, cfg.tile, cfg.head_dim
    say(f"[gpu-padded] {cfg.name}: raster path")
    for k_layout in (V.RASTER, V.ROWS):
        scores, qd, kd = torch.empty_like(r.scores), torch.empty_like(r.qd), torch.empty_like(r.kd)
        idx = torch.full_like(r.idx, -1)
        k_copy = torch.full_like(sa.k_t, float("nan")) if k_layout == V.RASTER else None
        v_copy = torch.full_like(sa.v_t, float("nan"))
        kb = torch.full_like(sa.k_bound, float("nan"))
        V.veda_trippool_score_raster(g, r.q, r.k if k_layout == V.RASTER else sa.k_t, sa.w1, sa.w2,
                                     score_scale=cfg.score_scale, scores=scores, q_desc=qd, k_desc=kd, topk=r.kk,
                                     idx=idx, workspace=sa.ws, k_layout=k_layout, k_tiled_out=k_copy,
                                     v=r.v, v_tiled_out=v_copy, k_bound=kb)
        torch.cuda.synchronize()
        assert torch.equal(v_copy.view(torch.int16), sa.v_t.view(torch.int16)), (cfg.name, "V's copy")
        assert torch.equal(qd, r.qd) and torch.equal(kd, r.kd), (cfg.name, k_layout)
        assert torch.equal(kb, sa.k_bound), (cfg.name, k_layout, "key-tile bounds")
        for h in range(H):   # a head's own rows (the rows past its tiles are not written)
            nth = g.head_tiles(h)
            assert torch.equal(scores[:, h, :nth], r.scores[:, h, :nth]), (cfg.name, k_layout, h)
            assert torch.equal(idx[:, h, :nth], r.idx[:, h, :nth]), (cfg.name, k_layout, h)
        if k_copy is not None:
            assert torch.equal(k_copy.view(torch.int16), sa.k_t.view(torch.int16)), cfg.name
    out = torch.zeros_like(r.q)
    lse = torch.empty((B, H, g.n_tokens), dtype=torch.float32, device="cuda")
    sa.attend_raster(r.q, r.idx, out, lse)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), r.out.view(torch.int16)), cfg.name
    # V channel-major (the attention above read it tile-major), in both calls
    v_cols = r.v_cols()
    o_t = torch.empty_like(sa.o_t)
    lse_t2 = torch.empty_like(r.lse)
    V.veda_sparse_attn_fwd(g, sa.q_t, sa.k_t, v_cols, r.idx, r.kk, sa.softmax_scale, o_t, lse_t2, v_layout=V.COLS,
                           k_bound=sa.k_bound)
    out2 = torch.zeros_like(r.q)
    V.veda_sparse_attn_fwd_raster(g, r.q, sa.k_t, v_cols, r.idx, r.kk, sa.softmax_scale, out2, k_layout=V.ROWS,
                                  v_layout=V.COLS, k_bound=sa.k_bound)
    torch.cuda.synchronize()
    for h in range(H):   # a head's own rows (rows past its tiles are not written)
        rows = g.head_tiles(h) * P
        assert torch.equal(o_t[:, h, :rows].view(torch.int16), sa.o_t[:, h, :rows].view(torch.int16)), (cfg.name, h)
        assert torch.equal(lse_t2[:, h, :rows], r.lse[:, h, :rows]), (cfg.name, h)
    assert torch.equal(out2.view(torch.int16), r.out.view(torch.int16)), cfg.name
    del o_t, out2
    lse_r, lse_t = lse.cpu().numpy(), r.lse.cpu().numpy()
    for b in range(B):
        for h in range(H):
            slots = O.tile_slots(cfg.grid, r.wl.shapes[h])
            real = slots >= 0
            assert bitwise_equal(lse_r[b, h, slots[real]], lse_t[b, h, :len(slots)][real]), (cfg.name, h)
    n_sel = min(8, cfg.sampled_q_tiles)
    qtl = torch.from_numpy(np.stack([r.wl.sample_tiles(h)[:n_sel] for h in range(H)]).astype(np.int32)[None]
                           .repeat(B, 0)).cuda().contiguous()
    m_t = torch.empty((B, H, n_sel, nt), dtype=torch.float32, device="cuda")
    m_r = torch.empty_like(m_t)
    l_t = torch.empty((B, H, n_sel * P), dtype=torch.float32, device="cuda")
    l_r = torch.empty_like(l_t)
    sa.tilemap(qtl, n_sel, m_t, l_t)
    sa.tilemap_raster(r.q, qtl, n_sel, m_r, l_r)
    torch.cuda.synchronize()
    assert torch.equal(m_t, m_r) and torch.equal(l_t, l_r), cfg.name


def test_padded_distill(r):
    """The distillation step on a padded tiling against the oracle: each head's logits,
    targets and gradients cover its own n_t(h) key tiles (TripPool over real rows only);
    a head with fewer tiles than the widest has zero target columns past them."""
    cfg, sa, g = r.cfg, r.sa, r.geom
    B, H, P, d, nt = cfg.batch, cfg.heads, cfg.tile, cfg.head_dim, r.nt
    n_sel = min(16, min(g.head_tiles(h) for h in range(H)))
    rng = np.random.default_rng(cfg.seed + 600)
    sel = np.stack([np.stack([np.sort(rng.choice(g.head_tiles(h), n_sel, replace=False)) for h in range(H)])
                    for _ in range(B)])
    tgt = np.zeros((B, H, n_sel, nt), np.float32)
    descs, q_tiles, targets = {}, {}, {}
    say(f"[gpu-padded] {cfg.name}: distillation, oracle descriptors of {B * H} heads")
    for b in range(B):
        for h in range(H):
            slots = O.tile_slots(cfg.grid, r.wl.shapes[h])
            valid = slots >= 0
            qt, kt = (O.to_tiles(r.wl.head(w, b, h), slots) for w in ("q", "k"))
            nth = g.head_tiles(h)
            bh = b * H + h
            descs[(bh, h)] = (O.trippool(qt, P, valid=valid), O.trippool(kt, P, valid=valid))
            q_tiles[bh] = sel[b, h]
            t = (rng.random((n_sel, nth)) ** 4 + 1e-3).astype(np.float32)
            tgt[b, h, :, :nth] = t
            targets[bh] = t.astype(np.float64)
    loss_o, g1_o, g2_o = O.distill_grads(descs, r.wl.w1, r.wl.w2, q_tiles, targets, cfg.score_scale)
    loss, dw1, dw2 = sa.distill_step(torch.from_numpy(sel.astype(np.int32)).cuda(), torch.from_numpy(tgt).cuda())
    torch.cuda.synchronize()
    loss_err = abs(float(loss.item()) - loss_o) / abs(loss_o)
    rel = []
    for got, want in ((dw1, g1_o), (dw2, g2_o)):
        got = got.cpu().numpy().astype(np.float64)
        rel.append((np.linalg.norm(got - want) / np.linalg.norm(want), np.abs(got - want).max() / np.abs(want).max()))
    measure(f"[gpu-padded] {cfg.name}: distillation ({H} heads x {n_sel} rows): loss rel err {loss_err:.2g}; "
            f"dw1 relFro {rel[0][0]:.2g} max/max {rel[0][1]:.2g}; dw2 relFro {rel[1][0]:.2g} max/max {rel[1][1]:.2g}")
    assert loss_err <= 1e-5
    for fro, mx in rel:
        assert fro <= 1e-4 and mx <= 1e-3
