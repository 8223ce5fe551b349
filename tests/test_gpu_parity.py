"""GPU parity: every call of the C ABI against the CPU oracle on the seeded workloads.

Tolerances: indices exact unless the k-th/(k+1)-th fp32 oracle scores differ by < 1e-5
(then any near-tie choice is accepted); scores 1.25e-5; attention max-abs <= 2e-2 and
relative Frobenius <= 1e-2 for bf16 (1e-4 for fp32), LSE 4e-3 (1e-5); gather and TripPool
max/min bit-exact; tile map within 1e-4 in log space (1e-5 for fp32).  Large workloads
compare 64 sampled query tiles per head (the tile map: 8 per head, all 64 on two heads)."""
import math
import sys

import numpy as np
import pytest
import torch

import oracle.veda_oracle as O
from conftest import record_measure
from workloads import get, make

pytestmark = pytest.mark.gpu

V = pytest.importorskip("video_dit_block_head_amd")
from video_dit_block_head_amd.pipeline import SparseAttention, dense_index  # noqa: E402


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def measure(line):
    """Print a line of achieved figures and keep it for the run's terminal summary."""
    say(line)
    record_measure(line)


def to_dev_raster(arr_hm, bf16):
    """Head-major host array [B,H,N,d] -> contiguous GPU raster [B,N,H,d]."""
    t = torch.from_numpy(arr_hm.view(np.int16) if bf16 else arr_hm).cuda()
    if bf16:
        t = t.view(torch.bfloat16)
    return t.permute(0, 2, 1, 3).contiguous()


def host(t):
    return t.float().cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


class Run:
    """One workload on the GPU through the full path (headline k)."""

    def __init__(self, ci):
        cfg = self.cfg = get(ci)
        say(f"[gpu-parity] config {cfg.name}: generating")
        wl = self.wl = make(cfg)
        self.bf16 = wl.is_bf16
        B, H, N, d, P, nt = cfg.batch, cfg.heads, cfg.n_tokens, cfg.head_dim, cfg.tile, cfg.n_tiles
        self.geom = V.Geom(B, H, d, cfg.grid, P, wl.shapes)
        dt = torch.bfloat16 if self.bf16 else torch.float32
        say(f"[gpu-parity] config {cfg.name}: upload + full path, k={cfg.topk[0]}")
        self.sa = SparseAttention(self.geom, dt, torch.from_numpy(wl.w1), torch.from_numpy(wl.w2),
                                  score_scale=cfg.score_scale)
        self.q, self.k, self.v = (to_dev_raster(a, self.bf16) for a in (wl.q, wl.k, wl.v))
        self.sa.gather(self.q, self.k, self.v)
        self.scores = torch.empty((B, H, nt, nt), dtype=torch.float32, device="cuda")
        self.probs = torch.empty_like(self.scores)
        self.qd = torch.empty((B, H, nt, 3 * d), dtype=torch.float32, device="cuda")
        self.kd = torch.empty_like(self.qd)
        self.kk = cfg.topk[0]
        self.idx = self.sa.score(self.kk, scores=self.scores, probs=self.probs, q_desc=self.qd, k_desc=self.kd)
        self.lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
        self.sa.attend(self.idx, self.lse)
        self.out = torch.empty_like(self.q)
        self.sa.scatter(self.out)
        torch.cuda.synchronize()
        say(f"[gpu-parity] config {cfg.name}: GPU path done")
        self._oh = {}

    def heads(self, limit=None):
        H = self.cfg.heads
        return list(range(H)) if limit is None or limit >= H else list(np.linspace(0, H - 1, limit).astype(int))

    def oracle_head(self, b, h):
        """Tile-major float64 Q, K, V of (b, h) and the permutation (oracle's own)."""
        key = (b, h)
        if key not in self._oh:
            self._oh.clear()
            perm = O.tile_permutation(self.cfg.grid, self.wl.shapes[h])
            self._oh[key] = tuple(O.to_tiles(self.wl.head(w, b, h), perm) for w in ("q", "k", "v")) + (perm,)
        return self._oh[key]

    def q_tiles(self, h):
        return self.wl.sample_tiles(h)

    def v_cols(self):
        """V gathered channel-major (VEDA_TILE_COLS), made once."""
        if not hasattr(self, "_v_cols"):
            self._v_cols = torch.empty_like(self.sa.v_t)
            V.veda_tile_gather(self.geom, self.v, self._v_cols, V.COLS)
            torch.cuda.synchronize()
        return self._v_cols


CFGS = [0, 1, 2, 3, 4]


@pytest.fixture(scope="module", params=CFGS, ids=[get(i).name for i in CFGS])
def r(request):
    """One workload at a time (pytest groups the tests by workload)."""
    run = Run(request.param)
    yield run
    del run
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


HEAD_LIMIT = {0: None, 1: None, 2: None, 3: 6, 4: 4}        # heads for bit-exact layout checks
SCORE_HEADS = {0: None, 1: None, 2: None, 3: None, 4: None}  # heads for index parity (all)


# Position -> key order inside a channel-major tile: groups of 16 ordered 0-3, 8-11, 4-7, 12-15
COLS_KEY = np.array([16 * (p // 16) + [0, 1, 2, 3, 8, 9, 10, 11, 4, 5, 6, 7, 12, 13, 14, 15][p % 16]
                     for p in range(128)])


def bitwise_equal(a, b):
    return np.array_equal(np.asarray(a, np.float32).view(np.uint32), np.asarray(b, np.float32).view(np.uint32))


# ----------------------------------------------------------------------------- gather
def test_gather_bitexact(r):
    cfg, ci = r.cfg, r.cfg.index
    P, d, nt = cfg.tile, cfg.head_dim, cfg.n_tiles
    for b in range(cfg.batch):
        for h in r.heads(HEAD_LIMIT[ci]):
            qt, kt, vt, perm = r.oracle_head(b, h)
            assert bitwise_equal(host(r.sa.q_t[b, h]), qt), (cfg.name, h, "q")
            assert bitwise_equal(host(r.sa.k_t[b, h]), kt), (cfg.name, h, "k")
            assert bitwise_equal(host(r.sa.v_t[b, h]), vt), (cfg.name, h, "v")
            vcols = host(r.v_cols()[b, h]).reshape(nt, d, P).transpose(0, 2, 1)      # [tile][pos][c]
            vkeys = vt.reshape(nt, P, d)[:, COLS_KEY[:P], :]                          # same order
            assert bitwise_equal(vcols, vkeys), (cfg.name, h, "v channel-major")
    # scatter(gather(q)) is the identity
    back = torch.empty_like(r.q)
    V.veda_tile_gather(r.geom, back, r.sa.q_t, V.ROWS, inverse=True)
    torch.cuda.synchronize()
    assert torch.equal(back.view(torch.int16) if r.bf16 else back, r.q.view(torch.int16) if r.bf16 else r.q)


# ----------------------------------------------------------------------------- scoring
def test_trippool_descriptors(r):
    cfg, ci = r.cfg, r.cfg.index
    d = cfg.head_dim
    for b in range(cfg.batch):
        for h in r.heads(HEAD_LIMIT[ci]):
            qt, kt, _, _ = r.oracle_head(b, h)
            for x, gd in ((qt, r.qd), (kt, r.kd)):
                ref = O.trippool(x, cfg.tile)
                got = host(gd[b, h])
                assert bitwise_equal(got[:, d:], ref[:, d:]), (cfg.name, h)      # max, min exact
                err = np.abs(got[:, :d] - ref[:, :d]) / np.maximum(np.abs(ref[:, :d]), 1.0)
                assert err.max() <= 1e-6, (cfg.name, h, err.max())


def test_scores_and_topk(r):
    cfg, ci = r.cfg, r.cfg.index
    kk = r.kk
    worst, exempt, rows = 0.0, 0, 0
    for b in range(cfg.batch):
        for h in r.heads(SCORE_HEADS[ci]):
            qt, kt, _, _ = r.oracle_head(b, h)
            yq = O.mlp(O.trippool(qt, cfg.tile), r.wl.w1[h], r.wl.w2[h])
            yk = O.mlp(O.trippool(kt, cfg.tile), r.wl.w1[h], r.wl.w2[h])
            s = O.tile_scores(yq, yk, cfg.score_scale)
            s32 = s.astype(np.float32)
            got_s = host(r.scores[b, h])
            worst = max(worst, float(np.abs(got_s - s).max()))
            got_p = host(r.probs[b, h])
            assert np.abs(got_p - O.row_softmax(s)).max() <= 2e-6, (cfg.name, h)
            idx = host(r.idx[b, h]).astype(np.int64)
            for i in range(cfg.n_tiles):
                ok, ex = O.topk_agrees(s32[i], idx[i], kk)
                assert ok, (cfg.name, h, i, idx[i], np.sort(s32[i])[::-1][kk - 2:kk + 2])
                exempt += ex
                rows += 1
    measure(f"[gpu-parity] {cfg.name}: score max|err| {worst:.3g} over {rows} rows of "
            f"{len(r.heads(SCORE_HEADS[ci]))} heads, {exempt} rows in the near-tie band")
    # fp32 MLP and score products against float64: about 1e-6 of the logit (|S| <= 16 here,
    # 14 fp32 ulps); measured 1.6e-6 (tiny) to 9.3e-6 (long) over every row of every head
    assert worst <= SCORE_TOL


SCORE_TOL = 1.25e-5   # absolute, on the fp32 logits


# ----------------------------------------------------------------------------- attention
def attention_errors(r, idx_dev, kk, heads, tiles_per_head=None, o_t=None, lse=None):
    cfg = r.cfg
    P = cfg.tile
    o_t = r.sa.o_t if o_t is None else o_t
    num = den = 0.0
    mx = lse_err = 0.0
    for b in range(cfg.batch):
        for h in heads:
            qt, kt, vt, _ = r.oracle_head(b, h)
            tiles = r.q_tiles(h)
            if tiles_per_head is not None:
                tiles = tiles[np.linspace(0, len(tiles) - 1, tiles_per_head).astype(int)]
            idx = host(idx_dev[b, h]).astype(np.int64)
            ref, ref_lse = O.sparse_attention(qt, kt, vt, idx, P, 1 / math.sqrt(cfg.head_dim), q_tiles=tiles,
                                              return_lse=True)
            rows = (tiles[:, None] * P + np.arange(P)[None]).ravel()
            got = host(o_t[b, h])[rows]
            num += float(((got - ref) ** 2).sum())
            den += float((ref ** 2).sum())
            mx = max(mx, float(np.abs(got - ref).max()))
            if lse is not None:
                lse_err = max(lse_err, float(np.abs(host(lse[b, h])[rows] - ref_lse).max()))
    return mx, math.sqrt(num / den), lse_err


def tol(r):
    return (2e-2, 1e-2) if r.bf16 else (1e-4, 1e-4)


def test_sparse_attention(r):
    heads = r.heads()
    mx, rel, lse_err = attention_errors(r, r.idx, r.kk, heads, lse=r.lse)
    measure(f"[gpu-parity] {r.cfg.name} k={r.kk}: {len(heads)} heads x {len(r.q_tiles(0))} query tiles: "
            f"max|dO| {mx:.3g}  relFro {rel:.3g}  max|dLSE| {lse_err:.3g}")
    amax, arel = tol(r)
    assert mx <= amax and rel <= arel
    # bf16: the kernel's normaliser sums the probabilities after rounding them to bf16 (the
    # values that multiply V).  Round-to-nearest-even changes each by at most the bf16 unit
    # roundoff 2^-8 = 3.9e-3 relative, so the sum, and with it exp(LSE), by at most that
    # much when every kept probability rounds the same way (a near one-hot row whose
    # dominant probability sits just above a power of two).  The fp32 accumulation adds
    # far less.  Gate: 4e-3 on the natural-log LSE.
    assert lse_err <= (4e-3 if r.bf16 else 1e-5)


def test_output_unpermuted(r):
    """The raster output is the tiled output scattered back through the permutation."""
    cfg, ci = r.cfg, r.cfg.index
    for b in range(cfg.batch):
        for h in r.heads(HEAD_LIMIT[ci]):
            _, _, _, perm = r.oracle_head(b, h)
            assert bitwise_equal(host(r.out[b, :, h])[perm], host(r.sa.o_t[b, h])), (cfg.name, h)


def test_dense_path(r):
    """k = n_t with every tile listed: equals full attention (with the key-tile bounds, as
    the benchmark's dense path runs)."""
    cfg, ci = r.cfg, r.cfg.index
    idx = dense_index(r.geom)
    o_t = torch.empty_like(r.sa.o_t)
    say(f"[gpu-parity] {cfg.name}: dense path k={cfg.n_tiles}")
    V.veda_sparse_attn_fwd(r.geom, r.sa.q_t, r.sa.k_t, r.sa.v_t, idx, cfg.n_tiles, 1 / math.sqrt(cfg.head_dim), o_t,
                           k_bound=r.sa.k_bound)
    torch.cuda.synchronize()
    heads = r.heads({0: None, 1: None, 2: 4, 3: 4, 4: 4}[ci])
    tph = {0: None, 1: None, 2: 8, 3: 8, 4: 4}[ci]
    mx, rel, _ = attention_errors(r, idx, cfg.n_tiles, heads, tiles_per_head=tph, o_t=o_t)
    measure(f"[gpu-parity] {cfg.name} dense (k = {cfg.n_tiles}): {len(heads)} heads x {tph or 'all'} query tiles: "
            f"max|dO| {mx:.3g}  relFro {rel:.3g}")
    amax, arel = tol(r)
    assert mx <= amax and rel <= arel


def test_sparsity_sweep(r):
    cfg = r.cfg
    if len(cfg.topk) < 3:
        pytest.skip("no sparsity sweep for this workload")
    # the selections themselves, on four heads: every row against the oracle's fp32 scores
    # (k up to 240 exercises the compacted search over up to 512 candidates on long rows)
    sel_heads = [int(h) for h in r.heads(4)]
    s32 = {}
    for h in sel_heads:
        qt, kt, _, _ = r.oracle_head(0, h)
        s32[h] = O.tile_scores(O.mlp(O.trippool(qt, cfg.tile), r.wl.w1[h], r.wl.w2[h]),
                               O.mlp(O.trippool(kt, cfg.tile), r.wl.w1[h], r.wl.w2[h]),
                               cfg.score_scale).astype(np.float32)
    for kk in cfg.topk[1:-1]:
        idx = r.sa.score(kk)
        for h in sel_heads:
            got = host(idx[0, h]).astype(np.int64)
            for i in range(cfg.n_tiles):
                assert O.topk_agrees(s32[h][i], got[i], kk)[0], (cfg.name, kk, h, i)
        o_t = torch.empty_like(r.sa.o_t)
        say(f"[gpu-parity] {cfg.name}: k={kk}")
        # no key-tile bounds: the sweep checks the running-maximum softmax at every k
        V.veda_sparse_attn_fwd(r.geom, r.sa.q_t, r.sa.k_t, r.sa.v_t, idx, kk, 1 / math.sqrt(cfg.head_dim), o_t)
        torch.cuda.synchronize()
        heads = r.heads(8)
        mx, rel, _ = attention_errors(r, idx, kk, heads, tiles_per_head=16, o_t=o_t)
        measure(f"[gpu-parity] {cfg.name} k={kk}: {len(heads)} heads x 16 query tiles: max|dO| {mx:.3g}  "
                f"relFro {rel:.3g}")
        assert mx <= 2e-2 and rel <= 1e-2


# Rows longer than 256 tiles pick the top-k compaction width from k (2 or 6 up to 768 tiles,
# 4 or 8 beyond); these k straddle each switch.
WIDTH_KS = {"large": (100, 101, 300), "long": (160, 161)}


def test_topk_compaction_widths(r):
    cfg = r.cfg
    if cfg.name not in WIDTH_KS:
        pytest.skip("rows of at most 256 tiles use one width")
    h = int(r.heads(1)[0])
    qt, kt, _, _ = r.oracle_head(0, h)
    s32 = O.tile_scores(O.mlp(O.trippool(qt, cfg.tile), r.wl.w1[h], r.wl.w2[h]),
                        O.mlp(O.trippool(kt, cfg.tile), r.wl.w1[h], r.wl.w2[h]), cfg.score_scale).astype(np.float32)
    for kk in WIDTH_KS[cfg.name]:
        say(f"[gpu-parity] {cfg.name}: top-k widths, k={kk}")
        got = host(r.sa.score(kk)[0, h]).astype(np.int64)
        for i in range(cfg.n_tiles):
            assert O.topk_agrees(s32[i], got[i], kk)[0], (cfg.name, kk, h, i)


# ----------------------------------------------------------------------------- tile map
# Map rows compared with the oracle: every head on `each` query tiles (seeded choice among the
# head's selected tiles), and every selected tile on the first `full` heads.
MAP_CHECK = {0: (None, 1), 1: (None, 12), 2: (16, 1), 3: (8, 2), 4: (8, 2)}
# |log M_gpu - log M_oracle| on entries >= 1e-30, bf16 inputs / fp32 inputs: both sides use
# the same rounded inputs, so only the fp32 accumulation of the logits and of the row
# log-sum-exp differs (measured <= 2.5e-5 at N = 153 600, 1.8e-6 for the fp32 workload)
MAP_LOG_TOL = {True: 1e-4, False: 1e-5}


def map_rows(cfg, h, n_sel):
    each, full = MAP_CHECK[cfg.index]
    if each is None or h < full or each >= n_sel:
        return np.arange(n_sel)
    return np.sort(np.random.default_rng(cfg.seed + 3000 + h).choice(n_sel, each, replace=False))


def test_tilemap_and_recall(r):
    cfg, ci = r.cfg, r.cfg.index
    B, H, nt, P = cfg.batch, cfg.heads, cfg.n_tiles, cfg.tile
    n_sel = cfg.sampled_q_tiles or nt
    qtl = torch.from_numpy(np.stack([r.q_tiles(h) for h in range(H)]).astype(np.int32)[None].repeat(B, 0)).cuda()
    tm = torch.empty((B, H, n_sel, nt), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H, n_sel * P), dtype=torch.float32, device="cuda")
    say(f"[gpu-parity] {cfg.name}: tile map, {n_sel} query tiles per head")
    r.sa.tilemap(qtl, n_sel, tm, lse)
    torch.cuda.synchronize()
    # oracle mask = top-k of the map: the library's top-k of the library's map
    omask = torch.empty((B, H, n_sel, r.kk), dtype=torch.int32, device="cuda")
    V.veda_topk_mask(tm, r.kk, omask)
    torch.cuda.synchronize()
    tmh, omh = host(tm), host(omask).astype(np.int64)
    tol_log = MAP_LOG_TOL[r.bf16]
    worst, n_rows, n_band = 0.0, 0, 0
    for b in range(B):
        for h in range(H):
            qt, kt, _, _ = r.oracle_head(b, h)
            sel = map_rows(cfg, h, n_sel)
            ref = O.tilemap(qt, kt, P, 1 / math.sqrt(cfg.head_dim), q_tiles=r.q_tiles(h)[sel])
            got = tmh[b, h, sel]
            keep = ref >= 1e-30
            assert np.all(got[~keep] < 1e-25), (cfg.name, h)
            worst = max(worst, float(np.abs(np.log(got[keep]) - np.log(ref[keep])).max()))
            assert np.all(got <= 1.0 + 1e-6)
            # the oracle mask against the oracle's own top-k of the oracle's map: entries of the
            # two maps agree to tol_log in log space, so two entries closer than 2 tol_log may
            # trade places (near-tie band, taken on log M)
            lref = np.log(np.maximum(ref, 1e-300))
            for a, row in enumerate(sel):
                ok, ex = O.topk_agrees(lref[a], omh[b, h, row], r.kk, gap=2 * tol_log)
                assert ok, (cfg.name, h, int(row), omh[b, h, row], O.topk_rows(lref[a][None], r.kk)[0])
                n_band += ex
            n_rows += len(sel)
        # every row: the library's top-k picks the k largest of the library's map
        for h in range(H):
            for a in range(n_sel):
                ok, _ = O.topk_agrees(tmh[b, h, a].astype(np.float64), omh[b, h, a], r.kk, gap=1e-12)
                assert ok
    est = host(r.idx).astype(np.int64)
    recall = np.mean([O.recall(est[b, h][r.q_tiles(h)], omh[b, h]) for b in range(B) for h in range(H)])
    measure(f"[gpu-parity] {cfg.name}: tile map {n_rows} rows of {B * H} heads vs oracle: max|dlog M| {worst:.3g}; "
            f"oracle mask equal to the oracle's top-k ({n_band} rows in the near-tie band); "
            f"estimator recall vs oracle mask {recall:.3f}")
    assert worst <= tol_log


# ----------------------------------------------------------------------------- determinism, edges
def test_determinism(r):
    if r.cfg.index not in (1, 2, 3):
        pytest.skip("checked on the small, mid and large workloads")
    o1 = r.sa.o_t.clone()
    i1 = r.idx.clone()
    idx = r.sa.score(r.kk)
    r.sa.attend(idx)
    torch.cuda.synchronize()
    assert torch.equal(idx, i1)
    assert torch.equal(r.sa.o_t.view(torch.int16), o1.view(torch.int16))


def small_geom_case(batch, grid, shapes, seed=7):
    rng = np.random.default_rng(seed)
    H = len(shapes)
    N = grid[0] * grid[1] * grid[2]
    geom = V.Geom(batch, H, 128, grid, 128, shapes)
    x = [torch.from_numpy(rng.standard_normal((batch, N, H, 128)).astype(np.float32)).to(torch.bfloat16).cuda()
         for _ in range(3)]
    return geom, x


def test_batch_and_edge_k():
    """batch > 1, k = 1 and k = n_t, on a 4x8x16 grid with three tile shapes, against the
    oracle; and the default raster path against the tiled one on the same batches."""
    shapes = [(1, 8, 16), (2, 8, 8), (4, 4, 8)]
    geom, (q, k, v) = small_geom_case(2, (4, 8, 16), shapes)
    rng = np.random.default_rng(3)
    w1 = torch.from_numpy((rng.standard_normal((3, 384, 256)) / math.sqrt(384)).astype(np.float32))
    w2 = torch.from_numpy((rng.standard_normal((3, 256, 64)) / 16).astype(np.float32))
    sa = SparseAttention(geom, torch.bfloat16, w1, w2)
    say("[gpu-parity] batch-2 edge case")
    sa.gather(q, k, v)
    nt = geom.n_tiles
    for kk in (1, 2, nt):
        idx = sa.score(kk)
        sa.attend(idx)
        torch.cuda.synchronize()
        idx_h = host(idx).astype(np.int64)
        for b in range(2):
            for h in range(3):
                perm = O.tile_permutation(geom.grid, shapes[h])
                qt, kt, vt = (O.to_tiles(host(x[b, :, h]), perm) for x in (q, k, v))
                yq = O.mlp(O.trippool(qt, 128), w1[h].numpy(), w2[h].numpy())
                yk = O.mlp(O.trippool(kt, 128), w1[h].numpy(), w2[h].numpy())
                s32 = O.tile_scores(yq, yk, 0.125).astype(np.float32)
                for i in range(nt):
                    assert O.topk_agrees(s32[i], idx_h[b, h, i], kk)[0]
                ref = O.sparse_attention(qt, kt, vt, idx_h[b, h], 128, 1 / math.sqrt(128))
                got = host(sa.o_t[b, h])
                assert np.abs(got - ref).max() <= 2e-2
                assert math.sqrt(((got - ref) ** 2).sum() / (ref ** 2).sum()) <= 1e-2
        # the default raster path (K and V tiled by the scoring launch) on two batches: the
        # same lists and, bit for bit, the same output as the tiled path just checked
        out_t, out_r = torch.empty_like(q), torch.empty_like(q)
        sa.scatter(out_t)
        idx_t = idx.clone()
        sa.forward_raster(q, k, v, kk, out_r)
        torch.cuda.synchronize()
        assert torch.equal(sa.idx_buffer(kk), idx_t), kk
        assert torch.equal(out_r.view(torch.int16), out_t.view(torch.int16)), kk


def test_strided_raster_gather():
    """A non-contiguous [B,N,H,d] view (head-major storage) gathers like a contiguous one."""
    shapes = [(2, 8, 8), (1, 8, 16)]
    geom, (q, _, _) = small_geom_case(1, (4, 8, 16), shapes)
    hm = q.permute(0, 2, 1, 3).contiguous()        # [B,H,N,d] storage
    view = hm.permute(0, 2, 1, 3)                  # [B,N,H,d] view with strides (HNd, d, Nd, 1)
    a = torch.empty((1, 2, 512, 128), dtype=torch.bfloat16, device="cuda")
    bb = torch.empty_like(a)
    V.veda_tile_gather(geom, q, a, V.ROWS)
    V.veda_tile_gather(geom, view, bb, V.ROWS)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), bb.view(torch.int16))


@pytest.mark.parametrize("n_cols,k", [(1, 1), (7, 3), (64, 64), (600, 60), (1200, 120), (1300, 5), (4096, 409)])
def test_topk_mask_standalone(n_cols, k):
    rng = np.random.default_rng(n_cols)
    rows = 37
    s = (np.round(rng.standard_normal((rows, n_cols)) * 4) / 4).astype(np.float32)   # many exact ties
    s[0] = 1.5                                                                       # an all-equal row
    sd = torch.from_numpy(s).cuda()
    idx = torch.empty((rows, k), dtype=torch.int32, device="cuda")
    mask = torch.empty((rows, n_cols), dtype=torch.uint8, device="cuda")
    say(f"[gpu-parity] topk n_cols={n_cols} k={k}")
    V.veda_topk_mask(sd, k, idx, mask)
    torch.cuda.synchronize()
    ref = O.topk_rows(s.astype(np.float64), k)
    assert np.array_equal(host(idx).astype(np.int64), ref)
    m = np.zeros((rows, n_cols), np.uint8)
    np.put_along_axis(m, ref, 1, axis=1)
    assert np.array_equal(host(mask), m)


# ----------------------------------------------------------------------------- V layouts
def same_bits(a, b):
    view = torch.int16 if a.dtype == torch.bfloat16 else torch.int32
    return a.dtype == b.dtype and torch.equal(a.view(view), b.view(view))


def test_v_layouts_match(r):
    """Attention with V channel-major (COLS: one 16-byte LDS read per operand) or raster
    (transposed LDS reads, as for the tile-major V of the tests above) gives bit for bit the
    output and LSE of the tile-major V, which the tests above check against the oracle: the
    same products meet the same MFMA slots in the same order.  Tiled call with a COLS V;
    raster call with K tiled or raster and V COLS or raster."""
    cfg, sa = r.cfg, r.sa
    say(f"[gpu-parity] {cfg.name}: V layouts")
    v_cols = r.v_cols()
    o_t = torch.empty_like(sa.o_t)
    lse = torch.empty_like(r.lse)
    V.veda_sparse_attn_fwd(r.geom, sa.q_t, sa.k_t, v_cols, r.idx, r.kk, sa.softmax_scale, o_t, lse, v_layout=V.COLS,
                           k_bound=sa.k_bound)
    torch.cuda.synchronize()
    assert same_bits(o_t, sa.o_t) and same_bits(lse, r.lse), cfg.name
    del o_t
    for k_layout, kop in ((V.ROWS, sa.k_t), (V.RASTER, r.k)):
        for v_layout, vop in ((V.COLS, v_cols), (V.RASTER, r.v)):
            out = torch.zeros_like(r.out)
            V.veda_sparse_attn_fwd_raster(r.geom, r.q, kop, vop, r.idx, r.kk, sa.softmax_scale, out,
                                          k_layout=k_layout, v_layout=v_layout, k_bound=sa.k_bound)
            torch.cuda.synchronize()
            assert same_bits(out, r.out), (cfg.name, k_layout, v_layout)


# ----------------------------------------------------------------------------- raster path
@pytest.mark.parametrize("k_raster", [False, True], ids=["k_tiled", "k_raster"])
def test_raster_path_matches_tiled(r, k_raster):
    """The raster-direct calls (Q and O raster; K raster or tiled) give bit-identical
    results to the tiled calls, which the tests above check against the oracle."""
    cfg, sa = r.cfg, r.sa
    B, H, N, nt = cfg.batch, cfg.heads, cfg.n_tokens, cfg.n_tiles
    say(f"[gpu-parity] {cfg.name}: raster-direct path, K {'raster' if k_raster else 'tiled'}")
    kk_ = r.k if k_raster else None
    scores, probs = torch.empty_like(r.scores), torch.empty_like(r.probs)
    qd, kd = torch.empty_like(r.qd), torch.empty_like(r.kd)
    idx = sa.score_raster(r.q, r.kk, k=kk_, scores=scores, probs=probs, q_desc=qd, k_desc=kd).clone()
    assert torch.equal(qd, r.qd) and torch.equal(kd, r.kd)
    assert torch.equal(scores, r.scores) and torch.equal(probs, r.probs)
    assert torch.equal(idx, r.idx)
    out = torch.zeros_like(r.out)
    lse = torch.empty_like(r.lse)
    sa.attend_raster(r.q, idx, out, lse, k=kk_)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16) if out.dtype == torch.bfloat16 else out,
                       r.out.view(torch.int16) if r.out.dtype == torch.bfloat16 else r.out)
    lse_t, lse_r = r.lse.cpu().numpy(), lse.cpu().numpy()
    for b in range(B):
        for h in range(H):
            perm = O.tile_permutation(cfg.grid, r.wl.shapes[h])
            assert bitwise_equal(lse_r[b, h, perm], lse_t[b, h])
    n_sel = min(8, nt)
    qtl = torch.from_numpy(np.stack([r.q_tiles(h)[:n_sel] for h in range(H)]).astype(np.int32)[None]
                           .repeat(B, 0)).cuda().contiguous()
    m_t = torch.empty((B, H, n_sel, nt), dtype=torch.float32, device="cuda")
    m_r = torch.empty_like(m_t)
    l_t = torch.empty((B, H, n_sel * cfg.tile), dtype=torch.float32, device="cuda")
    l_r = torch.empty_like(l_t)
    sa.tilemap(qtl, n_sel, m_t, l_t)
    sa.tilemap_raster(r.q, qtl, n_sel, m_r, l_r, k=kk_)
    torch.cuda.synchronize()
    assert torch.equal(m_t, m_r) and torch.equal(l_t, l_r)
    if k_raster:
        # the scoring pass that also writes K's tile-major copy: the copy equals the gather's,
        # and the selections are unchanged
        k_copy = torch.full_like(sa.k_t, float("nan"))
        v_copy = torch.full_like(sa.v_t, float("nan"))
        idx2 = torch.full_like(idx, -1)
        kb = torch.full_like(sa.k_bound, float("nan"))
        V.veda_trippool_score_raster(r.geom, r.q, r.k, sa.w1, sa.w2, score_scale=cfg.score_scale, topk=r.kk,
                                     idx=idx2, workspace=sa.ws, k_layout=V.RASTER, k_tiled_out=k_copy,
                                     v=r.v, v_tiled_out=v_copy, k_bound=kb)
        torch.cuda.synchronize()
        assert torch.equal(idx2, r.idx)
        assert same_bits(k_copy, sa.k_t) and same_bits(v_copy, sa.v_t) and same_bits(kb, sa.k_bound)
    else:
        # V's copy from the scoring launch with a tiled K as well
        v_copy = torch.full_like(sa.v_t, float("nan"))
        idx2 = torch.full_like(idx, -1)
        V.veda_trippool_score_raster(r.geom, r.q, sa.k_t, sa.w1, sa.w2, score_scale=cfg.score_scale, topk=r.kk,
                                     idx=idx2, workspace=sa.ws, k_layout=V.ROWS, v=r.v, v_tiled_out=v_copy)
        torch.cuda.synchronize()
        assert torch.equal(idx2, r.idx) and same_bits(v_copy, sa.v_t)


# ----------------------------------------------------------------------------- softmax offset
def test_key_tile_bounds_and_offset_paths(r):
    """The scoring call's per-key-tile bound (from the oracle's max and min descriptors:
    sqrt(sum_c max(max_c^2, min_c^2)), which bounds every key-row norm of the tile), and
    attention with and without it.  Both start each row's exponent offset at its first kept
    tile's row max; without bounds the kernel takes every later tile's row max and moves the
    offset when one exceeds it by more than 2^8, with bounds it keeps the offset fixed (the
    bound proving that no later exponential exceeds 2^64).  The fixed offset is checked
    against the oracle by test_sparse_attention, the running one here on sampled heads; the
    two agree bit for bit on every row whose offset the running maximum never moves.  A
    bound 2^40 too large sends every wave back to the running maximum, which must then give
    exactly the output and LSE of the call without bounds."""
    cfg, sa = r.cfg, r.sa
    d, P = cfg.head_dim, cfg.tile
    say(f"[gpu-parity] {cfg.name}: key-tile bounds and softmax offsets")
    kb = host(sa.k_bound)
    worst = 0.0
    for b in range(cfg.batch):
        for h in r.heads(8):
            _, kt, _, _ = r.oracle_head(b, h)
            desc = O.trippool(kt, P)
            ref = np.sqrt((np.maximum(np.abs(desc[:, d:2 * d]), np.abs(desc[:, 2 * d:])) ** 2).sum(1))
            worst = max(worst, float(np.abs(kb[b, h] / ref - 1).max()))
            rown = np.linalg.norm(kt.reshape(-1, P, d), axis=2).max(1)
            assert np.all(kb[b, h] >= rown * (1 - 1e-6)), (cfg.name, h)
    measure(f"[gpu-parity] {cfg.name}: key-tile bounds max rel err {worst:.3g}")
    assert worst <= 1e-5            # fp32 sum of 128 squares of exactly represented values
    if not r.bf16:
        return                      # the fp32 kernel keeps a running maximum throughout
    o_run, l_run = torch.empty_like(sa.o_t), torch.empty_like(r.lse)
    V.veda_sparse_attn_fwd(r.geom, sa.q_t, sa.k_t, sa.v_t, r.idx, r.kk, sa.softmax_scale, o_run, l_run)
    o_far, l_far = torch.empty_like(sa.o_t), torch.empty_like(r.lse)
    V.veda_sparse_attn_fwd(r.geom, sa.q_t, sa.k_t, sa.v_t, r.idx, r.kk, sa.softmax_scale, o_far, l_far,
                           k_bound=sa.k_bound * 2.0 ** 40)
    torch.cuda.synchronize()
    assert same_bits(o_far, o_run) and same_bits(l_far, l_run), cfg.name
    heads = r.heads(8)
    mx, rel, lse_err = attention_errors(r, r.idx, r.kk, heads, tiles_per_head=16, o_t=o_run, lse=l_run)
    same_rows = float((l_run.view(torch.int32) == r.lse.view(torch.int32)).float().mean())
    measure(f"[gpu-parity] {cfg.name}: running-maximum softmax, {len(heads)} heads x 16 query tiles: "
            f"max|dO| {mx:.3g} relFro {rel:.3g} max|dLSE| {lse_err:.3g}; rows bit-identical to the fixed offset "
            f"{same_rows:.4f}")
    amax, arel = tol(r)
    assert mx <= amax and rel <= arel and lse_err <= 4e-3


@pytest.mark.parametrize("case", ["fixed", "fallback"])
def test_offset_with_growing_logits(case):
    """Queries near one direction u and keys of time slice t along u with weight a_t growing
    along the kept list, so that later tiles' row maxima exceed the first tile's by more than
    2^8 (the running offset rescales) while the key-tile bounds stay close to the true key
    norms.  "fixed": the largest bound lies within 2^64 of every row's first-tile max, the
    fixed offset is kept and exponentials reach about 2^18 (the outputs differ from the
    running offset's in rounding); "fallback": the last slice's weight puts the bound beyond
    2^64 and every wave takes the running offset, bit for bit.  Both against the oracle, on
    a 4x8x16 grid with two tile shapes (the second puts two time slices in each tile)."""
    shapes = [(1, 8, 16), (2, 8, 8)]
    grid = (4, 8, 16)
    a = {"fixed": (2.0, 8.0, 14.0, 20.0), "fallback": (2.0, 8.0, 14.0, 200.0)}[case]
    rng = np.random.default_rng(11)
    H, N, d, P = 2, 512, 128, 128
    geom = V.Geom(1, H, d, grid, P, shapes)
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    t_of = np.repeat(np.arange(grid[0]), grid[1] * grid[2])            # raster token -> t
    qn = 8.0 * u + 0.3 * rng.standard_normal((1, N, H, d))
    kn = np.asarray(a)[t_of][None, :, None, None] * u + 0.3 * rng.standard_normal((1, N, H, d))
    vn = rng.standard_normal((1, N, H, d))
    up = lambda x: torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).cuda()
    q, k, v = up(qn), up(kn), up(vn)
    w1 = torch.from_numpy((rng.standard_normal((H, 3 * d, 256)) / math.sqrt(3 * d)).astype(np.float32))
    w2 = torch.from_numpy((rng.standard_normal((H, 256, 64)) / 16).astype(np.float32))
    sa = SparseAttention(geom, torch.bfloat16, w1, w2)
    say(f"[gpu-parity] growing logits, {case}")
    sa.gather(q, k, v)
    sa.score(2)                                   # writes the key-tile bounds of this K
    nt = geom.n_tiles
    idx = dense_index(geom)                       # every tile, ascending: logits grow along the list
    o_fix, o_run = torch.empty_like(sa.o_t), torch.empty_like(sa.o_t)
    l_fix = torch.empty((1, H, N), dtype=torch.float32, device="cuda")
    l_run = torch.empty_like(l_fix)
    V.veda_sparse_attn_fwd(geom, sa.q_t, sa.k_t, sa.v_t, idx, nt, sa.softmax_scale, o_fix, l_fix, k_bound=sa.k_bound)
    V.veda_sparse_attn_fwd(geom, sa.q_t, sa.k_t, sa.v_t, idx, nt, sa.softmax_scale, o_run, l_run)
    torch.cuda.synchronize()
    assert torch.isfinite(o_fix.float()).all() and torch.isfinite(l_fix).all()
    same = same_bits(o_fix, o_run) and same_bits(l_fix, l_run)
    assert same == (case == "fallback"), case
    worst = lse_worst = 0.0
    for h in range(H):
        perm = O.tile_permutation(grid, shapes[h])
        qt, kt, vt = (O.to_tiles(host(x[0, :, h]), perm) for x in (q, k, v))
        ref, ref_lse = O.sparse_attention(qt, kt, vt, host(idx[0, h]).astype(np.int64), P, 1 / math.sqrt(d),
                                          return_lse=True)
        for o, l in ((o_fix, l_fix), (o_run, l_run)):
            got = host(o[0, h])
            worst = max(worst, float(np.abs(got - ref).max()))
            assert math.sqrt(((got - ref) ** 2).sum() / (ref ** 2).sum()) <= 1e-2, (case, h)
            lse_worst = max(lse_worst, float(np.abs(host(l[0, h]) - ref_lse).max()))
    measure(f"[gpu-parity] growing logits ({case}): max|dO| {worst:.3g}, max|dLSE| {lse_worst:.3g}, "
            f"fixed offset bit-identical to running: {same}")
    assert worst <= 2e-2 and lse_worst <= 4e-3
