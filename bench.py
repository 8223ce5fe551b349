#!/usr/bin/env python3
"""Benchmark of the distilled sparse attention hot path on one MI355X.

One step = every stage of the path over one batch of the seeded synthetic workload
(default: the 14B-DiT-scale "large" workload, B=1, H=40, d=128, latent 20x48x80 so
N = 76 800 tokens, 128-token tiles with per-head shapes, 60 of 600 key tiles kept = 90 %
skipped).  The default (raster) path:
  1. TripPool -> per-head MLP -> tile scores -> top-k (one call, fused top-k) on raster Q and
     K; the same launch writes K's tile-major copy as it pools K, and streams raster V into
     its tile-major copy (the head-aware tile gather of K and V, fused)
  2. tile-skipping attention (bf16 MFMA) on the tiled K and V, Q read and O written in
     raster order
  3. max-pooled full-attention tile map on the 64 sampled query tiles per head
(--path tiled: gather Q, K, V; scoring; attention; inverse gather of O; tile map.)
Inputs are resident in HBM before the timed region.  Prints one JSON line.

value = kept attention FLOPs per step (4 N^2 d (k/n_t) H B) / step time, in TFLOP/s.
Per-stage times come from HIP events recorded on the launch stream inside the timed
steps; `roofline` is the attention kernel (the dominant one) against bf16 MFMA peak.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-attn ms/call + effective TFLOPS (kept FLOPs) at 90% sparsity, N≈77k"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
COUNTERS = os.path.join(ROOT, "profiles", "counters_attn_bf16_large.txt")
ATTN_SRC = os.path.join(ROOT, "video_dit_block_head_amd", "csrc", "attn.hip")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def traffic_from_counters(path):
    """HBM bytes per attention launch from committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    counts, scaled by the same counters' reading of a plain copy of known size.  None if
    the attention source changed since the counters were taken, or they were taken on the
    other path."""
    if not os.path.exists(COUNTERS):
        return None
    rec = json.load(open(COUNTERS))
    sha = hashlib.sha256(open(ATTN_SRC, "rb").read()).hexdigest()
    if rec.get("attn_source_sha256") != sha or rec.get("path", "tiled") != path:
        return None
    return rec.get("traffic_bytes_per_launch")


def cpu_baseline(cfg, wl, kk, n_sel, budget_s=15.0):
    """Time the CPU oracle (as it stands) on a bounded sample of one step and scale each
    stage to the full step.  Per sampled head: gather / scoring / scatter of all tiles,
    attention for 64 query tiles, the tile map for 4 query tiles.  Heads are taken in
    order until about `budget_s` seconds of CPU work have been measured."""
    import numpy as np
    import oracle.veda_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = None
    P, nt, H = cfg.tile, cfg.n_tiles, cfg.heads
    n_att, n_map = min(64, nt), min(4, n_sel)
    T = time.perf_counter
    acc = dict(gather=0.0, score=0.0, attn=0.0, scatter=0.0, tilemap=0.0)
    t_all = T()
    done = 0
    for h in range(H):   # consecutive heads cycle through the tile shapes
        t = T()
        perm = O.tile_permutation(cfg.grid, wl.shapes[h])
        qt, kt, vt = (O.to_tiles(wl.head(w, 0, h), perm) for w in ("q", "k", "v"))
        acc["gather"] += T() - t
        t = T()
        yq = O.mlp(O.trippool(qt, P), wl.w1[h], wl.w2[h])
        yk = O.mlp(O.trippool(kt, P), wl.w1[h], wl.w2[h])
        idx = O.topk_rows(O.tile_scores(yq, yk, cfg.score_scale).astype(np.float32), kk)
        acc["score"] += T() - t
        t = T()
        out = O.sparse_attention(qt, kt, vt, idx, P, 1 / math.sqrt(cfg.head_dim), q_tiles=np.arange(n_att))
        acc["attn"] += T() - t
        t = T()
        O.from_tiles(qt, perm)
        acc["scatter"] += T() - t
        t = T()
        O.tilemap(qt, kt, P, 1 / math.sqrt(cfg.head_dim), q_tiles=wl.sample_tiles(h)[:n_map])
        acc["tilemap"] += T() - t
        del out
        done += 1
        if T() - t_all >= budget_s:
            break
    wall = T() - t_all
    nh = done
    scale = dict(gather=H / nh, score=H / nh, attn=H * nt / (nh * n_att), scatter=H / nh,
                 tilemap=H * n_sel / (nh * n_map))
    step_s = sum(acc[s] * scale[s] for s in acc)
    return {
        "value": cfg.kept_flops(kk) / step_s / 1e12, "unit": "TFLOP/s",
        "cores": threads if threads else len(os.sched_getaffinity(0)), "kind": "oracle",
        "sample": (f"float64 numpy oracle on {nh} of {H} heads: gather/scoring/scatter of all {nt} tiles, "
                   f"attention for {n_att} query tiles per head, tile map for {n_map} query tiles per head; "
                   f"{wall:.1f} s measured, each stage scaled to the full step"),
        "sample_seconds": round(wall, 2), "extrapolated_step_s": round(step_s, 1),
        "stage_seconds_measured": {s: round(x, 2) for s, x in acc.items()},
        "host_cpus": len(os.sched_getaffinity(0)),
    }


def timed(fn, reps):
    """Mean milliseconds of `reps` calls of fn() between HIP events on the current stream
    (after one untimed call)."""
    import torch
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def long_sweep(reps=5, dense_reps=2):
    """The 720P-10 s-shaped workload (B 1, 48 heads, latent 40x48x80 so N = 153 600, 1200
    tiles per head) on the default path: the scoring pass (TripPool -> MLP -> scores ->
    top-k) and the tile-skipping attention at 80, 90 and 95 % of key tiles skipped, and
    this library's own dense path (every tile kept) for the speedups."""
    import numpy as np
    import torch
    import video_dit_block_head_amd as V
    from video_dit_block_head_amd.pipeline import SparseAttention, dense_index
    from workloads import get, make
    cfg = get("long")
    say(f"[bench] long workload: generating (N={cfg.n_tokens}, H={cfg.heads})")
    wl = make(cfg)
    B, H, N, d, P, nt = cfg.batch, cfg.heads, cfg.n_tokens, cfg.head_dim, cfg.tile, cfg.n_tiles
    geom = V.Geom(B, H, d, cfg.grid, P, wl.shapes)
    up = lambda a: torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16).permute(0, 2, 1, 3).contiguous()
    q, k, v = up(wl.q), up(wl.k), up(wl.v)
    del wl
    sa = SparseAttention(geom, torch.bfloat16, torch.from_numpy(make_weights(cfg)[0]),
                         torch.from_numpy(make_weights(cfg)[1]), score_scale=cfg.score_scale)
    out = torch.empty_like(q)
    sa.gather_kv(k, v)
    rows = {}
    say("[bench] long workload: sparsity sweep")
    for kk in sorted(cfg.topk[:-1], reverse=True):          # 240, 120, 60 of 1200
        score_ms = timed(lambda: sa.score_raster(q, kk), reps)
        idx = sa.idx_buffer(kk)
        attn_ms = timed(lambda: sa.attend_raster(q, idx, out), reps)
        fl = cfg.kept_flops(kk)
        sbytes = 2 * B * H * N * d * 2 + B * H * nt * kk * 4
        rows[f"k{kk}"] = {"skipped_pct": round(100 * (1 - kk / nt), 1), "attn_ms": round(attn_ms, 3),
                          "attn_tflops": round(fl / (attn_ms * 1e-3) / 1e12, 1),
                          "attn_frac_bf16_peak": round(fl / (attn_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                          "scoring_ms": round(score_ms, 4),
                          "scoring_frac_hbm_peak": round(sbytes / (score_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)}
    say("[bench] long workload: dense path (k = n_t)")
    didx = dense_index(geom)
    dense_ms = timed(lambda: sa.attend_raster(q, didx, out), dense_reps)
    for r in rows.values():
        r["speedup_vs_dense"] = round(dense_ms / r["attn_ms"], 2)
    res = {"workload": f"long: B={B} H={H} d={d} latent {'x'.join(map(str, cfg.grid))} (N={N}), tile {P}, "
                       f"{nt} tiles per head",
           "sweep": rows,
           "dense": {"ms": round(dense_ms, 2), "tflops": round(cfg.kept_flops(nt) / (dense_ms * 1e-3) / 1e12, 1)}}
    del sa, q, k, v, out, didx
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def make_weights(cfg):
    """The workload's estimator weights (the generator's first draws after the axis scales
    and sinks), without generating Q, K and V again."""
    from workloads import make
    wl = make(cfg, heads=[])
    return wl.w1, wl.w2


def distill_recall(sa, q, k, v, qtl, n_sel, cfg, steps=60, lr=0.1, seed_offset=4000):
    """The estimator before and after `steps` plain SGD steps of the distillation call on the
    sampled query tiles (training rows), on those rows and on as many held-out query tiles
    of every head: tile recall of the kept list against the oracle mask (the k largest
    entries of each max-pooled map row), and the share of each normalised map row (the
    distillation target) that falls outside the kept tiles."""
    import numpy as np
    import torch
    import video_dit_block_head_amd as V
    B, H, nt, kk = cfg.batch, cfg.heads, cfg.n_tiles, cfg.topk[0]
    rng = np.random.default_rng(cfg.seed + seed_offset)
    held = []
    for h in range(H):
        rest = np.setdiff1d(np.arange(nt), qtl[0, h].cpu().numpy())
        held.append(np.sort(rng.choice(rest, n_sel, replace=False)))
    htl = torch.from_numpy(np.stack(held).astype(np.int32)[None].repeat(B, 0)).cuda()
    sa.gather(q, k, v)
    maps = {}
    for tag, tl in (("train", qtl), ("held_out", htl)):
        m = torch.empty((B, H, n_sel, nt), dtype=torch.float32, device="cuda")
        sa.tilemap(tl, n_sel, m)
        o = torch.empty((B, H, n_sel, kk), dtype=torch.int32, device="cuda")
        V.veda_topk_mask(m, kk, o)
        maps[tag] = (tl, m, o)

    def measure(tag):
        tl, m, o = maps[tag]
        est = sa.score(kk).long()
        est = torch.gather(est, 2, tl.long()[..., None].expand(B, H, n_sel, kk)).reshape(-1, kk)
        hit = torch.zeros((est.shape[0], nt), dtype=torch.float32, device="cuda").scatter_(1, est, 1.0)
        rec = float(hit.gather(1, o.reshape(-1, kk).long()).sum()) / (est.shape[0] * kk)
        p = m.reshape(-1, nt) / m.reshape(-1, nt).sum(dim=1, keepdim=True)
        missed = float((p * (1.0 - hit)).sum(dim=1).mean())
        return {"tile_recall": round(rec, 4), "target_mass_outside_kept": round(missed, 5)}

    w1, w2 = sa.w1.clone(), sa.w2.clone()
    before = {t: measure(t) for t in maps}
    losses = []
    for _ in range(steps):
        loss, _, _ = sa.distill_step(qtl, maps["train"][1], lr=lr)
        losses.append(loss)
    after = {t: measure(t) for t in maps}
    sa.w1.copy_(w1)
    sa.w2.copy_(w2)
    return {"sgd_steps": steps, "lr": lr, "loss_first": round(float(losses[0].item()), 4),
            "loss_last": round(float(losses[-1].item()), 4), "before": before, "after": after,
            "chance_recall": round(kk / nt, 4),
            "note": "train: the sampled query tiles the steps fit (their max-pooled maps); held_out: as many other "
                    "query tiles per head, not trained on; the KL fit moves target mass into the kept tiles, "
                    "which is not the same as ranking the oracle's top k"}

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="large", help="tiny|small|mid|large|long")
    ap.add_argument("--topk", type=int, default=None, help="kept key tiles (default: the workload's headline)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true", help="skip the 0%%-skipping attention comparison")
    ap.add_argument("--path", choices=["raster", "tiled"], default="raster",
                    help="raster: the kernels read Q and write O through each head's tiling (K and V are "
                         "gathered); tiled: explicit gather of Q, K, V and scatter of O")
    ap.add_argument("--no-next", action="store_true",
                    help="skip timing the distillation step and the per-head error kernel")
    ap.add_argument("--no-long", action="store_true",
                    help="skip the long (N = 153 600) workload's sparsity sweep")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for HBM counter calibration)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU (got --gpus {args.gpus}, WORLD_SIZE {world}): the path is "
              "independent per head, so more GPUs would each run this same work on their share of the heads",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import video_dit_block_head_amd as V
    from video_dit_block_head_amd.pipeline import SparseAttention, dense_index
    from workloads import get, make, padded_variant

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    V.lib()  # fail loudly if the HIP library is missing
    cfg = get(args.workload)
    kk = args.topk or cfg.topk[0]
    if cfg.dtype != "bf16":
        raise SystemExit("the benchmark runs the bf16 workloads")
    say(f"[bench] generating workload {cfg.name} (N={cfg.n_tokens}, H={cfg.heads}, k={kk}/{cfg.n_tiles})")
    t0 = time.time()
    wl = make(cfg)
    say(f"[bench] generated in {time.time() - t0:.1f} s; uploading")
    B, H, N, d, P, nt = cfg.batch, cfg.heads, cfg.n_tokens, cfg.head_dim, cfg.tile, cfg.n_tiles
    geom = V.Geom(B, H, d, cfg.grid, P, wl.shapes)

    def upload(a):
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16).permute(0, 2, 1, 3).contiguous()

    q, k, v = upload(wl.q), upload(wl.k), upload(wl.v)
    sa = SparseAttention(geom, torch.bfloat16, torch.from_numpy(wl.w1), torch.from_numpy(wl.w2),
                         score_scale=cfg.score_scale)
    out = torch.empty_like(q)
    n_sel = cfg.sampled_q_tiles or nt
    qtl = torch.from_numpy(np.stack([wl.sample_tiles(h) for h in range(H)]).astype(np.int32)[None]
                           .repeat(B, 0)).cuda()
    tmap = torch.empty((B, H, n_sel, nt), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()

    if args.path == "tiled":
        stages = ["gather", "score_topk", "sparse_attn", "scatter", "tilemap"]

        def step(ev):
            ev[0].record()
            sa.gather(q, k, v)
            ev[1].record()
            idx = sa.score(kk)
            ev[2].record()
            sa.attend(idx)
            ev[3].record()
            sa.scatter(out)
            ev[4].record()
            sa.tilemap(qtl, n_sel, tmap)
            ev[5].record()
    else:
        stages = ["score_topk_tile_kv", "sparse_attn", "tilemap"]

        def step(ev):
            ev[0].record()
            idx = sa.score_raster(q, kk, k=k, tile_k=True, v=v)   # also writes K's and V's tiled copies
            ev[1].record()
            sa.attend_raster(q, idx, out)
            ev[2].record()
            sa.tilemap_raster(q, qtl, n_sel, tmap)
            ev[3].record()

    def events():
        return [torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]

    say(f"[bench] warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step(events())
    torch.cuda.synchronize()

    evs = [events() for _ in range(args.steps)]
    say(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_step = wall * 1e3 / args.steps
    per_stage = {s: [] for s in stages}
    for ev in evs:
        for j, s in enumerate(stages):
            per_stage[s].append(ev[j].elapsed_time(ev[j + 1]))
    med = {s: float(np.median(v)) for s, v in per_stage.items()}
    attn_ms = float(np.mean(per_stage["sparse_attn"]))
    kept = cfg.kept_flops(kk)
    attn_tflops = kept / (attn_ms * 1e-3) / 1e12
    # the scoring pass: Q and K read, the kept lists written; on the default path the step's
    # scoring stage also writes K's tile-major copy and reads and writes V's (3 B H N d bf16
    # more) in the same launch
    score_bytes = 2 * B * H * N * d * 2 + B * H * nt * kk * 4
    alone_bytes = score_bytes
    if args.path == "tiled":
        score_ms = float(np.mean(per_stage["score_topk"]))
    else:
        score_ms = float(np.mean(per_stage["score_topk_tile_kv"]))
        score_bytes += 3 * B * H * N * d * 2
    alone_ms = timed(lambda: sa.score_raster(q, kk), 20) if args.path != "tiled" else score_ms
    alone = {"ms": round(alone_ms, 4), "bytes": alone_bytes,
             "frac_hbm_peak": round(alone_bytes / (alone_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
             "note": "the scoring call alone (raster Q, tiled K), 20 calls back to back after the timed steps"}
    say(f"[bench] step {ms_step:.2f} ms; stages (median ms) {json.dumps({s: round(x, 3) for s, x in med.items()})}")

    # tile recall of the last step: the estimator's kept list against the oracle mask (the k
    # largest entries of each sampled row of the max-pooled attention map), averaged over rows
    est = sa.idx_buffer(kk).long()
    est = torch.gather(est, 2, qtl.long()[..., None].expand(B, H, n_sel, kk)).reshape(-1, kk)
    oidx = torch.empty((B, H, n_sel, kk), dtype=torch.int32, device="cuda")
    V.veda_topk_mask(tmap, kk, oidx)
    hit = torch.zeros((est.shape[0], nt), dtype=torch.float32, device="cuda").scatter_(1, est, 1.0)
    recall = float(hit.gather(1, oidx.reshape(-1, kk).long()).sum()) / (est.shape[0] * kk)
    torch.cuda.synchronize()

    # the scoring pass with the probability matrix written too (B*H*n_t^2 floats more)
    probs = torch.empty((B, H, nt, nt), dtype=torch.float32, device="cuda")
    score_p = (lambda: sa.score(kk, probs=probs)) if args.path == "tiled" else (lambda: sa.score_raster(q, kk, probs=probs))
    score_p()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        score_p()
    e1.record()
    torch.cuda.synchronize()
    score_p_ms = e0.elapsed_time(e1) / 10
    score_p_bytes = alone_bytes + B * H * nt * nt * 4   # the call alone, plus the probabilities
    del probs

    # the step's attention with V in each layout the kernel reads (bit-identical outputs):
    # tile-major rows (the default, copied by the scoring launch), channel-major tiles, and
    # the raster tensor itself
    v_layouts = None
    if args.path != "tiled":
        v_cols = torch.empty_like(sa.v_t)
        V.veda_tile_gather(geom, v, v_cols, V.COLS)
        o2 = torch.empty_like(out)
        runs = {"rows": [], "cols": [], "raster": []}
        for _ in range(3):   # interleaved rounds: the layouts see the same clock drift
            for name, vop, lay in (("rows", sa.v_t, V.ROWS), ("cols", v_cols, V.COLS), ("raster", v, V.RASTER)):
                runs[name].append(timed(lambda: V.veda_sparse_attn_fwd_raster(
                    geom, q, sa.k_t, vop, sa.idx_buffer(kk), kk, sa.softmax_scale, o2, k_layout=V.ROWS, v_layout=lay,
                    k_bound=sa.k_bound), 3))
        v_layouts = {f"{name}_ms": round(float(np.median(t)), 3) for name, t in runs.items()}
        v_layouts["note"] = ("attention alone with raster Q and O, tiled K; median of three interleaved rounds of "
                             "3 calls per layout, after the timed steps")
        del v_cols, o2

    # this library's own dense path (k = n_t, 0 % skipping), for the speedup
    dense = None
    if not args.no_dense:
        didx = dense_index(geom)
        say("[bench] dense path (k = n_t)")
        attend = (lambda ix: sa.attend(ix)) if args.path == "tiled" else (lambda ix: sa.attend_raster(q, ix, out))
        if args.path == "tiled":
            sa.gather(q, k, v)
        attend(didx)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 3
        e0.record()
        for _ in range(reps):
            attend(didx)
        e1.record()
        torch.cuda.synchronize()
        dense_ms = e0.elapsed_time(e1) / reps
        dense = {"ms": round(dense_ms, 3),
                 "tflops": round(cfg.kept_flops(nt) / (dense_ms * 1e-3) / 1e12, 1),
                 "speedup_sparse_vs_dense": round(dense_ms / attn_ms, 2),
                 "ideal_speedup": round(nt / kk, 2)}
        del didx

    # the rows built beyond the forward path, timed outside the step
    nxt = None
    if not args.no_next:
        say("[bench] distillation step and per-head error kernel")
        sa.gather(q, k, v)  # the distillation step reads tiled Q and K
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        sa.distill_step(qtl, tmap)  # warm-up (allocates its workspace once)
        torch.cuda.synchronize()
        reps = 5
        e0.record()
        for _ in range(reps):
            sa.distill_step(qtl, tmap)
        e1.record()
        torch.cuda.synchronize()
        distill_ms = e0.elapsed_time(e1) / reps
        err = torch.empty((B, H), dtype=torch.float32, device="cuda")
        ref = torch.empty_like(err)
        hws = torch.empty(V.veda_head_sq_error_workspace_bytes(B, N, H), dtype=torch.uint8, device="cuda")
        V.veda_head_sq_error(out, q, err, ref, workspace=hws)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            V.veda_head_sq_error(out, q, err, ref, workspace=hws)
        e1.record()
        torch.cuda.synchronize()
        herr_ms = e0.elapsed_time(e1) / reps
        herr_bytes = 2 * B * N * H * d * 2
        # Padded tilings: the same workload with its full shape cycle, where (8,4,4) does not divide
        # T = 20, on the default path (gather V; score with K tiled on the way; attention and
        # tile map with Q and O raster)
        pcfg = padded_variant(cfg)
        pshapes = pcfg.head_shapes()
        pgeom = V.Geom(B, H, d, cfg.grid, P, pshapes)
        pad_row = None
        if pgeom.padded:
            say("[bench] padded tiling step (full shape cycle)")
            psa = SparseAttention(pgeom, torch.bfloat16, torch.from_numpy(wl.w1), torch.from_numpy(wl.w2),
                                  score_scale=cfg.score_scale)
            prng = np.random.default_rng(cfg.seed + 2000)
            pqt = torch.from_numpy(np.stack([np.sort(prng.choice(pgeom.head_tiles(h), n_sel, replace=False))
                                             for h in range(H)]).astype(np.int32)[None].repeat(B, 0)).cuda()
            pmap = torch.empty((B, H, n_sel, pgeom.n_tiles), dtype=torch.float32, device="cuda")
            pout = torch.empty_like(q)

            def pstep():   # the default path: K and V tiled by the scoring launch, Q and O raster
                pidx = psa.score_raster(q, kk, k=k, tile_k=True, v=v)
                psa.attend_raster(q, pidx, pout)
                psa.tilemap_raster(q, pqt, n_sel, pmap)
                return pidx

            pidx = pstep()
            torch.cuda.synchronize()
            e0.record()
            for _ in range(reps):
                pstep()
            e1.record()
            torch.cuda.synchronize()
            pstep_ms = e0.elapsed_time(e1) / reps
            e0.record()
            for _ in range(reps):
                psa.attend_raster(q, pidx, pout)
            e1.record()
            torch.cuda.synchronize()
            pattn_ms = e0.elapsed_time(e1) / reps
            # kept work: every (query tile, kept key tile) pair of every head, padding rows included
            pflops = sum(4.0 * pgeom.head_tiles(h) * kk * P * P * d for h in range(H)) * B
            pad_row = {"padded_shapes": sorted(set(map(tuple, pshapes))),
                       "padded_tiles_per_head": sorted(set(pgeom.head_tiles(h) for h in range(H))),
                       "padded_step_ms": round(pstep_ms, 3), "padded_attn_ms": round(pattn_ms, 3),
                       "padded_attn_tflops": round(pflops / (pattn_ms * 1e-3) / 1e12, 1)}
            del psa, pmap, pout
        say("[bench] distillation: tile recall before and after SGD steps")
        drec = distill_recall(sa, q, k, v, qtl, n_sel, cfg)
        nxt = {"distill_step_ms": round(distill_ms, 4),
               "distill_recall": drec,
               # the step reads every K tile and the sampled Q tiles once
               "distill_step_qk_read_gbps": round(B * H * (nt + n_sel) * P * d * 2 / (distill_ms * 1e-3) / 1e9, 1),
               "distill_sampled_query_tiles_per_head": n_sel,
               "head_sq_error_ms": round(herr_ms, 4),
               "head_sq_error_gbps": round(herr_bytes / (herr_ms * 1e-3) / 1e9, 1),
               "head_sq_error_frac_hbm_peak": round(herr_bytes / (herr_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)}
        if pad_row is not None:
            nxt.update(pad_row)

    if args.copy_calibration:
        n = 1 << 29  # 1 GiB of bf16
        src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        say("[bench] copy calibration: 3 x 1 GiB device copies")
        del src, dst

    long_row = None
    if not args.no_long:
        del sa
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        long_row = long_sweep()

    cpu = None
    if not args.no_cpu_baseline:
        say("[bench] CPU oracle baseline (bounded sample)")
        cpu = cpu_baseline(cfg, wl, kk, n_sel)

    traffic = traffic_from_counters(args.path)
    roof = {"kernel": "attn_bf16_kernel", "bound": "mfma", "achieved": round(attn_tflops, 1),
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "flops_per_launch": kept, "avg_launch_ms": round(attn_ms, 4)}
    result = {
        "metric": METRIC,
        "value": round(kept / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{cfg.name}: B={B} H={H} d={d} latent {'x'.join(map(str, cfg.grid))} "
                               f"(N={N}), tile {P}, k={kk}/{nt} kept ({100 * (1 - kk / nt):.0f}% skipped)",
                   "path": args.path,
                   "batch": B, "heads": H, "seq_len": N, "head_dim": d, "tile": P, "topk": kk, "n_tiles": nt,
                   "tile_shapes": sorted(set(wl.shapes)), "tilemap_query_tiles_per_head": n_sel},
        "sparse_attn_ms_per_call": round(attn_ms, 4),
        "sparse_attn_ms_median_min": [round(float(np.median(per_stage["sparse_attn"])), 4),
                                      round(float(np.min(per_stage["sparse_attn"])), 4)],
        "sparse_attn_tflops": round(attn_tflops, 1),
        "sparse_attn_frac_bf16_peak": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
        "scoring_ms": round(score_ms, 4),
        "scoring_bytes": score_bytes,
        "scoring_gbps": round(score_bytes / (score_ms * 1e-3) / 1e9, 1),
        "scoring_frac_hbm_peak": round(score_bytes / (score_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
        "scoring_note": ("the step's scoring stage: TripPool of raster Q and K -> MLP -> scores -> top-k, with K's "
                         "tile-major copy written in the same pass and V's streamed by the same launch"
                         if args.path != "tiled" else
                         "the step's scoring stage (tiled Q and K read, lists written)"),
        "scoring_pass_alone": alone,
        "scoring_with_probs": {"ms": round(score_p_ms, 4), "gbps": round(score_p_bytes / (score_p_ms * 1e-3) / 1e9, 1),
                               "frac_hbm_peak": round(score_p_bytes / (score_p_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
                               "bytes": score_p_bytes},
        "stages_median_ms": {s: round(x, 4) for s, x in med.items()},
        "tile_recall": {"value": round(recall, 4), "k": kk, "sampled_query_tiles_per_head": n_sel,
                        "chance": round(kk / nt, 4),
                        "note": "estimator with the synthetic (untrained) MLP weights against the oracle mask"},
        "attention_v_layouts": v_layouts,
        "dense": dense,
        "next_rows": nxt,
        "long_workload": long_row,
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
