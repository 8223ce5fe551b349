"""CPU oracle of Veda's distilled sparse attention hot path.  TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline leg may import
this module.  The HIP library never does, and the two share no code: no helpers, tables or
constants.  Inputs come from ``workloads`` (seeded data only).

Everything is plain float64 numpy, written to be read against the pages
("Technical Summary: Veda - Scalable Video Diffusion via Distilled Sparse Attention",
gist.science, and the arXiv abstract on fugumt.com).  No blocking, fusion or reordering
beyond the definitions below; a library matmul, sort or erf serves as a step.

Where the pages leave a step open, the plainest reading is taken:
  * tiles and the tokens inside a tile are numbered row-major over (t, h, w);
  * TripPool = [mean | max | min] over the tile's tokens, per channel;
  * the estimator is one 2-layer MLP per head (no bias, exact-erf GELU) applied to the
    Q-tile and K-tile descriptors; tile score = dot(y_q, y_k) * score_scale; the row
    distribution is the softmax over key tiles;
  * selection keeps the k largest scores per row, ties to the lower tile index, listed in
    ascending tile index;
  * sparse attention renormalises the softmax over the kept keys only (scale 1/sqrt(d));
  * the oracle tile map is the max, over each (query tile x key tile) region, of the
    full-attention probabilities normalised over all N keys.

Parity pins (tests/test_oracle_pins.py): every function below is pinned by closed forms,
hand-worked fixtures under tests/golden/, brute-force loops, or library routines of torch;
see each docstring.  The estimator's *form* (widths 3d->256->64, GELU, 1/8) is not given by
the pages, which print no estimator formula: parity against the paper's estimator is
unpinned; the functions are pinned to the definition stated above.
"""
import numpy as np
from scipy.special import erf


# ---------------------------------------------------------------------------
# Head-aware tiling  [Veda Technical Summary, §2.2 Head-Aware Tiling: each head gets a
# tiling (p_t, p_h, p_w) that factorises the hardware tile size]
# ---------------------------------------------------------------------------
def tile_permutation(grid, shape):
    """perm[r] = raster token index held by row r of the tile-major sequence.

    Raster token n = (t*H + h)*W + w.  Tile (a, b, c) covers t in [a*p_t, (a+1)*p_t), etc.;
    tiles are numbered row-major over (a, b, c), tokens inside a tile row-major over
    (t mod p_t, h mod p_h, w mod p_w).  Pinned: hand-derived fixtures, an explicit-loop
    construction, bijection.
    """
    T, H, W = grid
    pt, ph, pw = shape
    if T % pt or H % ph or W % pw:
        raise ValueError(f"tile shape {shape} does not divide grid {grid}")
    tok = np.arange(T * H * W).reshape(T // pt, pt, H // ph, ph, W // pw, pw)
    return tok.transpose(0, 2, 4, 1, 3, 5).reshape(-1)


def tile_slots(grid, shape):
    """Head-aware tiling for any tile shape: slots[r] = raster token index held by row r of
    the tile-major sequence, or -1 for a slot of the padded grid that holds no token.

    The grid is padded up to whole tiles on every axis (T' = ceil(T/p_t)*p_t, etc.); tiles
    of the padded grid and rows inside a tile are numbered row-major as in
    tile_permutation, and a slot is padding when its (t, h, w) lies outside the real grid.
    Every tile keeps at least one real token.  For a dividing shape this is
    tile_permutation.  Pinned: hand-derived fixture, explicit-loop construction, each real
    token exactly once.
    """
    T, H, W = grid
    pt, ph, pw = shape
    nT, nH, nW = -(-T // pt), -(-H // ph), -(-W // pw)
    t = np.arange(nT * pt)[:, None, None]
    h = np.arange(nH * ph)[None, :, None]
    w = np.arange(nW * pw)[None, None, :]
    tok = np.where((t < T) & (h < H) & (w < W), (t * H + h) * W + w, -1)
    return tok.reshape(nT, pt, nH, ph, nW, pw).transpose(0, 2, 4, 1, 3, 5).reshape(-1)


def to_tiles(x, perm):
    """Rows of the raster-ordered [N, d] array x, in tile-major order; slots marked -1
    (padding of tile_slots) are zero rows."""
    x = np.asarray(x, dtype=np.float64)
    perm = np.asarray(perm)
    out = np.zeros((len(perm),) + x.shape[1:])
    real = perm >= 0
    out[real] = x[perm[real]]
    return out


def from_tiles(xt, perm, n=None):
    """Inverse of to_tiles: the rows of the real slots back in raster order ([n, d], n =
    the number of real slots by default)."""
    xt = np.asarray(xt, dtype=np.float64)
    perm = np.asarray(perm)
    real = perm >= 0
    out = np.empty((int(real.sum()) if n is None else n,) + xt.shape[1:])
    out[perm[real]] = xt[real]
    return out


# ---------------------------------------------------------------------------
# Distilled tile scoring  [Veda Technical Summary, §2.1 Distilled Tile Scoring]
# ---------------------------------------------------------------------------
def trippool(xt, P, valid=None):
    """TripPool descriptor of each tile: [mean | max | min] over the tile's P tokens, per
    channel, concatenated (§2.1, "Statistic-Aware Estimator").  [n_t, 3d].
    valid (bool per tile-major row, e.g. tile_slots(...) >= 0): only the real tokens of a
    padded tile count.  Pinned: brute-force loops, hand fixture, constant tile."""
    xt = np.asarray(xt, dtype=np.float64)
    n_t = xt.shape[0] // P
    t = xt.reshape(n_t, P, xt.shape[1])
    if valid is None:
        return np.concatenate([t.mean(axis=1), t.max(axis=1), t.min(axis=1)], axis=1)
    v = np.asarray(valid, bool).reshape(n_t, P, 1)
    mean = np.where(v, t, 0.0).sum(axis=1) / v.sum(axis=1)
    return np.concatenate([mean, np.where(v, t, -np.inf).max(axis=1), np.where(v, t, np.inf).min(axis=1)], axis=1)


def gelu(x):
    """x * Phi(x) with the exact normal CDF.  Pinned: tabulated Phi values, torch's gelu."""
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + erf(x / np.sqrt(2.0)))


def mlp(desc, w1, w2):
    """Per-head projection of tile descriptors (§2.1, "Head-Specific Projections"):
    y = GELU(desc @ W1) @ W2, no bias.  Pinned: torch linear + gelu in float64."""
    desc = np.asarray(desc, dtype=np.float64)
    return gelu(desc @ np.asarray(w1, np.float64)) @ np.asarray(w2, np.float64)


def tile_scores(yq, yk, scale):
    """S[i, j] = scale * <y_q[i], y_k[j]>: score of key tile j for query tile i.
    Pinned: hand fixture, symmetry."""
    return (np.asarray(yq, np.float64) @ np.asarray(yk, np.float64).T) * float(scale)


def row_softmax(s):
    """Predicted tile-score distribution of each query-tile row (§2.1, "Optimization":
    row-wise distributions).  Pinned: hand fixture, rows sum to 1, shift invariance."""
    s = np.asarray(s, dtype=np.float64)
    z = s - s.max(axis=1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=1, keepdims=True)


def topk_rows(scores, k):
    """Kept key tiles of each row: the k largest scores, ties to the lower tile index,
    returned in ascending tile index.  [rows, k] int64.
    Pinned: brute-force full sort, crafted ties."""
    s = np.asarray(scores, dtype=np.float64)
    rows, n = s.shape
    if not 1 <= k <= n:
        raise ValueError("k out of range")
    cols = np.arange(n)
    out = np.empty((rows, k), dtype=np.int64)
    for i in range(rows):
        order = np.lexsort((cols, -s[i]))      # primary: larger score; then lower index
        out[i] = np.sort(order[:k])
    return out


# ---------------------------------------------------------------------------
# Attention  [Veda Technical Summary, §1 Problem Statement (full self-attention over the
# spatiotemporal tokens) and §2.3 Hardware-Efficient Implementation (a kernel that skips
# the key/value tiles not selected)]
# ---------------------------------------------------------------------------
def _softmax_rows_with_lse(s):
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=1, keepdims=True)
    return e / z, (m + np.log(z))[:, 0]


def dense_attention(q, k, v, scale, return_lse=False):
    """softmax(q k^T * scale) v over all keys.  Pinned: torch SDPA in float64."""
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    p, lse = _softmax_rows_with_lse((q @ k.T) * float(scale))
    return (p @ v, lse) if return_lse else p @ v


def sparse_attention(qt, kt, vt, idx, P, scale, q_tiles=None, return_lse=False, key_valid=None):
    """Tile-skipping attention on tile-major rows: query tile i attends only to the keys of
    the tiles idx[i, :], with the softmax renormalised over those keys.

    qt, kt, vt: [N, d]; idx: [n_t, k] (row i = kept key tiles of query tile i).
    key_valid (bool per tile-major row): padding keys of a padded tiling take no weight.
    Returns [len(q_tiles) * P, d] for the query tiles listed (default: all), and the
    natural-log LSE per query row if asked.  Pinned: 100%-kept equals dense attention (also
    over the real tokens of a padded tiling), explicit -inf mask on the full matrix,
    constant V, Q = 0.
    """
    qt, kt, vt = (np.asarray(a, np.float64) for a in (qt, kt, vt))
    n_t = qt.shape[0] // P
    q_tiles = np.arange(n_t) if q_tiles is None else np.asarray(q_tiles)
    out = np.empty((len(q_tiles) * P, qt.shape[1]))
    lses = np.empty(len(q_tiles) * P)
    off = np.arange(P)
    for a, i in enumerate(q_tiles):
        rows = (np.asarray(idx[i])[:, None] * P + off[None, :]).ravel()
        s = (qt[i * P:(i + 1) * P] @ kt[rows].T) * float(scale)
        if key_valid is not None:
            s = np.where(np.asarray(key_valid, bool)[rows][None, :], s, -np.inf)
        p, lse = _softmax_rows_with_lse(s)
        out[a * P:(a + 1) * P] = p @ vt[rows]
        lses[a * P:(a + 1) * P] = lse
    return (out, lses) if return_lse else out


# ---------------------------------------------------------------------------
# Oracle tile map  [Veda Technical Summary, §2.1 "Target Construction": max-pooling of the
# full-attention matrix over query-key tile regions; §2.3: heatmaps built in two passes on
# random subsets of query tiles]
# ---------------------------------------------------------------------------
def tilemap(qt, kt, P, scale, q_tiles=None, key_valid=None, query_valid=None):
    """M[a, j] = max over q in query tile q_tiles[a], key in tile j, of the full-attention
    probability softmax_row(q k^T * scale).  First the per-row log-sum-exp over all N keys,
    then the max over each region of exp(s - lse).  [len(q_tiles), n_t].
    key_valid / query_valid (bool per tile-major row): on a padded tiling, padding keys
    take no probability and padding query rows are left out of the max.
    Pinned: Q = 0 gives 1/N, explicit dense-P max-pool (also on a padded tiling),
    1/N <= row max <= 1."""
    qt, kt = np.asarray(qt, np.float64), np.asarray(kt, np.float64)
    n_t = kt.shape[0] // P
    q_tiles = np.arange(qt.shape[0] // P) if q_tiles is None else np.asarray(q_tiles)
    out = np.empty((len(q_tiles), n_t))
    for a, i in enumerate(q_tiles):
        s = (qt[i * P:(i + 1) * P] @ kt.T) * float(scale)          # [P, N]
        if key_valid is not None:
            s = np.where(np.asarray(key_valid, bool)[None, :], s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        lse = m + np.log(np.exp(s - m).sum(axis=1, keepdims=True))  # pass 1
        p = np.exp(s - lse)                                          # pass 2
        if query_valid is not None:
            p = np.where(np.asarray(query_valid, bool)[i * P:(i + 1) * P, None], p, -np.inf)
        out[a] = p.reshape(P, n_t, P).max(axis=(0, 2))
    return out


def recall(idx_est, idx_ref):
    """Mean over rows of |est ∩ ref| / k."""
    idx_est, idx_ref = np.asarray(idx_est), np.asarray(idx_ref)
    k = idx_ref.shape[1]
    hits = [len(np.intersect1d(a, b)) for a, b in zip(idx_est, idx_ref)]
    return float(np.mean(hits)) / k


# ---------------------------------------------------------------------------
# Head-aware tiling search  [Veda Technical Summary, §2.2 Head-Aware Tiling: each head's
# (p_t, p_h, p_w) is selected offline on calibration data by the error between the
# full-attention output and the sparse-attention output]
# ---------------------------------------------------------------------------
def head_output_error(o_sparse, o_full):
    """Squared Frobenius error of one head's output (raster order, [N, d])."""
    dlt = np.asarray(o_sparse, np.float64) - np.asarray(o_full, np.float64)
    return float((dlt * dlt).sum())


def search_tile_shapes(q, k, v, grid, P, candidates, w1, w2, topk, score_scale, scale):
    """For every candidate tiling, every head runs the scored sparse attention of one layer
    (tiling -> TripPool -> MLP -> scores -> top-k -> tile-skipping attention -> un-tiling)
    and its output is compared with full attention.

    q, k, v: raster [B, N, H, d]; w1 [H, 3d, hidden], w2 [H, hidden, out].
    Returns (choice [H]: index of the candidate with the least error summed over the batch,
    ties to the lower index; err [C, B, H]; ref [B, H] = squared norm of the full output).
    Pinned: a head whose attention is block-local on one candidate's tiles, with an
    estimator that keeps exactly those tiles, selects that candidate with zero error;
    with every tile kept, all errors vanish; two calibration batches whose block-local
    tilings disagree (per head) are decided by the error summed over the batch."""
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    B, N, H, _ = q.shape
    err = np.zeros((len(candidates), B, H))
    ref = np.zeros((B, H))
    for b in range(B):
        for h in range(H):
            full = dense_attention(q[b, :, h], k[b, :, h], v[b, :, h], scale)
            ref[b, h] = float((full * full).sum())
            for ci, shape in enumerate(candidates):
                perm = tile_permutation(grid, shape)
                qt, kt, vt = (to_tiles(x[b, :, h], perm) for x in (q, k, v))
                yq = mlp(trippool(qt, P), w1[h], w2[h])
                yk = mlp(trippool(kt, P), w1[h], w2[h])
                idx = topk_rows(tile_scores(yq, yk, score_scale).astype(np.float32), topk)
                o = from_tiles(sparse_attention(qt, kt, vt, idx, P, scale), perm)
                err[ci, b, h] = head_output_error(o, full)
    total = err.sum(axis=1)
    choice = np.array([int(np.argmin(total[:, h])) for h in range(H)])
    return choice, err, ref


# ---------------------------------------------------------------------------
# Distillation of the estimator  [Veda Technical Summary, §2.1 Distilled Tile Scoring,
# "Optimization": row-wise KL divergence between the full-attention reference and the
# predicted tile-score distribution; stop-gradient on the features feeding the estimator]
# ---------------------------------------------------------------------------
def gelu_grad(x):
    """d/dx [x Phi(x)] = Phi(x) + x phi(x).  Pinned: central differences of gelu."""
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * (1.0 + erf(x / np.sqrt(2.0))) + x * np.exp(-0.5 * x * x) / np.sqrt(2.0 * np.pi)


def kl_rows(p, s):
    """KL(p || softmax(s)) per row, with 0 log 0 = 0.  Pinned: zero when p = softmax(s),
    a hand-worked two-entry row, non-negativity."""
    p, s = np.asarray(p, np.float64), np.asarray(s, np.float64)
    m = s.max(axis=1, keepdims=True)
    logq = s - m - np.log(np.exp(s - m).sum(axis=1, keepdims=True))
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.where(p > 0, p * (np.log(np.where(p > 0, p, 1.0)) - logq), 0.0)
    return t.sum(axis=1)


def distill_loss(descs, w1, w2, q_tiles, targets, score_scale):
    """Mean over every sampled row of KL(target row normalised to sum 1 || softmax of the
    estimator's logits).  descs: dict {(block, h): (D_q [n_t, 3d], D_k [n_t, 3d])}, one
    entry per (batch, head) block with its head index h; w1 [H, 3d, hid], w2 [H, hid, out];
    q_tiles[block]: [n_sel] (blocks may sample different numbers of tiles);
    targets[block]: [n_sel, n_t].  Pinned: the hand-worked two-block case of
    tests/golden/distill_hand.txt (1 and 3 sampled rows, unnormalised targets)."""
    total, rows = 0.0, 0
    for (bh, h), (dq, dk) in descs.items():
        yq = mlp(dq, w1[h], w2[h])
        yk = mlp(dk, w1[h], w2[h])
        sel = np.asarray(q_tiles[bh])
        s = tile_scores(yq[sel], yk, score_scale)
        t = np.asarray(targets[bh], np.float64)
        total += kl_rows(t / t.sum(axis=1, keepdims=True), s).sum()
        rows += len(sel)
    return total / rows


def distill_grads(descs, w1, w2, q_tiles, targets, score_scale):
    """Loss and its gradients with respect to w1, w2 (same arguments as distill_loss), by
    the chain rule written out: dL/ds = (softmax(s) - p) / rows; dy_q, dy_k from
    s = scale y_q y_k^T; through y = GELU(D W1) W2 with D constant.  Pinned: central
    differences of distill_loss."""
    w1 = np.asarray(w1, np.float64)
    w2 = np.asarray(w2, np.float64)
    g1, g2 = np.zeros_like(w1), np.zeros_like(w2)
    rows = sum(len(np.asarray(q_tiles[bh])) for bh, _ in descs)
    total = 0.0
    for (bh, h), (dq, dk) in descs.items():
        zq, zk = np.asarray(dq, np.float64) @ w1[h], np.asarray(dk, np.float64) @ w1[h]
        hq, hk = gelu(zq), gelu(zk)
        yq, yk = hq @ w2[h], hk @ w2[h]
        sel = np.asarray(q_tiles[bh])
        s = tile_scores(yq[sel], yk, score_scale)
        t = np.asarray(targets[bh], np.float64)
        p = t / t.sum(axis=1, keepdims=True)
        total += kl_rows(p, s).sum()
        ds = (row_softmax(s) - p) / rows
        dyq = np.zeros_like(yq)
        np.add.at(dyq, sel, score_scale * ds @ yk)
        dyk = score_scale * ds.T @ yq[sel]
        g2[h] += hq.T @ dyq + hk.T @ dyk
        dzq = (dyq @ w2[h].T) * gelu_grad(zq)
        dzk = (dyk @ w2[h].T) * gelu_grad(zk)
        g1[h] += np.asarray(dq, np.float64).T @ dzq + np.asarray(dk, np.float64).T @ dzk
    return total / rows, g1, g2


# ---------------------------------------------------------------------------
# Index agreement under near-ties
# ---------------------------------------------------------------------------
def topk_agrees(score_row, idx_row, k, gap=1e-5):
    """Does idx_row (ascending, k entries) select the k largest of score_row?

    If the k-th and (k+1)-th largest differ by at least ``gap`` the set must equal the
    oracle's exactly.  Otherwise any k distinct indices are accepted that include every
    index scoring above (k-th + gap) and none scoring below ((k+1)-th - gap).
    Returns (ok, exempt)."""
    s = np.asarray(score_row, dtype=np.float64)
    idx = np.asarray(idx_row)
    n = s.shape[0]
    if idx.shape != (k,) or np.any(np.diff(idx) <= 0) or idx.min() < 0 or idx.max() >= n:
        return False, False
    ref = topk_rows(s[None, :], k)[0]
    if k == n:
        return bool(np.array_equal(idx, ref)), False
    srt = np.sort(s)[::-1]
    kth, nxt = srt[k - 1], srt[k]
    if kth - nxt >= gap:
        return bool(np.array_equal(idx, ref)), False
    sel = np.zeros(n, bool)
    sel[idx] = True
    must = s > kth + gap
    never = s < nxt - gap
    return bool(np.all(sel[must]) and not np.any(sel[never])), True
