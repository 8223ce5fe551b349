"""Plant plausible mistakes in copies of oracle functions (on the CPU) and check that at
least one pin catches each: a dropped term, a wrong sign or index, a transposed operand,
a swapped axis, a wrong tie order."""
import numpy as np
import pytest
from scipy.special import erf

import oracle.veda_oracle as O
import test_oracle_pins as pins


def _fails(pin, *fns):
    try:
        pin(*fns)
    except (AssertionError, ValueError, IndexError):
        return True
    return False


def perm_swapped_inner(grid, shape):
    T, H, W = grid
    pt, ph, pw = shape
    tok = np.arange(T * H * W).reshape(T // pt, pt, H // ph, ph, W // pw, pw)
    return tok.transpose(0, 2, 4, 1, 5, 3).reshape(-1)        # (h, w) swapped inside tile


def perm_tile_order_colmajor(grid, shape):
    T, H, W = grid
    pt, ph, pw = shape
    tok = np.arange(T * H * W).reshape(T // pt, pt, H // ph, ph, W // pw, pw)
    return tok.transpose(4, 2, 0, 1, 3, 5).reshape(-1)        # tiles numbered w-fastest... reversed


def perm_no_tiling(grid, shape):
    return np.arange(grid[0] * grid[1] * grid[2])


def trippool_min_is_max(xt, P):
    t = np.asarray(xt, np.float64).reshape(-1, P, xt.shape[1])
    return np.concatenate([t.mean(1), t.max(1), t.max(1)], 1)


def trippool_sum_not_mean(xt, P):
    t = np.asarray(xt, np.float64).reshape(-1, P, xt.shape[1])
    return np.concatenate([t.sum(1), t.max(1), t.min(1)], 1)


def trippool_order_swapped(xt, P):
    t = np.asarray(xt, np.float64).reshape(-1, P, xt.shape[1])
    return np.concatenate([t.max(1), t.mean(1), t.min(1)], 1)


def gelu_tanh(x):
    x = np.asarray(x, np.float64)
    return 0.5 * x * (1 + np.tanh(np.sqrt(2 / np.pi) * (x + 0.044715 * x ** 3)))


def gelu_no_sqrt2(x):
    x = np.asarray(x, np.float64)
    return 0.5 * x * (1 + erf(x))


def mlp_no_gelu(desc, w1, w2):
    return (desc @ w1) @ w2


def mlp_relu(desc, w1, w2):
    return np.maximum(desc @ w1, 0) @ w2


def scores_wrong_scale(yq, yk, scale):
    return (yq @ yk.T) / np.sqrt(yq.shape[1])


def softmax_cols(s):
    e = np.exp(s - s.max(axis=0, keepdims=True))
    return e / e.sum(axis=0, keepdims=True)


def topk_ties_high(scores, k):
    s = np.asarray(scores, np.float64)
    cols = np.arange(s.shape[1])
    return np.stack([np.sort(np.lexsort((-cols, -row))[:k]) for row in s])


def topk_smallest(scores, k):
    s = np.asarray(scores, np.float64)
    cols = np.arange(s.shape[1])
    return np.stack([np.sort(np.lexsort((cols, row))[:k]) for row in s])


def topk_unsorted(scores, k):
    s = np.asarray(scores, np.float64)
    cols = np.arange(s.shape[1])
    return np.stack([np.lexsort((cols, -row))[:k] for row in s])


def dense_no_scale(q, k, v, scale, return_lse=False):
    return O.dense_attention(q, k, v, 1.0)


def dense_transposed_p(q, k, v, scale, return_lse=False):
    s = (q @ k.T) * scale
    p = np.exp(s - s.max(axis=0, keepdims=True))
    p /= p.sum(axis=0, keepdims=True)
    return p @ v


def sparse_no_renorm(qt, kt, vt, idx, P, scale, q_tiles=None, return_lse=False):
    """Softmax over all keys, then zero the dropped ones (no renormalisation)."""
    n = qt.shape[0]
    n_t = n // P
    s = (qt @ kt.T) * scale
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    keep = np.zeros((n, n), bool)
    for i in range(n_t):
        for j in idx[i]:
            keep[i * P:(i + 1) * P, j * P:(j + 1) * P] = True
    out = np.where(keep, p, 0) @ vt
    if q_tiles is not None:
        out = np.concatenate([out[i * P:(i + 1) * P] for i in q_tiles])
    return (out, np.zeros(len(out))) if return_lse else out


def sparse_wrong_tile(qt, kt, vt, idx, P, scale, q_tiles=None, return_lse=False):
    """Off by one in the kept-tile rows."""
    idx2 = (np.asarray(idx) + 1) % (qt.shape[0] // P)
    return O.sparse_attention(qt, kt, vt, idx2, P, scale, q_tiles, return_lse)


def tilemap_mean(qt, kt, P, scale, q_tiles=None):
    n_t = kt.shape[0] // P
    q_tiles = np.arange(qt.shape[0] // P) if q_tiles is None else q_tiles
    out = []
    for i in q_tiles:
        s = (qt[i * P:(i + 1) * P] @ kt.T) * scale
        p = np.exp(s - s.max(1, keepdims=True))
        p /= p.sum(1, keepdims=True)
        out.append(p.reshape(P, n_t, P).mean(axis=(0, 2)))
    return np.array(out)


def tilemap_unnormalised(qt, kt, P, scale, q_tiles=None):
    n_t = kt.shape[0] // P
    q_tiles = np.arange(qt.shape[0] // P) if q_tiles is None else q_tiles
    out = []
    for i in q_tiles:
        s = (qt[i * P:(i + 1) * P] @ kt.T) * scale
        out.append(np.exp(s - s.max(1, keepdims=True)).reshape(P, n_t, P).max(axis=(0, 2)))
    return np.array(out)


def search_argmax(q, k, v, grid, P, candidates, w1, w2, topk, score_scale, scale):
    """Picks the worst candidate."""
    choice, err, ref = O.search_tile_shapes(q, k, v, grid, P, candidates, w1, w2, topk, score_scale, scale)
    return err.sum(axis=1).argmax(axis=0), err, ref


def search_no_untiling(q, k, v, grid, P, candidates, w1, w2, topk, score_scale, scale):
    """Compares the tile-major output with the raster-order full output."""
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    B, N, H, _ = q.shape
    err = np.zeros((len(candidates), B, H))
    ref = np.zeros((B, H))
    for b in range(B):
        for h in range(H):
            full = O.dense_attention(q[b, :, h], k[b, :, h], v[b, :, h], scale)
            ref[b, h] = (full ** 2).sum()
            for ci, shape in enumerate(candidates):
                perm = O.tile_permutation(grid, shape)
                qt, kt, vt = (O.to_tiles(x[b, :, h], perm) for x in (q, k, v))
                yq = O.mlp(O.trippool(qt, P), w1[h], w2[h])
                yk = O.mlp(O.trippool(kt, P), w1[h], w2[h])
                idx = O.topk_rows(O.tile_scores(yq, yk, score_scale).astype(np.float32), topk)
                err[ci, b, h] = O.head_output_error(O.sparse_attention(qt, kt, vt, idx, P, scale), full)
    return err.sum(axis=1).argmin(axis=0), err, ref


def search_batch0_only(q, k, v, grid, P, candidates, w1, w2, topk, score_scale, scale):
    """Chooses from the first calibration batch alone."""
    _, err, ref = O.search_tile_shapes(q, k, v, grid, P, candidates, w1, w2, topk, score_scale, scale)
    return err[:, 0, :].argmin(axis=0), err, ref


def search_last_batch_only(q, k, v, grid, P, candidates, w1, w2, topk, score_scale, scale):
    """Chooses from the last calibration batch alone."""
    _, err, ref = O.search_tile_shapes(q, k, v, grid, P, candidates, w1, w2, topk, score_scale, scale)
    return err[:, -1, :].argmin(axis=0), err, ref


def search_sum_over_heads(q, k, v, grid, P, candidates, w1, w2, topk, score_scale, scale):
    """Sums the errors over heads too, so every head gets the same tiling."""
    _, err, ref = O.search_tile_shapes(q, k, v, grid, P, candidates, w1, w2, topk, score_scale, scale)
    best = int(err.sum(axis=(1, 2)).argmin())
    return np.full(err.shape[2], best), err, ref


def _rows_and_blocks(descs, q_tiles):
    return sum(len(np.asarray(q_tiles[bh])) for bh, _ in descs), len(descs)


def distill_loss_mean_blocks(descs, w1, w2, q_tiles, targets, score_scale):
    """Divides the summed KL by the number of (batch, head) blocks instead of the rows."""
    rows, blocks = _rows_and_blocks(descs, q_tiles)
    return O.distill_loss(descs, w1, w2, q_tiles, targets, score_scale) * rows / blocks


def distill_grads_mean_blocks(descs, w1, w2, q_tiles, targets, score_scale):
    """The same divisor in the gradients (so they stay consistent with that loss)."""
    rows, blocks = _rows_and_blocks(descs, q_tiles)
    loss, g1, g2 = O.distill_grads(descs, w1, w2, q_tiles, targets, score_scale)
    return loss * rows / blocks, g1 * rows / blocks, g2 * rows / blocks


def distill_loss_unnormalised(descs, w1, w2, q_tiles, targets, score_scale):
    """Takes the target rows as they come, without dividing by their sums."""
    total, rows = 0.0, 0
    for (bh, h), (dq, dk) in descs.items():
        sel = np.asarray(q_tiles[bh])
        s = O.tile_scores(O.mlp(dq, w1[h], w2[h])[sel], O.mlp(dk, w1[h], w2[h]), score_scale)
        total += O.kl_rows(np.asarray(targets[bh], np.float64), s).sum()
        rows += len(sel)
    return total / rows


def gelu_grad_no_density(x):
    """Drops the x phi(x) term."""
    x = np.asarray(x, np.float64)
    return 0.5 * (1.0 + erf(x / np.sqrt(2.0)))


def kl_reversed(p, s):
    """KL(softmax(s) || p) instead of KL(p || softmax(s))."""
    p, s = np.asarray(p, np.float64), np.asarray(s, np.float64)
    q = O.row_softmax(s)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.where(q > 0, q * (np.log(q) - np.log(np.where(p > 0, p, 1e-300))), 0.0)
    return t.sum(axis=1)


def distill_grads_sign(descs, w1, w2, q_tiles, targets, score_scale):
    """dL/ds = p - softmax(s) (wrong sign)."""
    loss, g1, g2 = O.distill_grads(descs, w1, w2, q_tiles, targets, score_scale)
    return loss, -g1, -g2


def distill_grads_no_dyk(descs, w1, w2, q_tiles, targets, score_scale):
    """Forgets that the key-tile outputs depend on the weights too."""
    w1, w2 = np.asarray(w1, np.float64), np.asarray(w2, np.float64)
    g1, g2 = np.zeros_like(w1), np.zeros_like(w2)
    rows = sum(len(np.asarray(q_tiles[bh])) for bh, _ in descs)
    total = 0.0
    for (bh, h), (dq, dk) in descs.items():
        zq = np.asarray(dq, np.float64) @ w1[h]
        hq = O.gelu(zq)
        yq, yk = hq @ w2[h], O.mlp(dk, w1[h], w2[h])
        sel = np.asarray(q_tiles[bh])
        s = O.tile_scores(yq[sel], yk, score_scale)
        t = np.asarray(targets[bh], np.float64)
        p = t / t.sum(axis=1, keepdims=True)
        total += O.kl_rows(p, s).sum()
        ds = (O.row_softmax(s) - p) / rows
        dyq = np.zeros_like(yq)
        np.add.at(dyq, sel, score_scale * ds @ yk)
        g2[h] += hq.T @ dyq
        g1[h] += np.asarray(dq, np.float64).T @ ((dyq @ w2[h].T) * O.gelu_grad(zq))
    return total / rows, g1, g2


def slots_wraparound(grid, shape):
    T, H, W = grid
    pt, ph, pw = shape
    nT, nH, nW = -(-T // pt), -(-H // ph), -(-W // pw)
    t = np.arange(nT * pt)[:, None, None] % T
    h = np.arange(nH * ph)[None, :, None] % H
    w = np.arange(nW * pw)[None, None, :] % W
    tok = (t * H + h) * W + w                                   # padding wraps to real tokens
    return tok.reshape(nT, pt, nH, ph, nW, pw).transpose(0, 2, 4, 1, 3, 5).reshape(-1)


def trippool_padded_mean_over_p(xt, P, valid=None):
    t = np.asarray(xt, np.float64).reshape(-1, P, xt.shape[1])
    v = np.ones(t.shape[:2] + (1,), bool) if valid is None else np.asarray(valid, bool).reshape(-1, P, 1)
    return np.concatenate([np.where(v, t, 0).sum(1) / P, np.where(v, t, -np.inf).max(1),
                           np.where(v, t, np.inf).min(1)], 1)


def trippool_padded_unmasked(xt, P, valid=None):
    return O.trippool(xt, P)                                    # padding rows (zeros) counted


def sparse_ignores_key_mask(qt, kt, vt, idx, P, scale, q_tiles=None, return_lse=False, key_valid=None):
    return O.sparse_attention(qt, kt, vt, idx, P, scale, q_tiles, return_lse)


def tilemap_ignores_key_mask(qt, kt, P, scale, q_tiles=None, key_valid=None, query_valid=None):
    return O.tilemap(qt, kt, P, scale, q_tiles, None, query_valid)


def tilemap_ignores_query_mask(qt, kt, P, scale, q_tiles=None, key_valid=None, query_valid=None):
    return O.tilemap(qt, kt, P, scale, q_tiles, key_valid, None)


MUTANTS = [
    ("perm: in-tile axes swapped", [pins.pin_perm_golden, pins.pin_perm_loops], [perm_swapped_inner]),
    ("perm: tile order reversed", [pins.pin_perm_golden, pins.pin_perm_loops], [perm_tile_order_colmajor]),
    ("perm: identity", [pins.pin_perm_golden, pins.pin_perm_loops], [perm_no_tiling]),
    ("trippool: min dropped", [pins.pin_trippool_golden, pins.pin_trippool_loops], [trippool_min_is_max]),
    ("trippool: sum for mean", [pins.pin_trippool_golden, pins.pin_trippool_loops], [trippool_sum_not_mean]),
    ("trippool: block order", [pins.pin_trippool_golden, pins.pin_trippool_loops], [trippool_order_swapped]),
    ("gelu: tanh form", [pins.pin_gelu_table], [gelu_tanh]),
    ("gelu: missing sqrt2", [pins.pin_gelu_table], [gelu_no_sqrt2]),
    ("mlp: activation dropped", [pins.pin_mlp_torch], [mlp_no_gelu]),
    ("mlp: relu", [pins.pin_mlp_torch], [mlp_relu]),
    ("scores: 1/sqrt(dim) scale", [lambda f: pins.pin_scores_hand(f, O.row_softmax)], [scores_wrong_scale]),
    ("softmax: over columns", [lambda f: pins.pin_scores_hand(O.tile_scores, f)], [softmax_cols]),
    ("topk: ties to higher index", [pins.pin_topk_bruteforce, pins.pin_topk_ties], [topk_ties_high]),
    ("topk: smallest", [pins.pin_topk_bruteforce, pins.pin_topk_ties], [topk_smallest]),
    ("topk: not ascending", [pins.pin_topk_bruteforce, pins.pin_topk_ties], [topk_unsorted]),
    ("attention: no scale", [pins.pin_attention_sdpa], [dense_no_scale]),
    ("attention: softmax over queries", [pins.pin_attention_hand, pins.pin_attention_sdpa], [dense_transposed_p]),
    ("sparse: no renormalisation", [pins.pin_sparse_vs_masked_matrix], [sparse_no_renorm]),
    ("sparse: wrong kept tile", [pins.pin_sparse_vs_masked_matrix], [sparse_wrong_tile]),
    ("tilemap: mean pooling", [pins.pin_tilemap_hand, pins.pin_tilemap_bruteforce], [tilemap_mean]),
    ("tilemap: not normalised", [pins.pin_tilemap_hand, pins.pin_tilemap_bruteforce], [tilemap_unnormalised]),
    ("search: argmax", [pins.pin_search_block_local], [search_argmax]),
    ("gelu': density term dropped", [pins.pin_gelu_grad_fd], [gelu_grad_no_density]),
    ("kl: direction reversed", [pins.pin_kl_rows], [kl_reversed]),
    ("distill: gradient sign", [pins.pin_distill_fd], [distill_grads_sign]),
    ("distill: key-tile path dropped", [pins.pin_distill_fd], [distill_grads_no_dyk]),
    ("search: first batch only", [pins.pin_search_batch_sum], [search_batch0_only]),
    ("search: last batch only", [pins.pin_search_batch_sum], [search_last_batch_only]),
    ("search: errors summed over heads", [pins.pin_search_batch_sum], [search_sum_over_heads]),
    ("distill: mean over blocks (loss and gradients)", [pins.pin_distill_hand],
     [distill_loss_mean_blocks, distill_grads_mean_blocks]),
    ("distill: target rows not normalised", [pins.pin_distill_hand], [distill_loss_unnormalised]),
    ("search: output left tile-major", [pins.pin_search_block_local, pins.pin_search_all_kept], [search_no_untiling]),
    ("slots: padding wraps around", [pins.pin_slots_golden, pins.pin_slots_loops], [slots_wraparound]),
    ("trippool padded: mean over P", [pins.pin_trippool_padded_loops], [trippool_padded_mean_over_p]),
    ("trippool padded: padding counted", [pins.pin_trippool_padded_loops], [trippool_padded_unmasked]),
    ("sparse padded: padding keys kept", [pins.pin_sparse_padded_full_equals_dense], [sparse_ignores_key_mask]),
    ("tilemap padded: padding keys kept", [pins.pin_tilemap_padded_bruteforce], [tilemap_ignores_key_mask]),
    ("tilemap padded: padding queries pooled", [pins.pin_tilemap_padded_bruteforce], [tilemap_ignores_query_mask]),
]


@pytest.mark.parametrize("name,pin_list,fns", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, pin_list, fns):
    assert any(_fails(p, *fns) for p in pin_list), f"no pin caught: {name}"
