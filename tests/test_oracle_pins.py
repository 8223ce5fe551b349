"""Pins of the CPU oracle to facts outside itself: hand-worked fixtures (tests/golden),
closed forms, brute-force loops, and torch's own routines.  CPU only.

Each pin is a plain function of the oracle function(s) it checks, so that
test_oracle_mutations.py can plant a mistake in a copy of the oracle and show that some
pin fails.
"""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle.veda_oracle as O
from conftest import read_golden


# ------------------------------------------------------------------ permutation
def pin_perm_golden(tile_permutation):
    for name in ("perm_tiny.txt", "perm_nonsquare.txt"):
        tagged, rows = read_golden(name)
        grid = tuple(int(x) for x in tagged["grid"][0])
        shape = tuple(int(x) for x in tagged["shape"][0])
        perm = tile_permutation(grid, shape)
        for r, n in rows:
            assert perm[int(r)] == int(n), (name, r, perm[int(r)], n)


def perm_by_loops(grid, shape):
    """Explicit construction: walk tiles row-major, then offsets inside the tile row-major."""
    T, H, W = grid
    pt, ph, pw = shape
    out = []
    for a in range(T // pt):
        for b in range(H // ph):
            for c in range(W // pw):
                for i in range(pt):
                    for j in range(ph):
                        for l in range(pw):
                            t, h, w = a * pt + i, b * ph + j, c * pw + l
                            out.append((t * H + h) * W + w)
    return np.array(out)


def pin_perm_loops(tile_permutation):
    cases = [((4, 8, 8), (4, 4, 4)), ((2, 4, 6), (1, 2, 3)), ((8, 16, 32), (2, 8, 8)),
             ((8, 16, 32), (8, 4, 4)), ((8, 16, 32), (1, 8, 16)), ((6, 4, 10), (3, 2, 5))]
    for grid, shape in cases:
        assert np.array_equal(tile_permutation(grid, shape), perm_by_loops(grid, shape)), (grid, shape)


def test_perm_golden():
    pin_perm_golden(O.tile_permutation)


def test_perm_loops():
    pin_perm_loops(O.tile_permutation)


def test_perm_bijection_and_roundtrip():
    rng = np.random.default_rng(0)
    for grid, shape in [((20, 32, 48), (2, 8, 8)), ((20, 32, 48), (1, 8, 16)), ((8, 16, 32), (8, 4, 4))]:
        perm = O.tile_permutation(grid, shape)
        n = grid[0] * grid[1] * grid[2]
        assert np.array_equal(np.sort(perm), np.arange(n))
        x = rng.standard_normal((n, 3))
        assert np.array_equal(O.from_tiles(O.to_tiles(x, perm), perm), x)


def test_perm_tile_is_a_box():
    """Every tile's tokens form exactly one (p_t, p_h, p_w) box of the grid."""
    grid, shape = (8, 16, 32), (4, 4, 8)
    perm = O.tile_permutation(grid, shape)
    P = 128
    T, H, W = grid
    for j in range(len(perm) // P):
        n = perm[j * P:(j + 1) * P]
        t, h, w = n // (H * W), (n // W) % H, n % W
        assert t.max() - t.min() + 1 == shape[0] and h.max() - h.min() + 1 == shape[1]
        assert w.max() - w.min() + 1 == shape[2] and len(set(n.tolist())) == P
        assert t.min() % shape[0] == 0 and h.min() % shape[1] == 0 and w.min() % shape[2] == 0


def test_perm_rejects_non_dividing():
    with pytest.raises(ValueError):
        O.tile_permutation((20, 48, 80), (8, 4, 4))


# ------------------------------------------------------------------ TripPool
def pin_trippool_golden(trippool):
    tagged, _ = read_golden("trippool_hand.txt")
    x = np.array(tagged["token"])
    assert np.allclose(trippool(x, 2)[0], tagged["desc"][0], rtol=0, atol=1e-15)


def pin_trippool_loops(trippool):
    rng = np.random.default_rng(1)
    P, n_t, d = 8, 5, 6
    x = rng.standard_normal((P * n_t, d))
    got = trippool(x, P)
    for j in range(n_t):
        for c in range(d):
            vals = [x[j * P + r, c] for r in range(P)]
            assert math.isclose(got[j, c], sum(vals) / P, rel_tol=1e-13, abs_tol=1e-13)
            assert got[j, d + c] == max(vals)
            assert got[j, 2 * d + c] == min(vals)


def test_trippool_golden():
    pin_trippool_golden(O.trippool)


def test_trippool_loops():
    pin_trippool_loops(O.trippool)


def test_trippool_constant_tile():
    x = np.full((128, 4), 2.5)
    assert np.all(O.trippool(x, 128) == 2.5)


# ------------------------------------------------------------------ MLP
def pin_gelu_table(gelu):
    _, rows = read_golden("gelu_phi.txt")
    for x, y in rows:
        assert math.isclose(float(gelu(np.array([x]))[0]), y, rel_tol=1e-14, abs_tol=1e-15), (x, y)


def pin_mlp_torch(mlp):
    rng = np.random.default_rng(2)
    desc = rng.standard_normal((7, 12))
    w1 = rng.standard_normal((12, 9)) / np.sqrt(12)
    w2 = rng.standard_normal((9, 5)) / 3.0
    t = torch.from_numpy
    ref = torch.nn.functional.linear(
        torch.nn.functional.gelu(torch.nn.functional.linear(t(desc), t(w1).T), approximate="none"), t(w2).T)
    assert np.allclose(mlp(desc, w1, w2), ref.numpy(), rtol=1e-13, atol=1e-13)


def test_gelu_table():
    pin_gelu_table(O.gelu)


def test_gelu_vs_torch_and_limits():
    x = np.linspace(-8, 8, 1001)
    ref = torch.nn.functional.gelu(torch.from_numpy(x), approximate="none").numpy()
    assert np.allclose(O.gelu(x), ref, rtol=1e-14, atol=1e-15)
    assert O.gelu(np.array([40.0]))[0] == 40.0 and O.gelu(np.array([-40.0]))[0] == 0.0


def test_mlp_torch():
    pin_mlp_torch(O.mlp)


# ------------------------------------------------------------------ scores, softmax
def pin_scores_hand(tile_scores, row_softmax):
    tagged, _ = read_golden("scores_hand.txt")
    yq = np.array(tagged["yq"])
    yk = np.array(tagged["yk"][0]).reshape(2, 2)
    assert np.allclose(tile_scores(yq, yk, 1 / 8), [tagged["s"][0]], rtol=0, atol=1e-15)
    assert np.allclose(row_softmax(np.array([[0.0, math.log(3.0)]])), [[0.25, 0.75]], rtol=0, atol=1e-15)


def test_scores_hand():
    pin_scores_hand(O.tile_scores, O.row_softmax)


def test_scores_symmetric_and_softmax_props():
    rng = np.random.default_rng(3)
    y = rng.standard_normal((10, 64))
    s = O.tile_scores(y, y, 1 / 8)
    assert np.allclose(s, s.T, rtol=0, atol=1e-13)
    p = O.row_softmax(s)
    assert np.allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    assert np.allclose(O.row_softmax(s + 7.5), p, rtol=0, atol=1e-15)
    ref = torch.softmax(torch.from_numpy(s), dim=1).numpy()
    assert np.allclose(p, ref, rtol=1e-13, atol=1e-16)


# ------------------------------------------------------------------ top-k
def pin_topk_bruteforce(topk_rows):
    rng = np.random.default_rng(4)
    s = np.round(rng.standard_normal((40, 23)) * 2) / 2        # many exact ties
    for k in (1, 3, 7, 23):
        got = topk_rows(s, k)
        for i in range(s.shape[0]):
            ranked = sorted(range(s.shape[1]), key=lambda j: (-s[i, j], j))
            assert list(got[i]) == sorted(ranked[:k]), (i, k)


def pin_topk_ties(topk_rows):
    s = np.array([[1.0, 3.0, 3.0, 2.0, 3.0]])
    assert list(topk_rows(s, 2)[0]) == [1, 2]
    assert list(topk_rows(s, 3)[0]) == [1, 2, 4]
    assert list(topk_rows(s, 4)[0]) == [1, 2, 3, 4]
    assert list(topk_rows(np.zeros((1, 6)), 3)[0]) == [0, 1, 2]


def test_topk_bruteforce():
    pin_topk_bruteforce(O.topk_rows)


def test_topk_ties():
    pin_topk_ties(O.topk_rows)


def test_topk_agrees_rule():
    s = np.array([5.0, 1.0, 4.0, 4.0 + 5e-6, 0.0])
    ok, ex = O.topk_agrees(s, np.array([0, 3]), 2)
    assert ok and ex                                    # exact choice inside the near-tie band
    ok, ex = O.topk_agrees(s, np.array([0, 2]), 2)
    assert ok and ex                                    # the other member of the near-tie
    ok, _ = O.topk_agrees(s, np.array([0, 1]), 2)
    assert not ok
    s2 = np.array([5.0, 1.0, 4.0, 3.0])
    assert O.topk_agrees(s2, np.array([0, 2]), 2) == (True, False)
    assert O.topk_agrees(s2, np.array([0, 3]), 2) == (False, False)
    assert O.topk_agrees(s2, np.array([2, 0]), 2) == (False, False)   # must be ascending


def test_recall():
    assert O.recall(np.array([[0, 1, 2], [3, 4, 5]]), np.array([[0, 1, 5], [3, 4, 5]])) == pytest.approx(5 / 6)


# ------------------------------------------------------------------ attention
def pin_attention_hand(dense_attention):
    tagged, _ = read_golden("attention_hand.txt")
    q = np.array(tagged["q"][0])[:, None]
    k = np.array(tagged["k"][0])[:, None]
    v = np.array(tagged["v"][0])[:, None]
    assert np.allclose(dense_attention(q, k, v, 1.0)[:, 0], tagged["o"][0], rtol=0, atol=1e-14)


def pin_attention_sdpa(dense_attention):
    rng = np.random.default_rng(5)
    q, k, v = (rng.standard_normal((37, 16)) for _ in range(3))
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(a)[None, None] for a in (q, k, v)))[0, 0].numpy()
    assert np.allclose(dense_attention(q, k, v, 1 / 4.0), ref, rtol=1e-12, atol=1e-13)


def pin_sparse_full_equals_dense(sparse_attention, dense_attention):
    rng = np.random.default_rng(6)
    P, n_t, d = 8, 6, 16
    q, k, v = (rng.standard_normal((P * n_t, d)) for _ in range(3))
    idx = np.tile(np.arange(n_t), (n_t, 1))
    assert np.allclose(sparse_attention(q, k, v, idx, P, 0.25), dense_attention(q, k, v, 0.25),
                       rtol=1e-12, atol=1e-13)


def pin_sparse_vs_masked_matrix(sparse_attention):
    """Kept-tile attention equals full attention with -inf on every dropped key tile."""
    rng = np.random.default_rng(7)
    P, n_t, d, kk = 8, 6, 16, 2
    q, k, v = (rng.standard_normal((P * n_t, d)) for _ in range(3))
    idx = np.stack([np.sort(rng.choice(n_t, kk, replace=False)) for _ in range(n_t)])
    s = (q @ k.T) * 0.25
    keep = np.zeros((P * n_t, P * n_t), bool)
    for i in range(n_t):
        for j in idx[i]:
            keep[i * P:(i + 1) * P, j * P:(j + 1) * P] = True
    s = np.where(keep, s, -np.inf)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    assert np.allclose(sparse_attention(q, k, v, idx, P, 0.25), p @ v, rtol=1e-12, atol=1e-13)
    out, lse = sparse_attention(q, k, v, idx, P, 0.25, q_tiles=[4, 1], return_lse=True)
    assert np.allclose(out[:P], (p @ v)[4 * P:5 * P], rtol=1e-12, atol=1e-13)
    s4 = (q[4 * P:5 * P] @ k.T) * 0.25
    s4 = np.where(keep[4 * P:5 * P], s4, -np.inf)
    assert np.allclose(lse[:P], np.log(np.exp(s4).sum(axis=1)), rtol=1e-13)


def test_attention_hand():
    pin_attention_hand(O.dense_attention)


def test_attention_sdpa():
    pin_attention_sdpa(O.dense_attention)


def test_sparse_full_equals_dense():
    pin_sparse_full_equals_dense(O.sparse_attention, O.dense_attention)


def test_sparse_vs_masked_matrix():
    pin_sparse_vs_masked_matrix(O.sparse_attention)


def test_sparse_constant_v_and_zero_q():
    rng = np.random.default_rng(8)
    P, n_t, d = 8, 5, 16
    q, k = rng.standard_normal((P * n_t, d)), rng.standard_normal((P * n_t, d))
    idx = np.stack([np.sort(rng.choice(n_t, 3, replace=False)) for _ in range(n_t)])
    v = np.full((P * n_t, d), -1.75)
    assert np.allclose(O.sparse_attention(q, k, v, idx, P, 0.3), -1.75, rtol=0, atol=1e-13)
    v = rng.standard_normal((P * n_t, d))
    out = O.sparse_attention(np.zeros_like(q), k, v, idx, P, 0.3)
    for i in range(n_t):
        rows = np.concatenate([np.arange(j * P, (j + 1) * P) for j in idx[i]])
        assert np.allclose(out[i * P:(i + 1) * P], v[rows].mean(axis=0), rtol=0, atol=1e-13)


def test_dominant_key():
    rng = np.random.default_rng(9)
    n, d = 64, 8
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    k[17] = q[3] * 50.0
    out = O.dense_attention(q, k, v, 1.0)
    assert np.allclose(out[3], v[17], atol=1e-10)


def test_unpermuted_dense_invariant_to_tile_shape():
    """With every tile kept, attention after un-permuting does not depend on the tiling."""
    rng = np.random.default_rng(10)
    grid = (8, 16, 32)
    n, d = 4096, 16
    q, k, v = (rng.standard_normal((n, d)) * 0.5 for _ in range(3))
    ref = O.dense_attention(q[:256], k, v, 0.25)
    for shape in [(2, 8, 8), (8, 4, 4), (1, 8, 16), (4, 4, 8)]:
        perm = O.tile_permutation(grid, shape)
        inv = np.empty_like(perm)
        inv[perm] = np.arange(n)
        qt, kt, vt = (O.to_tiles(a, perm) for a in (q, k, v))
        n_t = n // 128
        rows_needed = np.unique(inv[:256] // 128)
        idx = np.tile(np.arange(n_t), (n_t, 1))
        out_t = np.zeros((n, d))
        part = O.sparse_attention(qt, kt, vt, idx, 128, 0.25, q_tiles=rows_needed)
        for a, i in enumerate(rows_needed):
            out_t[i * 128:(i + 1) * 128] = part[a * 128:(a + 1) * 128]
        out = O.from_tiles(out_t, perm)
        assert np.allclose(out[:256], ref, rtol=1e-12, atol=1e-13), shape


# ------------------------------------------------------------------ tile map
def pin_tilemap_hand(tilemap):
    tagged, _ = read_golden("attention_hand.txt")
    q = np.array(tagged["q"][0])[:, None]
    k = np.array(tagged["k"][0])[:, None]
    assert np.allclose(tilemap(q, k, 1, 1.0).ravel(), tagged["p"][0], rtol=0, atol=1e-15)


def pin_tilemap_bruteforce(tilemap):
    rng = np.random.default_rng(11)
    P, n_t, d = 4, 5, 8
    q, k = rng.standard_normal((P * n_t, d)), rng.standard_normal((P * n_t, d))
    s = (q @ k.T) * 0.5
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    got = tilemap(q, k, P, 0.5, q_tiles=[3, 0, 4])
    for a, i in enumerate([3, 0, 4]):
        for j in range(n_t):
            best = max(p[r, c] for r in range(i * P, (i + 1) * P) for c in range(j * P, (j + 1) * P))
            assert math.isclose(got[a, j], best, rel_tol=1e-12)


def test_tilemap_hand():
    pin_tilemap_hand(O.tilemap)


def test_tilemap_bruteforce():
    pin_tilemap_bruteforce(O.tilemap)


def test_tilemap_zero_q_and_bounds():
    rng = np.random.default_rng(12)
    P, n_t, d = 8, 6, 16
    k = rng.standard_normal((P * n_t, d))
    m = O.tilemap(np.zeros((P * n_t, d)), k, P, 0.25)
    assert np.allclose(m, 1.0 / (P * n_t), rtol=1e-14)
    q = rng.standard_normal((P * n_t, d)) * 3
    m = O.tilemap(q, k, P, 0.25)
    assert np.all(m <= 1.0 + 1e-15) and np.all(m.max(axis=1) >= 1.0 / (P * n_t))


# ------------------------------------------------------------------ padded tiling (shapes that do not divide the grid)
PADDED_CASES = [((3, 2, 3), (2, 2, 2)), ((20, 8, 12), (8, 4, 4)), ((5, 6, 7), (2, 4, 2)), ((40, 4, 8), (16, 2, 4)),
                ((4, 8, 8), (4, 4, 4))]


def pin_slots_golden(tile_slots):
    tagged, rows = read_golden("slots_padded.txt")
    grid = tuple(int(x) for x in tagged["grid"][0])
    shape = tuple(int(x) for x in tagged["shape"][0])
    slots = tile_slots(grid, shape)
    assert len(slots) == len(rows)
    for r, n in rows:
        assert slots[int(r)] == int(n), (r, slots[int(r)], n)


def slots_by_loops(grid, shape):
    """Explicit construction on the padded grid: tiles row-major, rows row-major inside a
    tile, -1 where (t, h, w) is outside the real grid."""
    T, H, W = grid
    pt, ph, pw = shape
    out = []
    for a in range(-(-T // pt)):
        for b in range(-(-H // ph)):
            for c in range(-(-W // pw)):
                for i in range(pt):
                    for j in range(ph):
                        for l in range(pw):
                            t, h, w = a * pt + i, b * ph + j, c * pw + l
                            out.append((t * H + h) * W + w if (t < T and h < H and w < W) else -1)
    return np.array(out)


def pin_slots_loops(tile_slots):
    for grid, shape in PADDED_CASES:
        slots = tile_slots(grid, shape)
        assert np.array_equal(slots, slots_by_loops(grid, shape)), (grid, shape)
        n = grid[0] * grid[1] * grid[2]
        assert np.array_equal(np.sort(slots[slots >= 0]), np.arange(n))     # each real token once
        P = shape[0] * shape[1] * shape[2]
        assert np.all((slots.reshape(-1, P) >= 0).any(axis=1))              # no all-padding tile


def pin_trippool_padded_loops(trippool):
    rng = np.random.default_rng(21)
    for grid, shape in [((5, 6, 7), (2, 4, 2)), ((3, 2, 3), (2, 2, 2))]:
        P = shape[0] * shape[1] * shape[2]
        n, d = grid[0] * grid[1] * grid[2], 5
        x = rng.standard_normal((n, d)) - 2.0            # all below zero: a padding zero would show in max
        slots = O.tile_slots(grid, shape)
        got = trippool(O.to_tiles(x, slots), P, valid=slots >= 0)
        for j in range(len(slots) // P):
            toks = [slots[j * P + r] for r in range(P) if slots[j * P + r] >= 0]
            for c in range(d):
                vals = [x[t, c] for t in toks]
                assert math.isclose(got[j, c], sum(vals) / len(vals), rel_tol=1e-13, abs_tol=1e-13)
                assert got[j, d + c] == max(vals)
                assert got[j, 2 * d + c] == min(vals)


def pin_sparse_padded_full_equals_dense(sparse_attention):
    """All tiles kept on a padded tiling = dense attention over the real tokens."""
    rng = np.random.default_rng(22)
    for grid, shape in [((3, 5, 6), (2, 2, 2)), ((5, 6, 7), (2, 4, 2))]:
        P = shape[0] * shape[1] * shape[2]
        n, d = grid[0] * grid[1] * grid[2], 8
        q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
        slots = O.tile_slots(grid, shape)
        n_t = len(slots) // P
        idx = np.tile(np.arange(n_t), (n_t, 1))
        qt, kt, vt = (O.to_tiles(a, slots) for a in (q, k, v))
        out_t, lse_t = sparse_attention(qt, kt, vt, idx, P, 0.3, return_lse=True, key_valid=slots >= 0)
        ref, lse = O.dense_attention(q, k, v, 0.3, return_lse=True)
        assert np.allclose(O.from_tiles(out_t, slots, n), ref, rtol=1e-12, atol=1e-13)
        real = slots >= 0
        assert np.allclose(lse_t[real], lse[slots[real]], rtol=1e-13)


def pin_tilemap_padded_bruteforce(tilemap):
    rng = np.random.default_rng(23)
    grid, shape = (3, 4, 5), (2, 2, 2)
    P, n, d = 8, 60, 8
    q, k = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    s = (q @ k.T) * 0.5
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)                    # over the real keys only
    slots = O.tile_slots(grid, shape)
    n_t = len(slots) // P
    sel = [n_t - 1, 0, 3]
    got = tilemap(O.to_tiles(q, slots), O.to_tiles(k, slots), P, 0.5, q_tiles=sel, key_valid=slots >= 0,
                  query_valid=slots >= 0)
    for a, i in enumerate(sel):
        for j in range(n_t):
            best = max(p[slots[i * P + r], slots[j * P + c]] for r in range(P) for c in range(P)
                       if slots[i * P + r] >= 0 and slots[j * P + c] >= 0)
            assert math.isclose(got[a, j], best, rel_tol=1e-12)


def test_slots_golden():
    pin_slots_golden(O.tile_slots)


def test_slots_loops():
    pin_slots_loops(O.tile_slots)


def test_slots_dividing_is_permutation():
    for grid, shape in [((8, 16, 32), (2, 8, 8)), ((4, 8, 8), (4, 4, 4))]:
        assert np.array_equal(O.tile_slots(grid, shape), O.tile_permutation(grid, shape))


def test_padded_roundtrip():
    rng = np.random.default_rng(24)
    slots = O.tile_slots((5, 6, 7), (2, 4, 2))
    x = rng.standard_normal((210, 3))
    xt = O.to_tiles(x, slots)
    assert np.all(xt[slots < 0] == 0.0)
    assert np.array_equal(O.from_tiles(xt, slots, 210), x)


def test_trippool_padded_loops():
    pin_trippool_padded_loops(O.trippool)


def test_sparse_padded_full_equals_dense():
    pin_sparse_padded_full_equals_dense(O.sparse_attention)


def test_tilemap_padded_bruteforce():
    pin_tilemap_padded_bruteforce(O.tilemap)


# ------------------------------------------------------------------ tiling search
SEARCH_GRID, SEARCH_P, SEARCH_D = (4, 8, 8), 64, 64
SEARCH_CANDIDATES = [(4, 4, 4), (1, 8, 8), (2, 4, 8)]


def pin_search_block_local(search_tile_shapes):
    """Attention confined to the (1, 8, 8) tiles and an estimator that keeps each query
    tile's own tile (top-1): that candidate reproduces full attention up to e^-50 weights,
    the others miss most of each query's keys."""
    from cases import block_local_case
    q, k, v, w1, w2 = block_local_case(SEARCH_GRID, SEARCH_CANDIDATES[1], SEARCH_D, heads=2, batch=1)
    choice, err, ref = search_tile_shapes(q, k, v, SEARCH_GRID, SEARCH_P, SEARCH_CANDIDATES, w1, w2, 1, 0.125,
                                          1 / math.sqrt(SEARCH_D))
    assert list(choice) == [1, 1]
    rel = err[:, 0, :] / ref[0][None, :]
    assert np.all(rel[1] < 1e-15)
    assert np.all(rel[0] > 1e-2) and np.all(rel[2] > 1e-2)


def pin_search_all_kept(search_tile_shapes):
    """With every tile kept, the sparse output is full attention for every candidate."""
    rng = np.random.default_rng(13)
    N, H, d = 4 * 8 * 8, 1, SEARCH_D
    q, k, v = (rng.standard_normal((1, N, H, d)) for _ in range(3))
    w1 = rng.standard_normal((H, 3 * d, 256)) / np.sqrt(3 * d)
    w2 = rng.standard_normal((H, 256, 64)) / 16
    _, err, ref = search_tile_shapes(q, k, v, SEARCH_GRID, SEARCH_P, SEARCH_CANDIDATES, w1, w2, 4, 0.125, 0.125)
    assert np.all(err / ref[None] < 1e-24)


def pin_search_batch_sum(search_tile_shapes):
    """Two calibration batches that disagree: head 0 is block-local on candidate 0 in batch 0
    (V x 8) and on candidate 1 in batch 1; head 1 on candidate 1 in batch 0 and on
    candidate 2 in batch 1 (V x 8).  The error summed over the batch picks 0 for head 0 and
    2 for head 1.  Batch 0 alone would pick (0, 1), the last batch alone (1, 2), and one
    choice from errors summed over heads would be the same for both heads."""
    from cases import block_local_inputs
    c = SEARCH_CANDIDATES
    q, k, v, w1, w2 = block_local_inputs(SEARCH_GRID, [[c[0], c[1]], [c[1], c[2]]], SEARCH_D,
                                         v_scale=[[8.0, 1.0], [1.0, 8.0]])
    choice, err, ref = search_tile_shapes(q, k, v, SEARCH_GRID, SEARCH_P, c, w1, w2, 1, 0.125,
                                          1 / math.sqrt(SEARCH_D))
    assert list(choice) == [0, 2], (list(choice), err.sum(axis=1))
    assert err.shape == (3, 2, 2) and ref.shape == (2, 2)
    # each block's own tiling reproduces full attention
    assert err[0, 0, 0] < 1e-12 * ref[0, 0] and err[1, 1, 0] < 1e-12 * ref[1, 0]
    assert err[1, 0, 1] < 1e-12 * ref[0, 1] and err[2, 1, 1] < 1e-12 * ref[1, 1]


def test_search_block_local():
    pin_search_block_local(O.search_tile_shapes)


def test_search_batch_sum():
    pin_search_batch_sum(O.search_tile_shapes)


def test_search_all_kept():
    pin_search_all_kept(O.search_tile_shapes)


def test_head_output_error_closed_form():
    a = np.arange(12.0).reshape(3, 4)
    assert O.head_output_error(a, a) == 0.0
    assert O.head_output_error(a + 0.5, a) == 12 * 0.25


# ------------------------------------------------------------------ distillation
def pin_gelu_grad_fd(gelu_grad):
    x = np.array([-6.0, -2.5, -1.0, -0.3, 0.0, 0.4, 1.0, 2.2, 5.0])
    h = 1e-6
    fd = (O.gelu(x + h) - O.gelu(x - h)) / (2 * h)
    assert np.allclose(gelu_grad(x), fd, rtol=0, atol=1e-8)
    assert math.isclose(float(gelu_grad(np.array(0.0))), 0.5, abs_tol=1e-15)


def pin_kl_rows(kl_rows):
    s = np.array([[0.3, -1.2, 2.0, 0.1]])
    q = np.exp(s - s.max()) / np.exp(s - s.max()).sum()
    assert abs(kl_rows(q, s)[0]) < 1e-15
    assert math.isclose(kl_rows(np.array([[1.0, 0.0]]), np.array([[0.0, 0.0]]))[0], math.log(2.0), rel_tol=1e-14)
    # p = (0.5, 0.5), q = (0.2, 0.8): 0.5 log(0.5/0.2) + 0.5 log(0.5/0.8)
    s2 = np.log(np.array([[0.2, 0.8]]))
    want = 0.5 * math.log(2.5) + 0.5 * math.log(0.625)
    assert math.isclose(kl_rows(np.array([[0.5, 0.5]]), s2)[0], want, rel_tol=1e-13)
    rng = np.random.default_rng(21)
    p = rng.random((5, 7))
    p /= p.sum(axis=1, keepdims=True)
    assert np.all(kl_rows(p, rng.standard_normal((5, 7))) >= 0)


def _distill_case(seed=22, H=2, B=2, nt=6, d3=12, hid=5, out=4, n_sel=3):
    rng = np.random.default_rng(seed)
    descs = {(b * H + h, h): (rng.standard_normal((nt, d3)), rng.standard_normal((nt, d3)))
             for b in range(B) for h in range(H)}
    w1 = rng.standard_normal((H, d3, hid)) / np.sqrt(d3)
    w2 = rng.standard_normal((H, hid, out)) / np.sqrt(hid)
    q_tiles = {bh: np.array([0, 4, 4][:n_sel]) if bh == 1 else rng.choice(nt, n_sel, replace=False)
               for bh, _ in descs}
    targets = {bh: rng.random((n_sel, nt)) ** 3 for bh, _ in descs}
    return descs, w1, w2, q_tiles, targets


def distill_hand_case():
    """The blocks, sampled tiles, targets and hand-worked loss of tests/golden/distill_hand.txt,
    with seeded Q-tile descriptors and weights (the loss does not depend on them: every
    K-tile descriptor is zero, so every logit is 0)."""
    tagged, _ = read_golden("distill_hand.txt")
    nt = int(tagged["n_t"][0][0])
    rng = np.random.default_rng(31)
    d3, hid, out, H = 6, 5, 3, 2
    descs, q_tiles, targets = {}, {}, {}
    for row in tagged["block"]:
        bh, h = int(row[0]), int(row[1])
        descs[(bh, h)] = (rng.standard_normal((nt, d3)), np.zeros((nt, d3)))
        q_tiles[bh] = np.array([int(x) for x in row[2:]])
        targets[bh] = np.array([r[1:] for r in tagged["target"] if int(r[0]) == bh])
    w1 = rng.standard_normal((H, d3, hid))
    w2 = rng.standard_normal((H, hid, out))
    return descs, w1, w2, q_tiles, targets, tagged["loss"][0][0]


def pin_distill_hand(distill_loss, distill_grads=None):
    """The hand-worked loss: the mean over all four sampled rows of two blocks (1 and 3 rows)
    of KL(normalised target || uniform)."""
    descs, w1, w2, q_tiles, targets, want = distill_hand_case()
    assert math.isclose(distill_loss(descs, w1, w2, q_tiles, targets, 0.7), want, rel_tol=1e-13)
    if distill_grads is not None:
        assert math.isclose(distill_grads(descs, w1, w2, q_tiles, targets, 0.7)[0], want, rel_tol=1e-13)


def pin_distill_fd(distill_grads, distill_loss=None):
    """Central differences of the loss in every weight (one head's query tile sampled twice)."""
    distill_loss = O.distill_loss if distill_loss is None else distill_loss
    descs, w1, w2, q_tiles, targets = _distill_case()
    loss, g1, g2 = distill_grads(descs, w1, w2, q_tiles, targets, 0.3)
    assert math.isclose(loss, distill_loss(descs, w1, w2, q_tiles, targets, 0.3), rel_tol=1e-12)
    h = 1e-6
    for w, g in ((w1, g1), (w2, g2)):
        fd = np.zeros_like(w)
        for idx in np.ndindex(*w.shape):
            wp, wm = w.copy(), w.copy()
            wp[idx] += h
            wm[idx] -= h
            lp = distill_loss(descs, wp if w is w1 else w1, wp if w is w2 else w2, q_tiles, targets, 0.3)
            lm = distill_loss(descs, wm if w is w1 else w1, wm if w is w2 else w2, q_tiles, targets, 0.3)
            fd[idx] = (lp - lm) / (2 * h)
        assert np.allclose(g, fd, rtol=1e-5, atol=1e-9), np.abs(g - fd).max()


def test_gelu_grad_fd():
    pin_gelu_grad_fd(O.gelu_grad)


def test_kl_rows():
    pin_kl_rows(O.kl_rows)


def test_distill_grads_fd():
    pin_distill_fd(O.distill_grads)


def test_distill_hand():
    pin_distill_hand(O.distill_loss, O.distill_grads)


def test_distill_zero_at_match():
    """If the target rows are the estimator's own distribution, loss and gradients vanish."""
    descs, w1, w2, q_tiles, _ = _distill_case(seed=23)
    targets = {}
    for (bh, h), (dq, dk) in descs.items():
        s = O.tile_scores(O.mlp(dq, w1[h], w2[h])[q_tiles[bh]], O.mlp(dk, w1[h], w2[h]), 0.3)
        targets[bh] = O.row_softmax(s) * 7.0   # any positive scale: rows are normalised
    loss, g1, g2 = O.distill_grads(descs, w1, w2, q_tiles, targets, 0.3)
    assert abs(loss) < 1e-15 and np.abs(g1).max() < 1e-15 and np.abs(g2).max() < 1e-15
