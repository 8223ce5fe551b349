"""Constructed inputs for the tiling-search pins and tests (test helpers, not workload data).

A block-local head has Q = K = c * one-hot of each token's tile under one tiling, so a
query's attention weight stays inside its own tile of that tiling (score c^2 * scale
there, 0 elsewhere).  Estimator weights that pass the tile mean straight through make each
query tile score highest against itself, so top-1 selection under that tiling keeps
exactly the tile that full attention uses.  Every value is exact in bfloat16.
"""
import numpy as np

from workloads.synth import bf16_bits_to_f32, f32_to_bf16_bits


def block_id(grid, shape):
    """Tile index of every raster token under tiling `shape` (tiles row-major over the
    tile grid), written with explicit coordinate loops rather than an array reshape."""
    T, Hs, Ws = grid
    pt, ph, pw = shape
    nth, ntw = Hs // ph, Ws // pw
    out = np.empty(T * Hs * Ws, np.int64)
    for t in range(T):
        for h in range(Hs):
            for w in range(Ws):
                out[(t * Hs + h) * Ws + w] = ((t // pt) * nth + h // ph) * ntw + w // pw
    return out


def passthrough_weights(heads, d, hidden=256, out=64):
    """W1, W2 = identity on the leading channels: y = GELU(tile mean) on those channels."""
    w1 = np.zeros((heads, 3 * d, hidden), np.float32)
    w2 = np.zeros((heads, hidden, out), np.float32)
    for i in range(min(d, hidden)):
        w1[:, i, i] = 1.0
    for i in range(min(hidden, out)):
        w2[:, i, i] = 1.0
    return w1, w2


def block_local_inputs(grid, shape_of, d, v_scale=None, c=20.0, hidden=256, out=64, seed=0):
    """Raster [B, N, H, d] float32 q, k, v and pass-through weights, where head h of batch b
    is block-local on the tiling shape_of[b][h].  v_scale[b][h] (a power of two, so bf16
    stays exact) multiplies that block's V."""
    B, H = len(shape_of), len(shape_of[0])
    N = grid[0] * grid[1] * grid[2]
    q = np.zeros((B, N, H, d), np.float32)
    for b in range(B):
        for h in range(H):
            ids = block_id(grid, shape_of[b][h])
            if int(ids.max()) + 1 > min(d, out):
                raise ValueError("one-hot code needs d and the MLP width >= number of tiles")
            q[b, np.arange(N), h, ids] = np.float32(c)
    k = q.copy()
    rng = np.random.default_rng(seed)
    v = bf16_bits_to_f32(f32_to_bf16_bits(rng.standard_normal((B, N, H, d), dtype=np.float32)))
    if v_scale is not None:
        v = v * np.asarray(v_scale, np.float32)[:, None, :, None]
    w1, w2 = passthrough_weights(H, d, hidden, out)
    return q, k, v, w1, w2


def block_local_case(grid, shape, d, heads=1, batch=1, **kw):
    """Every head of every batch block-local on the one tiling `shape`."""
    return block_local_inputs(grid, [[shape] * heads for _ in range(batch)], d, **kw)
