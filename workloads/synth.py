"""Seeded synthetic inputs for the workloads in ``configs``.

Shared by the tests, the benchmark and the oracle's callers.  It only draws and lays
out inputs; it computes no step of the method.

Recipe (per workload, seed s):
  * ``rng = default_rng(s)`` draws, in order: per-head position-code axis scales
    ``U(0.25, 2)`` of shape [H, 3] (all 1.0 for the tiny workload), the sink key
    indices (``choice(N, n_sink, replace=False)``), then the estimator weights
    ``W1 ~ N(0, 1/(3d))`` [H, 3d, hidden] and ``W2 ~ N(0, 1/hidden)`` [H, hidden, out],
    float32 (variance = 1/fan_in).
  * Head h draws qn, kn, v ~ N(0,1) of shape [B, N, d] (float32) from its own stream
    ``default_rng([s, h])``, so any head can be regenerated alone.
  * A 3D sinusoidal code PE of each token's integer (t, h, w): the channels split into
    [t | h | w] blocks of widths (d - 2m, m, m), m = 2*floor(d/6); in a block of width w
    with coordinate c and head axis scale a, channel 2i = sin(a*c*f_i), 2i+1 = cos(a*c*f_i),
    f_i = 10000^(-2i/w).  Computed in float64, stored as float32.
  * Q = 0.5*qn + PE, K = 0.5*kn + PE, V = v (float32); then K at the sink tokens is
    multiplied by 4 in every head.  bf16 workloads round Q, K, V to bfloat16
    (round to nearest, ties to even); everything downstream sees the rounded values.
  * Sampled query tiles (large workloads): ``default_rng(s + 1000)`` draws, per head,
    ``sorted(choice(n_t, n_sample, replace=False))``.

The raster layout a DiT block hands over is [B, N, H, d] with token n = (t*H + h)*W + w.
Inputs are generated and held head-major, [B, H, N, d] (contiguous per head);
``Workload.raster`` gives the [B, N, H, d] view.
"""
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import List, Optional

import numpy as np

from .configs import Config


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns the uint16 bit patterns.

    Inputs here are finite, so no NaN handling is needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(b).astype(np.uint32) << np.uint32(16)).view(np.float32)


def position_code(grid, d: int, axis_scale) -> np.ndarray:
    """3D sinusoidal code, float32 [N, d], for one head with axis scales (a_t, a_h, a_w)."""
    T, Hs, Ws = grid
    m = 2 * (d // 6)
    widths = (d - 2 * m, m, m)
    blocks = []
    for extent, width, a in zip((T, Hs, Ws), widths, axis_scale):
        c = np.arange(extent, dtype=np.float64)[:, None]
        f = 10000.0 ** (-2.0 * np.arange(width // 2, dtype=np.float64) / width)
        ang = float(a) * c * f[None, :]
        blk = np.empty((extent, width), dtype=np.float64)
        blk[:, 0::2] = np.sin(ang)
        blk[:, 1::2] = np.cos(ang)
        blocks.append(blk)
    blocks = [b.astype(np.float32) for b in blocks]
    pe = np.empty((T, Hs, Ws, d), dtype=np.float32)
    o = 0
    pe[..., o:o + widths[0]] = blocks[0][:, None, None, :]
    o += widths[0]
    pe[..., o:o + widths[1]] = blocks[1][None, :, None, :]
    o += widths[1]
    pe[..., o:o + widths[2]] = blocks[2][None, None, :, :]
    return pe.reshape(T * Hs * Ws, d)


@dataclass
class Workload:
    cfg: Config
    q: np.ndarray                 # [B,H,N,d]: uint16 bf16 bits (bf16) or float32 (f32)
    k: np.ndarray
    v: np.ndarray
    w1: np.ndarray                # [H, 3d, hidden] float32
    w2: np.ndarray                # [H, hidden, out] float32
    axis_scales: np.ndarray       # [H, 3] float64
    sinks: np.ndarray             # [n_sink] int64
    shapes: List[tuple]           # per-head (p_t, p_h, p_w)
    q_sample: Optional[np.ndarray]  # [H, n_sample] int64 sorted, or None (all tiles)

    @property
    def is_bf16(self) -> bool:
        return self.cfg.dtype == "bf16"

    def head(self, which: str, b: int, h: int) -> np.ndarray:
        """float32 [N, d] values (after bf16 rounding, if any) of Q, K or V for (b, h)."""
        a = {"q": self.q, "k": self.k, "v": self.v}[which][b, h]
        return bf16_bits_to_f32(a) if self.is_bf16 else np.array(a, dtype=np.float32)

    def raster(self, which: str) -> np.ndarray:
        """[B, N, H, d] view (not contiguous) of Q, K or V."""
        return {"q": self.q, "k": self.k, "v": self.v}[which].transpose(0, 2, 1, 3)

    def sample_tiles(self, h: int) -> np.ndarray:
        if self.q_sample is None:
            return np.arange(self.cfg.head_tiles(h))
        return self.q_sample[h]


def make(cfg: Config, heads: Optional[List[int]] = None) -> Workload:
    """Generate the workload.  ``heads`` restricts Q/K/V generation to those heads
    (the other heads stay zero); weights, sinks and samples are always complete."""
    B, H, d, N = cfg.batch, cfg.heads, cfg.head_dim, cfg.n_tokens
    rng = np.random.default_rng(cfg.seed)
    if cfg.unit_axis_scale:
        scales = np.ones((H, 3))
    else:
        scales = rng.uniform(0.25, 2.0, size=(H, 3))
    sinks = (np.sort(rng.choice(N, cfg.n_sink, replace=False)).astype(np.int64)
             if cfg.n_sink else np.zeros(0, np.int64))
    fan1 = 3 * d
    w1 = (rng.standard_normal((H, fan1, cfg.mlp_hidden), dtype=np.float32)
          / np.float32(np.sqrt(fan1))).astype(np.float32)
    w2 = (rng.standard_normal((H, cfg.mlp_hidden, cfg.mlp_out), dtype=np.float32)
          / np.float32(np.sqrt(cfg.mlp_hidden))).astype(np.float32)

    store = np.uint16 if cfg.dtype == "bf16" else np.float32
    q = np.zeros((B, H, N, d), dtype=store)
    k = np.zeros((B, H, N, d), dtype=store)
    v = np.zeros((B, H, N, d), dtype=store)
    half = np.float32(0.5)

    def one_head(h):
        hr = np.random.default_rng([cfg.seed, h])
        qn = hr.standard_normal((B, N, d), dtype=np.float32)
        kn = hr.standard_normal((B, N, d), dtype=np.float32)
        vn = hr.standard_normal((B, N, d), dtype=np.float32)
        pe = position_code(cfg.grid, d, scales[h])
        qh = half * qn + pe[None]
        kh = half * kn + pe[None]
        if len(sinks):
            kh[:, sinks, :] *= np.float32(4.0)
        if cfg.dtype == "bf16":
            q[:, h] = f32_to_bf16_bits(qh)
            k[:, h] = f32_to_bf16_bits(kh)
            v[:, h] = f32_to_bf16_bits(vn)
        else:
            q[:, h] = qh
            k[:, h] = kh
            v[:, h] = vn

    todo = list(range(H) if heads is None else heads)
    workers = max(1, min(len(todo), (os.cpu_count() or 1), 16))
    if workers == 1:
        for h in todo:
            one_head(h)
    else:
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(one_head, todo))

    q_sample = None
    if cfg.sampled_q_tiles is not None:
        r2 = np.random.default_rng(cfg.seed + 1000)
        q_sample = np.stack([np.sort(r2.choice(cfg.head_tiles(h) if cfg.padded else cfg.n_tiles,
                                               cfg.sampled_q_tiles, replace=False))
                             for h in range(H)]).astype(np.int64)
    return Workload(cfg, q, k, v, w1, w2, scales, sinks, cfg.head_shapes(), q_sample)

