"""One DiT self-attention layer through the library: head-aware tiling of Q, K, V ->
distilled tile scoring with top-k -> tile-skipping attention -> un-tiling of the output.

PyTorch only allocates device buffers (reused across calls) and supplies the stream; every
step is a call into libveda.
"""
import math

import torch

from . import (RASTER, ROWS, Geom, veda_distill_step, veda_distill_workspace_bytes, veda_head_sq_error,
               veda_head_sq_error_workspace_bytes,
               veda_oracle_tilemap, veda_oracle_tilemap_raster, veda_oracle_tilemap_workspace_bytes,
               veda_sparse_attn_fwd, veda_sparse_attn_fwd_raster, veda_tile_gather, veda_trippool_score,
               veda_trippool_score_raster, veda_trippool_workspace_bytes)


class SparseAttention:
    """Holds the geometry, the per-head estimator weights and reusable device buffers."""

    def __init__(self, geom: Geom, dtype: torch.dtype, w1, w2, w1_k=None, w2_k=None, score_scale=0.125,
                 softmax_scale=None, device="cuda"):
        self.geom, self.dtype, self.device = geom, dtype, device
        self.w1 = w1.to(device=device, dtype=torch.float32).contiguous()
        self.w2 = w2.to(device=device, dtype=torch.float32).contiguous()
        self.w1_k = self.w1 if w1_k is None else w1_k.to(device=device, dtype=torch.float32).contiguous()
        self.w2_k = self.w2 if w2_k is None else w2_k.to(device=device, dtype=torch.float32).contiguous()
        self.score_scale = float(score_scale)
        self.softmax_scale = 1.0 / math.sqrt(geom.head_dim) if softmax_scale is None else float(softmax_scale)
        g = geom
        shape = (g.batch, g.heads, g.n_tiled, g.head_dim)   # n_tiled = n_tokens unless the tiling is padded
        self.q_t = torch.empty(shape, dtype=dtype, device=device)
        self.k_t = torch.empty(shape, dtype=dtype, device=device)
        self.v_t = torch.empty(shape, dtype=dtype, device=device)   # tile-major (ROWS), like q_t and k_t
        self.o_t = torch.empty(shape, dtype=dtype, device=device)
        # each key tile's row-norm bound, written by the scoring calls and passed to attention
        # while it describes the K that attention reads (_kb_src: the tensors it was computed
        # from, k_t and/or a raster K)
        self.k_bound = torch.empty((g.batch, g.heads, g.n_tiles), dtype=torch.float32, device=device)
        self._kb_src = ()
        nbytes = veda_trippool_workspace_bytes(g, self.w1.shape[-1], self.w2.shape[-1])
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self._idx = {}
        self._tm_ws = {}

    def idx_buffer(self, k):
        if k not in self._idx:
            g = self.geom
            self._idx[k] = torch.empty((g.batch, g.heads, g.n_tiles, k), dtype=torch.int32, device=self.device)
        return self._idx[k]

    def gather(self, q, k, v):
        """q, k, v: [B, N, H, d] (last dim contiguous)."""
        veda_tile_gather(self.geom, q, self.q_t, ROWS)
        veda_tile_gather(self.geom, k, self.k_t, ROWS)
        veda_tile_gather(self.geom, v, self.v_t, ROWS)
        self._kb_src = ()

    def _bound_for(self, k):
        """The key-tile bounds if they were computed from k (the tensor attention reads)."""
        return self.k_bound if any(x is k for x in self._kb_src) else None

    def score(self, topk, scores=None, probs=None, q_desc=None, k_desc=None):
        idx = self.idx_buffer(topk) if topk > 0 else None
        veda_trippool_score(self.geom, self.q_t, self.k_t, self.w1, self.w2, self.w1_k, self.w2_k,
                            self.score_scale, scores=scores, probs=probs, q_desc=q_desc, k_desc=k_desc,
                            topk=topk, idx=idx, workspace=self.ws, k_bound=self.k_bound)
        self._kb_src = (self.k_t,)
        return idx

    def attend(self, idx, lse=None):
        veda_sparse_attn_fwd(self.geom, self.q_t, self.k_t, self.v_t, idx, int(idx.shape[-1]),
                             self.softmax_scale, self.o_t, lse, v_layout=ROWS, k_bound=self._bound_for(self.k_t))
        return self.o_t

    def scatter(self, out):
        """Write the tiled output back to raster order: out [B, N, H, d]."""
        veda_tile_gather(self.geom, out, self.o_t, ROWS, inverse=True)
        return out

    def tilemap(self, q_tiles, n_sel, out, lse=None):
        if n_sel not in self._tm_ws:
            nbytes = veda_oracle_tilemap_workspace_bytes(self.geom, n_sel)
            self._tm_ws[n_sel] = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        veda_oracle_tilemap(self.geom, self.q_t, self.k_t, self.softmax_scale, q_tiles, n_sel, out, lse,
                            self._tm_ws[n_sel])
        return out

    def distill_step(self, q_tiles, target, lr=0.0):
        """One KL distillation step of this layer's estimator on the gathered Q, K: the
        sampled query tiles q_tiles [B, H, n_sel] (int32) against target rows
        [B, H, n_sel, n_t] (e.g. tilemap() of the same tiles).  Returns (loss [1], dw1, dw2);
        with lr != 0 the weights are updated in place.  Needs one MLP shared by Q and K."""
        if self.w1_k is not self.w1 or self.w2_k is not self.w2:
            raise ValueError("the distillation step trains one MLP per head shared by Q and K")
        n_sel = int(q_tiles.shape[-1])
        key = ("distill", n_sel)
        if key not in self._tm_ws:
            nbytes = veda_distill_workspace_bytes(self.geom, n_sel)
            self._tm_ws[key] = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        loss = torch.empty(1, dtype=torch.float32, device=self.device)
        dw1, dw2 = torch.empty_like(self.w1), torch.empty_like(self.w2)
        veda_distill_step(self.geom, self.q_t, self.k_t, self.w1, self.w2, q_tiles, target, loss, dw1, dw2,
                          score_scale=self.score_scale, lr=lr, workspace=self._tm_ws[key])
        return loss, dw1, dw2

    # ---- raster-direct path: Q and O stay in the raster layout.  K is read raster (pass k)
    # or from its tiled copy (k=None: gather_kv first, or the scoring pass with tile_k); V
    # from its tiled copy (gather_kv, gather_v, or the scoring pass given v).
    def gather_kv(self, k, v):
        veda_tile_gather(self.geom, k, self.k_t, ROWS)
        veda_tile_gather(self.geom, v, self.v_t, ROWS)
        self._kb_src = ()

    def gather_v(self, v):
        veda_tile_gather(self.geom, v, self.v_t, ROWS)

    def _k(self, k):
        return (self.k_t, ROWS) if k is None else (k, RASTER)

    def score_raster(self, q, topk, k=None, scores=None, probs=None, q_desc=None, k_desc=None, tile_k=False,
                     v=None):
        """Scoring on raster Q; K raster (k given) or its tiled copy.  tile_k (raster K only):
        also write K's tiled copy while pooling it, in place of gather_kv's K gather; v (raster,
        strides of q): the same launch also writes V's tiled copy, in place of gather_v."""
        idx = self.idx_buffer(topk) if topk > 0 else None
        kt, lay = self._k(k)
        veda_trippool_score_raster(self.geom, q, kt, self.w1, self.w2, self.w1_k, self.w2_k, self.score_scale,
                                   scores=scores, probs=probs, q_desc=q_desc, k_desc=k_desc, topk=topk, idx=idx,
                                   workspace=self.ws, k_layout=lay, k_tiled_out=self.k_t if tile_k else None,
                                   v=v, v_tiled_out=None if v is None else self.v_t, k_bound=self.k_bound)
        # the bounds describe the K read, and its tiled copy when this call wrote it
        self._kb_src = (self.k_t,) if k is None else ((k, self.k_t) if tile_k else (k,))
        return idx

    def attend_raster(self, q, idx, out, lse=None, k=None):
        kt, lay = self._k(k)
        veda_sparse_attn_fwd_raster(self.geom, q, kt, self.v_t, idx, int(idx.shape[-1]), self.softmax_scale, out,
                                    lse, k_layout=lay, v_layout=ROWS, k_bound=self._bound_for(kt))
        return out

    def tilemap_raster(self, q, q_tiles, n_sel, out, lse=None, k=None):
        if n_sel not in self._tm_ws:
            nbytes = veda_oracle_tilemap_workspace_bytes(self.geom, n_sel)
            self._tm_ws[n_sel] = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        kt, lay = self._k(k)
        veda_oracle_tilemap_raster(self.geom, q, kt, self.softmax_scale, q_tiles, n_sel, out, lse,
                                   self._tm_ws[n_sel], k_layout=lay)
        return out

    def forward_raster(self, q, k, v, topk, out):
        """Same result as forward(), without the tiled copies of Q and O; the scoring launch
        tiles K as it pools it and streams V into its tiled copy beside."""
        idx = self.score_raster(q, topk, k=k, tile_k=True, v=v)
        return self.attend_raster(q, idx, out)

    def forward(self, q, k, v, topk, out):
        self.gather(q, k, v)
        idx = self.score(topk)
        self.attend(idx)
        return self.scatter(out)


def dense_index(geom: Geom, device="cuda"):
    """Kept-tile list with every key tile (0 % skipping): the dense path."""
    g = geom
    if g.padded:
        raise ValueError("the dense kept-tile list needs one tile count for every head")
    return (torch.arange(g.n_tiles, dtype=torch.int32, device=device)
            .expand(g.batch, g.heads, g.n_tiles, g.n_tiles).contiguous())


def search_tile_shapes(grid, tile, candidates, q, k, v, w1, w2, topk, score_scale=0.125, softmax_scale=None,
                       device="cuda"):
    """Head-aware tiling search on calibration inputs: every candidate tiling runs the
    scored sparse attention of the layer for all heads, and each head keeps the candidate
    whose output is closest to full attention (squared error summed over the batch; ties
    to the earlier candidate).

    q, k, v: raster [B, N, H, d] GPU tensors; candidates: list of (p_t, p_h, p_w).
    Returns (choice: list of candidate indices per head, err [C, B, H] and ref [B, H] as
    float32 GPU tensors, ref being the squared norm of the full output).  The outputs,
    errors, batch sums and norms come from the library's kernels; only the argmin over the
    candidates is taken here."""
    B, N, H, d = (int(x) for x in q.shape)
    dt = q.dtype
    if not candidates:
        raise ValueError("no candidate tilings")
    err = torch.empty((len(candidates), B, H), dtype=torch.float32, device=device)
    total = torch.empty((len(candidates), H), dtype=torch.float32, device=device)
    ref = torch.empty((B, H), dtype=torch.float32, device=device)
    full = torch.empty_like(q)
    # full attention: every key tile kept (the un-tiled output does not depend on the tiling)
    sa = SparseAttention(Geom(B, H, d, grid, tile, [candidates[0]] * H), dt, w1, w2, score_scale=score_scale,
                         softmax_scale=softmax_scale, device=device)
    sa.gather(q, k, v)
    sa.attend(dense_index(sa.geom, device))
    sa.scatter(full)
    out = torch.empty_like(q)
    ws = torch.empty(veda_head_sq_error_workspace_bytes(B, N, H), dtype=torch.uint8, device=device)
    for ci, shape in enumerate(candidates):
        sa = SparseAttention(Geom(B, H, d, grid, tile, [tuple(shape)] * H), dt, w1, w2, score_scale=score_scale,
                             softmax_scale=softmax_scale, device=device)
        sa.forward(q, k, v, topk, out)
        veda_head_sq_error(out, full, err[ci], ref if ci == 0 else None, workspace=ws, err_batch_sum=total[ci])
    total = total.cpu()
    choice = [int(torch.argmin(total[:, h]).item()) for h in range(H)]
    return choice, err, ref
