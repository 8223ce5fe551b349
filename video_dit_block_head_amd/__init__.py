"""Python binding of libveda (the gfx950 HIP library behind include/veda.h).

Argument marshalling only: every step runs in the library's HIP kernels.  PyTorch supplies
device memory and the current HIP stream.  The functions keep the C names; tensors stand
in for device pointers, and outputs are caller-allocated tensors written in place.  Any
non-zero status raises VedaError.  Importing this module does not load the library; the
first call does, and raises if libveda.so has not been built.
"""
import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libveda.so")

F32, BF16 = 0, 1
ROWS, COLS, RASTER = 0, 1, 2
MAX_HEADS = 128


class VedaError(RuntimeError):
    pass


class _CGeom(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("t", ctypes.c_int32), ("h", ctypes.c_int32), ("w", ctypes.c_int32), ("tile", ctypes.c_int32),
                ("tile_shapes", ctypes.POINTER(ctypes.c_int32))]


class Geom:
    """Problem geometry: batch, heads, head_dim, latent grid (t, h, w), tile and the
    per-head tile shapes [(p_t, p_h, p_w)] * heads."""

    def __init__(self, batch, heads, head_dim, grid, tile, shapes):
        self.batch, self.heads, self.head_dim = int(batch), int(heads), int(head_dim)
        self.grid = tuple(int(x) for x in grid)
        self.tile = int(tile)
        self.shapes = [tuple(int(x) for x in s) for s in shapes]
        flat = [x for s in self.shapes for x in s]
        self._arr = (ctypes.c_int32 * max(1, len(flat)))(*flat)
        self._c = _CGeom(self.batch, self.heads, self.head_dim, *self.grid, self.tile,
                         ctypes.cast(self._arr, ctypes.POINTER(ctypes.c_int32)))

    @property
    def n_tokens(self):
        """Real tokens of the latent grid (raster layout)."""
        return self.grid[0] * self.grid[1] * self.grid[2]

    def head_tiles(self, h):
        """Tiles of head h on the grid padded up to whole tiles (n_tokens / tile unless the
        head's shape does not divide the grid)."""
        (T, H, W), (pt, ph, pw) = self.grid, self.shapes[h]
        return (-(-T // pt)) * (-(-H // ph)) * (-(-W // pw))

    @property
    def padded(self):
        """Some head's tile shape does not divide the grid."""
        T, H, W = self.grid
        return any(T % pt or H % ph or W % pw for pt, ph, pw in self.shapes)

    @property
    def n_tiles(self):
        """Tiles per head of the tiled layouts and of score / index rows (the largest
        head_tiles; n_tokens / tile unless padded)."""
        return max(self.head_tiles(h) for h in range(self.heads))

    @property
    def n_tiled(self):
        """Rows per head of the tiled layouts."""
        return self.n_tiles * self.tile

    @property
    def ref(self):
        return ctypes.byref(self._c)


_lib = None


def lib():
    """Load libveda.so (built in-tree by video_dit_block_head_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise VedaError(f"{LIB_PATH} is missing: build it with `python -m video_dit_block_head_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
        G = ctypes.POINTER(_CGeom)
        sig = {
            "veda_tile_gather": (i32, [G, i32, vp, i64, i64, i64, vp, i32, i32, vp]),
            "veda_trippool_workspace_bytes": (sz, [G, i32, i32]),
            "veda_trippool_score": (i32, [G, i32, vp, vp, vp, vp, vp, vp, i32, i32, f32, vp, vp, vp, vp, vp, i32,
                                          vp, vp, sz, vp]),
            "veda_topk_mask": (i32, [i64, i32, vp, i32, vp, vp, vp]),
            "veda_sparse_attn_fwd": (i32, [G, i32, vp, vp, vp, i32, vp, vp, i32, f32, vp, vp, vp]),
            "veda_oracle_tilemap_workspace_bytes": (sz, [G, i32]),
            "veda_oracle_tilemap": (i32, [G, i32, vp, vp, f32, vp, i32, vp, vp, vp, sz, vp]),
            "veda_head_sq_error_workspace_bytes": (sz, [i32, i32, i32]),
            "veda_head_sq_error": (i32, [i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp]),
            "veda_distill_workspace_bytes": (sz, [G, i32]),
            "veda_trippool_score_raster": (i32, [G, i32, vp, vp, i32, i64, i64, i64, vp, vp, vp, vp, i32, i32, f32,
                                                 vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp, sz, vp]),
            "veda_trippool_score_raster_noalloc": (i32, [G, i32, vp, vp, i32, i64, i64, i64, vp, vp, vp, vp, i32,
                                                         i32, f32, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp]),
            "veda_sparse_attn_fwd_raster": (i32, [G, i32, vp, vp, i32, i64, i64, i64, vp, i32, vp, vp, i32, f32,
                                                  vp, i64, i64, i64, vp, vp]),
            "veda_oracle_tilemap_raster": (i32, [G, i32, vp, vp, i32, i64, i64, i64, f32, vp, i32, vp, vp, vp, sz,
                                                 vp]),
            "veda_distill_step": (i32, [G, i32, vp, vp, vp, vp, i32, i32, f32, vp, i32, vp, vp, vp, vp, f32, vp, sz,
                                        vp]),
            "veda_tiled_tokens": (i64, [G, i32]),
            "veda_head_tiles": (i32, [G, i32, i32]),
            "veda_status_str": (ctypes.c_char_p, [i32]),
            "veda_last_hip_error": (ctypes.c_int, []),
            "veda_version": (ctypes.c_char_p, []),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype, fn.argtypes = res, args
        _lib = L
    return _lib


def _check(name, status):
    if status != 0:
        msg = lib().veda_status_str(status).decode()
        if status == -7:
            msg += f" (hipError {lib().veda_last_hip_error()})"
        raise VedaError(f"{name}: {msg} [{status}]")


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise VedaError(f"unsupported tensor dtype {t.dtype}")


class _Arg:
    """A tensor argument whose dtype and size have been checked; its device pointer is taken
    by _call once every argument of the call has passed those checks."""
    __slots__ = ("t", "name", "contig")

    def __init__(self, t, name, contig):
        self.t, self.name, self.contig = t, name, contig

    def ptr(self):
        if not self.t.is_cuda:
            raise VedaError(f"{self.name} must be a GPU tensor")
        if self.contig and not self.t.is_contiguous():
            raise VedaError(f"{self.name} must be contiguous")
        return ctypes.c_void_p(self.t.data_ptr())


def _p(t, name, need_contig=True, dtype=None, numel=None, shape=None):
    """Tensor argument t (None stays None) after checking its dtype and its size (at least
    `numel` elements, or exactly `shape`).  The C ABI cannot see buffer sizes: a short
    buffer would be read or written out of bounds, so every size is checked here, for every
    argument, before _call checks devices and takes any pointer."""
    if t is None:
        return None
    if dtype is not None and t.dtype != dtype:
        raise VedaError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise VedaError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if numel is not None and t.numel() < numel:
        raise VedaError(f"{name}: {t.numel()} elements, at least {numel} needed")
    return _Arg(t, name, need_contig)


def _call(name, *args):
    """Call entry point `name` of the library: tensor arguments must be GPU tensors (and
    contiguous where required); any non-zero status raises VedaError."""
    conv = [a.ptr() if isinstance(a, _Arg) else a for a in args]
    conv = [a.handle() if isinstance(a, _Stream) else a for a in conv]
    _check(name, getattr(lib(), name)(*conv))


def _ws(workspace):
    return 0 if workspace is None else workspace.numel() * workspace.element_size()


def _torch():
    import torch
    return torch


def _elem_dtype(t):
    """The element type of a Q/K/V operand (bf16 or fp32), as a torch dtype."""
    _dtype_code(t)
    return t.dtype


def _tiled_numel(geom):
    return geom.batch * geom.heads * geom.n_tiled * geom.head_dim


def _raster_shape(geom):
    return (geom.batch, geom.n_tokens, geom.heads, geom.head_dim)


class _Stream:
    """The HIP stream of a call (torch's current stream by default), resolved by _call after
    the tensor arguments have been checked."""
    __slots__ = ("s",)

    def __init__(self, s):
        self.s = s

    def handle(self):
        import torch
        s = torch.cuda.current_stream() if self.s is None else self.s
        return ctypes.c_void_p(s.cuda_stream)


def _stream(stream):
    return _Stream(stream)


def version():
    return lib().veda_version().decode()


def veda_tile_gather(geom, raster, tiled, layout=ROWS, inverse=False, stream=None):
    """raster: [B, N, H, d] tensor (any strides, last dim contiguous); tiled: contiguous
    tensor of B*H*N*d elements in `layout`.  inverse=True scatters tiled -> raster."""
    dt = _elem_dtype(raster)
    if raster.stride(-1) != 1:
        raise VedaError("raster: last dimension must be contiguous")
    _call("veda_tile_gather",
        geom.ref, _dtype_code(raster), _p(raster, "raster", False, dt, shape=_raster_shape(geom)),
        raster.stride(0), raster.stride(1), raster.stride(2), _p(tiled, "tiled", True, dt, _tiled_numel(geom)),
        int(layout), int(bool(inverse)), _stream(stream))


def veda_trippool_workspace_bytes(geom, mlp_hidden, mlp_out):
    return int(lib().veda_trippool_workspace_bytes(geom.ref, int(mlp_hidden), int(mlp_out)))


def _weights(geom, w1_q, w2_q, w1_k, w2_k):
    """Checked pointers of the estimator weights and the MLP widths (hidden, out)."""
    f32 = _torch().float32
    H, d3 = geom.heads, 3 * geom.head_dim
    if w1_q.dim() != 3 or w2_q.dim() != 3:
        raise VedaError("w1 [H, 3d, hidden] and w2 [H, hidden, out] expected")
    hidden, mout = int(w1_q.shape[-1]), int(w2_q.shape[-1])
    ws = (_p(w1_q, "w1_q", True, f32, shape=(H, d3, hidden)), _p(w2_q, "w2_q", True, f32, shape=(H, hidden, mout)),
          _p(w1_k, "w1_k", True, f32, shape=(H, d3, hidden)), _p(w2_k, "w2_k", True, f32, shape=(H, hidden, mout)))
    return ws, hidden, mout


def _score_outputs(geom, scores, probs, q_desc, k_desc, k_bound, topk, idx):
    torch = _torch()
    B, H, nt = geom.batch, geom.heads, geom.n_tiles
    rows = B * H * nt
    return (_p(scores, "scores", True, torch.float32, rows * nt), _p(probs, "probs", True, torch.float32, rows * nt),
            _p(q_desc, "q_desc", True, torch.float32, rows * 3 * geom.head_dim),
            _p(k_desc, "k_desc", True, torch.float32, rows * 3 * geom.head_dim),
            _k_bound(geom, k_bound, "k_bound"), _p(idx, "idx", True, torch.int32, rows * max(int(topk), 0)))


def _k_bound(geom, t, name):
    """Checked pointer of a per-key-tile bound array [B, H, n_t] float32, or None."""
    return _p(t, name, True, _torch().float32, geom.batch * geom.heads * geom.n_tiles)


def veda_trippool_score(geom, q_tiled, k_tiled, w1_q, w2_q, w1_k=None, w2_k=None, score_scale=0.125,
                        scores=None, probs=None, q_desc=None, k_desc=None, topk=0, idx=None, workspace=None,
                        stream=None, k_bound=None):
    """k_bound: optional [B, H, n_t] float32 output, each key tile's bound on its key-row
    norms (from its max and min descriptors), which the attention calls take."""
    w1_k = w1_q if w1_k is None else w1_k
    w2_k = w2_q if w2_k is None else w2_k
    dt = _elem_dtype(q_tiled)
    n = _tiled_numel(geom)
    qp, kp = _p(q_tiled, "q_tiled", True, dt, n), _p(k_tiled, "k_tiled", True, dt, n)
    (a, b, c, e), hidden, mout = _weights(geom, w1_q, w2_q, w1_k, w2_k)
    outs = _score_outputs(geom, scores, probs, q_desc, k_desc, k_bound, topk, idx)
    _call("veda_trippool_score",
        geom.ref, _dtype_code(q_tiled), qp, kp, a, b, c, e, hidden, mout, float(score_scale), *outs[:5], int(topk),
        outs[5], _p(workspace, "workspace"), _ws(workspace), _stream(stream))


def veda_topk_mask(scores, k, idx, mask=None, stream=None):
    """scores: [..., n_cols] float32 contiguous; idx: [..., k] int32; mask: [..., n_cols] uint8."""
    torch = _torch()
    n_cols = int(scores.shape[-1])
    rows = scores.numel() // max(n_cols, 1)
    sp = _p(scores, "scores", True, torch.float32)
    _call("veda_topk_mask", rows, n_cols, sp, int(k),
                                                   _p(idx, "idx", True, torch.int32, rows * int(k)),
                                                   _p(mask, "mask", True, torch.uint8, rows * n_cols), _stream(stream))


def _kv_idx(geom, kv_idx, k):
    """Checked pointer of a kept-tile list [B, H, n_t, k]: its last dimension must be k."""
    if kv_idx is None:
        return None
    if kv_idx.dim() < 1 or int(kv_idx.shape[-1]) != int(k):
        raise VedaError(f"kv_idx: last dimension {tuple(kv_idx.shape)[-1:]} does not match k = {k}")
    return _p(kv_idx, "kv_idx", True, _torch().int32, geom.batch * geom.heads * geom.n_tiles * int(k))


def veda_sparse_attn_fwd(geom, q_tiled, k_tiled, v_tiled, kv_idx, k, softmax_scale, o_tiled, lse=None,
                         v_layout=ROWS, stream=None, k_bound=None):
    """v_tiled holds V in v_layout: COLS (channel-major tiles) or ROWS (tile-major, like Q
    and K).  k_bound: the scoring call's [B, H, n_t] key-tile norm bounds of this K, or None
    (running softmax maximum)."""
    if v_layout not in (COLS, ROWS):
        raise VedaError("v_layout must be COLS or ROWS (a raster V goes to veda_sparse_attn_fwd_raster)")
    dt = _elem_dtype(q_tiled)
    n = _tiled_numel(geom)
    _call("veda_sparse_attn_fwd",
        geom.ref, _dtype_code(q_tiled), _p(q_tiled, "q_tiled", True, dt, n), _p(k_tiled, "k_tiled", True, dt, n),
        _p(v_tiled, "v_tiled", True, dt, n), int(v_layout), _kv_idx(geom, kv_idx, k), _k_bound(geom, k_bound, "k_bound"),
        int(k), float(softmax_scale),
        _p(o_tiled, "o_tiled", True, dt, n),
        _p(lse, "lse", True, _torch().float32, geom.batch * geom.heads * geom.n_tiled), _stream(stream))


def veda_oracle_tilemap_workspace_bytes(geom, n_sel):
    return int(lib().veda_oracle_tilemap_workspace_bytes(geom.ref, int(n_sel)))


def _tilemap_io(geom, q_tiles, n_sel, tilemap, lse):
    torch = _torch()
    bh = geom.batch * geom.heads
    return (_p(q_tiles, "q_tiles", True, torch.int32, bh * int(n_sel)),
            _p(tilemap, "tilemap", True, torch.float32, bh * int(n_sel) * geom.n_tiles),
            _p(lse, "lse", True, torch.float32, bh * int(n_sel) * geom.tile))


def veda_oracle_tilemap(geom, q_tiled, k_tiled, softmax_scale, q_tiles, n_sel, tilemap, lse=None, workspace=None,
                        stream=None):
    dt = _elem_dtype(q_tiled)
    n = _tiled_numel(geom)
    qt, tm, lp = _tilemap_io(geom, q_tiles, n_sel, tilemap, lse)
    _call("veda_oracle_tilemap",
        geom.ref, _dtype_code(q_tiled), _p(q_tiled, "q_tiled", True, dt, n), _p(k_tiled, "k_tiled", True, dt, n),
        float(softmax_scale), qt, int(n_sel), tm, lp, _p(workspace, "workspace"), _ws(workspace), _stream(stream))


def veda_tiled_tokens(geom, dtype_code):
    """Rows per head of the tiled layouts, as the library computes them."""
    n = int(lib().veda_tiled_tokens(geom.ref, int(dtype_code)))
    if n < 0:
        _check("veda_tiled_tokens", n)
    return n


def veda_head_tiles(geom, dtype_code, head):
    n = int(lib().veda_head_tiles(geom.ref, int(dtype_code), int(head)))
    if n < 0:
        _check("veda_head_tiles", n)
    return n


def veda_head_sq_error_workspace_bytes(batch, n_tokens, heads):
    return int(lib().veda_head_sq_error_workspace_bytes(int(batch), int(n_tokens), int(heads)))


def veda_head_sq_error(a, b, err, ref_sq=None, workspace=None, err_batch_sum=None, stream=None):
    """a, b: contiguous raster [B, N, H, d] tensors of one dtype; err (and ref_sq): [B, H]
    float32, written with sum (a - b)^2 (and sum b^2) per (batch, head); err_batch_sum: [H]
    float32, written with the sum of err over the batch.  workspace: a device buffer of at
    least veda_head_sq_error_workspace_bytes(B, N, H) bytes; allocated on a's device when
    None."""
    torch = _torch()
    if a.shape != b.shape or a.dtype != b.dtype or a.dim() != 4:
        raise VedaError("a and b must be [B, N, H, d] tensors of one shape and dtype")
    B, N, H, d = (int(x) for x in a.shape)
    outs = (_p(err, "err", True, torch.float32, B * H), _p(err_batch_sum, "err_batch_sum", True, torch.float32, H),
            _p(ref_sq, "ref_sq", True, torch.float32, B * H))
    if workspace is None:
        workspace = torch.empty(max(1, veda_head_sq_error_workspace_bytes(B, N, H)), dtype=torch.uint8,
                                device=a.device)
    _call("veda_head_sq_error",
        B, N, H, d, _dtype_code(a), _p(a, "a"), _p(b, "b"), *outs, _p(workspace, "workspace"), _ws(workspace),
        _stream(stream))


def veda_distill_workspace_bytes(geom, n_sel):
    return int(lib().veda_distill_workspace_bytes(geom.ref, int(n_sel)))


def veda_distill_step(geom, q_tiled, k_tiled, w1, w2, q_tiles, target, loss, dw1, dw2, score_scale=0.125, lr=0.0,
                      workspace=None, stream=None):
    """One KL distillation step of the per-head estimator (shared Q/K MLP).  w1, w2 are
    updated in place when lr != 0; loss [1], dw1, dw2 are outputs."""
    torch = _torch()
    dt = _elem_dtype(q_tiled)
    n = _tiled_numel(geom)
    (a, b, _, _), hidden, mout = _weights(geom, w1, w2, w1, w2)
    n_sel = int(q_tiles.shape[-1])
    bh = geom.batch * geom.heads
    _call("veda_distill_step",
        geom.ref, _dtype_code(q_tiled), _p(q_tiled, "q_tiled", True, dt, n), _p(k_tiled, "k_tiled", True, dt, n), a,
        b, hidden, mout, float(score_scale), _p(q_tiles, "q_tiles", True, torch.int32, bh * n_sel), n_sel,
        _p(target, "target", True, torch.float32, bh * n_sel * geom.n_tiles),
        _p(loss, "loss", True, torch.float32, 1), _p(dw1, "dw1", True, torch.float32, shape=tuple(w1.shape)),
        _p(dw2, "dw2", True, torch.float32, shape=tuple(w2.shape)), float(lr), _p(workspace, "workspace"),
        _ws(workspace), _stream(stream))


def _raster_strides(*ts):
    """Shared element strides (b, n, h) of raster [B, N, H, d] tensors (d contiguous)."""
    st = tuple(int(x) for x in ts[0].stride()[:3])
    for t in ts:
        if t.dim() != 4 or t.stride(-1) != 1 or tuple(int(x) for x in t.stride()[:3]) != st:
            raise VedaError("raster operands must be [B, N, H, d] with d contiguous and one set of strides")
    return st


def _raster(geom, t, name, dt):
    """Checked pointer of a raster [B, N, H, d] operand (strided; last dim contiguous)."""
    return _p(t, name, False, dt, shape=_raster_shape(geom))


def _k_operand(geom, q, k, k_layout, *others):
    """Strides shared by the raster operands, and the checked K pointer."""
    dt = _elem_dtype(q)
    if k_layout == RASTER:
        return _raster_strides(q, k, *others), _raster(geom, k, "k", dt)
    if k_layout != ROWS:
        raise VedaError("k_layout must be RASTER or ROWS")
    return _raster_strides(q, *others), _p(k, "k", True, dt, _tiled_numel(geom))


def _k_tiled_out(geom, q, t):
    return _p(t, "k_tiled_out", True, _elem_dtype(q), _tiled_numel(geom))


def _v_copy(geom, q, v, v_tiled_out):
    """Checked pointers of the V copy of the raster scoring calls: both or neither."""
    if (v is None) != (v_tiled_out is None):
        raise VedaError("v and v_tiled_out go together")
    if v is None:
        return None, None
    dt = _elem_dtype(q)
    return _raster(geom, v, "v", dt), _p(v_tiled_out, "v_tiled_out", True, dt, _tiled_numel(geom))


def veda_trippool_score_raster(geom, q, k, w1_q, w2_q, w1_k=None, w2_k=None, score_scale=0.125, scores=None,
                               probs=None, q_desc=None, k_desc=None, topk=0, idx=None, workspace=None,
                               k_layout=RASTER, k_tiled_out=None, v=None, v_tiled_out=None, stream=None,
                               k_bound=None):
    """veda_trippool_score on raster Q [B, N, H, d] (read through each head's tiling); K
    raster too, or tile-major with k_layout=ROWS.  With a raster K, k_tiled_out (if given)
    receives K's tile-major copy, written while K is pooled; with a raster V (strides of Q),
    v_tiled_out receives V's tile-major copy from the same launch."""
    w1_k = w1_q if w1_k is None else w1_k
    w2_k = w2_q if w2_k is None else w2_k
    rs, kp = _k_operand(geom, q, k, k_layout, *(() if v is None else (v,)))
    qp = _raster(geom, q, "q", _elem_dtype(q))
    (a, b, c, e), hidden, mout = _weights(geom, w1_q, w2_q, w1_k, w2_k)
    outs = _score_outputs(geom, scores, probs, q_desc, k_desc, k_bound, topk, idx)
    vc = _v_copy(geom, q, v, v_tiled_out)
    _call("veda_trippool_score_raster",
          geom.ref, _dtype_code(q), qp, kp, int(k_layout), *rs, a, b, c, e, hidden, mout, float(score_scale),
          *outs[:5], int(topk), outs[5], _k_tiled_out(geom, q, k_tiled_out), *vc, _p(workspace, "workspace"),
          _ws(workspace), _stream(stream))


def veda_sparse_attn_fwd_raster(geom, q, k, v, kv_idx, kk, softmax_scale, o, lse=None, k_layout=RASTER,
                                v_layout=ROWS, stream=None, k_bound=None):
    """veda_sparse_attn_fwd with raster Q and output O [B, N, H, d]; K raster or tile-major
    (k_layout=ROWS); V channel-major tiled (COLS), tile-major (ROWS) or raster (RASTER, with
    the strides of Q); O with strides of its own; lse [B, H, N] in raster token order."""
    dt = _elem_dtype(q)
    if v_layout == RASTER:
        rs, kp = _k_operand(geom, q, k, k_layout, v)
        vp = _raster(geom, v, "v", dt)
    elif v_layout in (COLS, ROWS):
        rs, kp = _k_operand(geom, q, k, k_layout)
        vp = _p(v, "v", True, dt, _tiled_numel(geom))
    else:
        raise VedaError("v_layout must be COLS, ROWS or RASTER")
    op = _raster(geom, o, "o", dt)
    _call("veda_sparse_attn_fwd_raster",
        geom.ref, _dtype_code(q), _raster(geom, q, "q", dt), kp, int(k_layout), *rs,
        vp, int(v_layout), _kv_idx(geom, kv_idx, kk), _k_bound(geom, k_bound, "k_bound"), int(kk),
        float(softmax_scale), op, *_raster_strides(o),
        _p(lse, "lse", True, _torch().float32, geom.batch * geom.heads * geom.n_tokens), _stream(stream))


def veda_oracle_tilemap_raster(geom, q, k, softmax_scale, q_tiles, n_sel, tilemap, lse=None, workspace=None,
                               k_layout=RASTER, stream=None):
    """veda_oracle_tilemap on raster Q [B, N, H, d]; K raster or tile-major (k_layout=ROWS)."""
    rs, kp = _k_operand(geom, q, k, k_layout)
    qt, tm, lp = _tilemap_io(geom, q_tiles, n_sel, tilemap, lse)
    _call("veda_oracle_tilemap_raster",
        geom.ref, _dtype_code(q), _raster(geom, q, "q", _elem_dtype(q)), kp, int(k_layout), *rs,
        float(softmax_scale), qt, int(n_sel), tm, lp, _p(workspace, "workspace"), _ws(workspace), _stream(stream))


def veda_trippool_score_raster_noalloc(geom, q, k, w1_q, w2_q, w1_k=None, w2_k=None, score_scale=0.125,
                                       scores=None, probs=None, q_desc=None, k_desc=None, topk=0, idx=None,
                                       k_layout=RASTER, k_tiled_out=None, v=None, v_tiled_out=None, stream=None,
                                       k_bound=None):
    """veda_trippool_score_raster with no workspace: the library's static scratch holds the
    MLP outputs (B * H * n_t <= 65536 tiles; calls that overlap on one GPU race)."""
    w1_k = w1_q if w1_k is None else w1_k
    w2_k = w2_q if w2_k is None else w2_k
    rs, kp = _k_operand(geom, q, k, k_layout, *(() if v is None else (v,)))
    qp = _raster(geom, q, "q", _elem_dtype(q))
    (a, b, c, e), hidden, mout = _weights(geom, w1_q, w2_q, w1_k, w2_k)
    outs = _score_outputs(geom, scores, probs, q_desc, k_desc, k_bound, topk, idx)
    vc = _v_copy(geom, q, v, v_tiled_out)
    _call("veda_trippool_score_raster_noalloc", geom.ref, _dtype_code(q), qp, kp, int(k_layout), *rs, a, b, c, e,
          hidden, mout, float(score_scale), *outs[:5], int(topk), outs[5], _k_tiled_out(geom, q, k_tiled_out), *vc,
          _stream(stream))
