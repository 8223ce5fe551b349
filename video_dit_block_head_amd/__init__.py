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
            "veda_trippool_score": (i32, [G, i32, vp, vp, vp, vp, vp, vp, i32, i32, f32, vp, vp, vp, vp, i32, vp,
                                          vp, sz, vp]),
            "veda_topk_mask": (i32, [i64, i32, vp, i32, vp, vp, vp]),
            "veda_sparse_attn_fwd": (i32, [G, i32, vp, vp, vp, vp, i32, f32, vp, vp, vp]),
            "veda_oracle_tilemap_workspace_bytes": (sz, [G, i32]),
            "veda_oracle_tilemap": (i32, [G, i32, vp, vp, f32, vp, i32, vp, vp, vp, sz, vp]),
            "veda_head_sq_error_workspace_bytes": (sz, [i32, i32, i32]),
            "veda_head_sq_error": (i32, [i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp]),
            "veda_distill_workspace_bytes": (sz, [G, i32]),
            "veda_trippool_score_raster": (i32, [G, i32, vp, vp, i32, i64, i64, i64, vp, vp, vp, vp, i32, i32, f32,
                                                 vp, vp, vp, vp, i32, vp, vp, sz, vp]),
            "veda_sparse_attn_fwd_raster": (i32, [G, i32, vp, vp, i32, i64, i64, i64, vp, vp, i32, f32, vp, vp,
                                                  vp]),
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


def _p(t, name, need_contig=True):
    if t is None:
        return None
    if not t.is_cuda:
        raise VedaError(f"{name} must be a GPU tensor")
    if need_contig and not t.is_contiguous():
        raise VedaError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def version():
    return lib().veda_version().decode()


def veda_tile_gather(geom, raster, tiled, layout=ROWS, inverse=False, stream=None):
    """raster: [B, N, H, d] tensor (any strides, last dim contiguous); tiled: contiguous
    tensor of B*H*N*d elements in `layout`.  inverse=True scatters tiled -> raster."""
    if raster.stride(-1) != 1:
        raise VedaError("raster: last dimension must be contiguous")
    _check("veda_tile_gather", lib().veda_tile_gather(
        geom.ref, _dtype_code(raster), _p(raster, "raster", False), raster.stride(0), raster.stride(1),
        raster.stride(2), _p(tiled, "tiled"), int(layout), int(bool(inverse)), _stream(stream)))


def veda_trippool_workspace_bytes(geom, mlp_hidden, mlp_out):
    return int(lib().veda_trippool_workspace_bytes(geom.ref, int(mlp_hidden), int(mlp_out)))


def veda_trippool_score(geom, q_tiled, k_tiled, w1_q, w2_q, w1_k=None, w2_k=None, score_scale=0.125,
                        scores=None, probs=None, q_desc=None, k_desc=None, topk=0, idx=None, workspace=None,
                        stream=None):
    w1_k = w1_q if w1_k is None else w1_k
    w2_k = w2_q if w2_k is None else w2_k
    hidden, mout = int(w1_q.shape[-1]), int(w2_q.shape[-1])
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("veda_trippool_score", lib().veda_trippool_score(
        geom.ref, _dtype_code(q_tiled), _p(q_tiled, "q_tiled"), _p(k_tiled, "k_tiled"), _p(w1_q, "w1_q"),
        _p(w2_q, "w2_q"), _p(w1_k, "w1_k"), _p(w2_k, "w2_k"), hidden, mout, float(score_scale),
        _p(scores, "scores"), _p(probs, "probs"), _p(q_desc, "q_desc"), _p(k_desc, "k_desc"), int(topk),
        _p(idx, "idx"), _p(workspace, "workspace"), ws_bytes, _stream(stream)))


def veda_topk_mask(scores, k, idx, mask=None, stream=None):
    """scores: [..., n_cols] float32 contiguous; idx: [..., k] int32; mask: [..., n_cols] uint8."""
    n_cols = int(scores.shape[-1])
    rows = scores.numel() // n_cols
    _check("veda_topk_mask", lib().veda_topk_mask(rows, n_cols, _p(scores, "scores"), int(k), _p(idx, "idx"),
                                                   _p(mask, "mask"), _stream(stream)))


def veda_sparse_attn_fwd(geom, q_tiled, k_tiled, v_tiled, kv_idx, k, softmax_scale, o_tiled, lse=None,
                         stream=None):
    _check("veda_sparse_attn_fwd", lib().veda_sparse_attn_fwd(
        geom.ref, _dtype_code(q_tiled), _p(q_tiled, "q_tiled"), _p(k_tiled, "k_tiled"), _p(v_tiled, "v_tiled"),
        _p(kv_idx, "kv_idx"), int(k), float(softmax_scale), _p(o_tiled, "o_tiled"), _p(lse, "lse"),
        _stream(stream)))


def veda_oracle_tilemap_workspace_bytes(geom, n_sel):
    return int(lib().veda_oracle_tilemap_workspace_bytes(geom.ref, int(n_sel)))


def veda_oracle_tilemap(geom, q_tiled, k_tiled, softmax_scale, q_tiles, n_sel, tilemap, lse=None, workspace=None,
                        stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("veda_oracle_tilemap", lib().veda_oracle_tilemap(
        geom.ref, _dtype_code(q_tiled), _p(q_tiled, "q_tiled"), _p(k_tiled, "k_tiled"), float(softmax_scale),
        _p(q_tiles, "q_tiles"), int(n_sel), _p(tilemap, "tilemap"), _p(lse, "lse"), _p(workspace, "workspace"),
        ws_bytes, _stream(stream)))


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


def veda_head_sq_error(a, b, err, ref_sq=None, workspace=None, stream=None):
    """a, b: contiguous raster [B, N, H, d] tensors of one dtype; err (and ref_sq): [B, H]
    float32, written with sum (a - b)^2 (and sum b^2) per (batch, head).  workspace: a device
    buffer of at least veda_head_sq_error_workspace_bytes(B, N, H) bytes; allocated on a's
    device when None."""
    if a.shape != b.shape or a.dtype != b.dtype or a.dim() != 4:
        raise VedaError("a and b must be [B, N, H, d] tensors of one shape and dtype")
    B, N, H, d = (int(x) for x in a.shape)
    if workspace is None:
        import torch
        workspace = torch.empty(max(1, veda_head_sq_error_workspace_bytes(B, N, H)), dtype=torch.uint8,
                                device=a.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check("veda_head_sq_error", lib().veda_head_sq_error(
        B, N, H, d, _dtype_code(a), _p(a, "a"), _p(b, "b"), _p(err, "err"), _p(ref_sq, "ref_sq"),
        _p(workspace, "workspace"), ws_bytes, _stream(stream)))


def veda_distill_workspace_bytes(geom, n_sel):
    return int(lib().veda_distill_workspace_bytes(geom.ref, int(n_sel)))


def veda_distill_step(geom, q_tiled, k_tiled, w1, w2, q_tiles, target, loss, dw1, dw2, score_scale=0.125, lr=0.0,
                      workspace=None, stream=None):
    """One KL distillation step of the per-head estimator (shared Q/K MLP).  w1, w2 are
    updated in place when lr != 0; loss [1], dw1, dw2 are outputs."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("veda_distill_step", lib().veda_distill_step(
        geom.ref, _dtype_code(q_tiled), _p(q_tiled, "q_tiled"), _p(k_tiled, "k_tiled"), _p(w1, "w1"), _p(w2, "w2"),
        int(w1.shape[-1]), int(w2.shape[-1]), float(score_scale), _p(q_tiles, "q_tiles"), int(q_tiles.shape[-1]),
        _p(target, "target"), _p(loss, "loss"), _p(dw1, "dw1"), _p(dw2, "dw2"), float(lr), _p(workspace, "workspace"),
        ws_bytes, _stream(stream)))


def _raster_strides(*ts):
    """Shared element strides (b, n, h) of raster [B, N, H, d] tensors (d contiguous)."""
    st = tuple(int(x) for x in ts[0].stride()[:3])
    for t in ts:
        if t.dim() != 4 or t.stride(-1) != 1 or tuple(int(x) for x in t.stride()[:3]) != st:
            raise VedaError("raster operands must be [B, N, H, d] with d contiguous and one set of strides")
    return st


def _k_operand(q, k, k_layout, *others):
    """Strides shared by the raster operands, and the checked K pointer."""
    if k_layout == RASTER:
        return _raster_strides(q, k, *others), _p(k, "k", False)
    if k_layout != ROWS:
        raise VedaError("k_layout must be RASTER or ROWS")
    return _raster_strides(q, *others), _p(k, "k")


def veda_trippool_score_raster(geom, q, k, w1_q, w2_q, w1_k=None, w2_k=None, score_scale=0.125, scores=None,
                               probs=None, q_desc=None, k_desc=None, topk=0, idx=None, workspace=None,
                               k_layout=RASTER, stream=None):
    """veda_trippool_score on raster Q [B, N, H, d] (read through each head's tiling); K
    raster too, or tile-major with k_layout=ROWS."""
    w1_k = w1_q if w1_k is None else w1_k
    w2_k = w2_q if w2_k is None else w2_k
    rs, kp = _k_operand(q, k, k_layout)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("veda_trippool_score_raster", lib().veda_trippool_score_raster(
        geom.ref, _dtype_code(q), _p(q, "q", False), kp, int(k_layout), *rs, _p(w1_q, "w1_q"), _p(w2_q, "w2_q"),
        _p(w1_k, "w1_k"), _p(w2_k, "w2_k"), int(w1_q.shape[-1]), int(w2_q.shape[-1]), float(score_scale),
        _p(scores, "scores"), _p(probs, "probs"), _p(q_desc, "q_desc"), _p(k_desc, "k_desc"), int(topk),
        _p(idx, "idx"), _p(workspace, "workspace"), ws_bytes, _stream(stream)))


def veda_sparse_attn_fwd_raster(geom, q, k, v_cols, kv_idx, kk, softmax_scale, o, lse=None, k_layout=RASTER,
                                stream=None):
    """veda_sparse_attn_fwd with raster Q and output O [B, N, H, d]; K raster or tile-major
    (k_layout=ROWS); V channel-major tiled; lse [B, H, N] in raster token order."""
    rs, kp = _k_operand(q, k, k_layout, o)
    _check("veda_sparse_attn_fwd_raster", lib().veda_sparse_attn_fwd_raster(
        geom.ref, _dtype_code(q), _p(q, "q", False), kp, int(k_layout), *rs, _p(v_cols, "v_cols"),
        _p(kv_idx, "kv_idx"), int(kk), float(softmax_scale), _p(o, "o", False), _p(lse, "lse"), _stream(stream)))


def veda_oracle_tilemap_raster(geom, q, k, softmax_scale, q_tiles, n_sel, tilemap, lse=None, workspace=None,
                               k_layout=RASTER, stream=None):
    """veda_oracle_tilemap on raster Q [B, N, H, d]; K raster or tile-major (k_layout=ROWS)."""
    rs, kp = _k_operand(q, k, k_layout)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("veda_oracle_tilemap_raster", lib().veda_oracle_tilemap_raster(
        geom.ref, _dtype_code(q), _p(q, "q", False), kp, int(k_layout), *rs, float(softmax_scale),
        _p(q_tiles, "q_tiles"), int(n_sel), _p(tilemap, "tilemap"), _p(lse, "lse"), _p(workspace, "workspace"),
        ws_bytes, _stream(stream)))
