"""The C ABI on the CPU: the library loads, exports every entry point include/veda.h
declares, and rejects bad arguments with the documented status before touching the GPU.

No call here has arguments that pass validation, so nothing is ever launched (the fake
device addresses below are never dereferenced).  The module skips itself wherever a GPU
is visible, so that a regression in a check could never launch a kernel on a fake address."""
import ctypes
import os
import re

import pytest

import video_dit_block_head_amd as V
from conftest import ROOT, gpu_visible

pytestmark = pytest.mark.skipif(gpu_visible(), reason="fake device addresses: CPU-only (no GPU visible)")

HEADER = os.path.join(ROOT, "include", "veda.h")
OK, NULL, SHAPE, DTYPE, UNSUP, WS, ALIGN = 0, -1, -2, -3, -4, -5, -6
A = ctypes.c_void_p(0x10000)       # aligned fake device address (never dereferenced)
B_ = ctypes.c_void_p(0x20000)
MIS = ctypes.c_void_p(0x10008)     # misaligned


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(veda_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(V.LIB_PATH):
        pytest.skip("libveda.so not built")
    return V.lib()


def test_exports_every_declared_symbol(L):
    syms = declared_symbols()
    assert len(syms) == 20, syms
    for s in syms:
        assert hasattr(L, s), s


def test_status_strings(L):
    for code in (OK, NULL, SHAPE, DTYPE, UNSUP, WS, ALIGN, -7):
        assert len(L.veda_status_str(code)) > 0
    assert b"gfx950" in L.veda_version()
    assert L.veda_last_hip_error() == 0


def geom(d=128, tile=128, grid=(8, 16, 32), shapes=((2, 8, 8),) * 2, heads=None, batch=1):
    heads = len(shapes) if heads is None else heads
    return V.Geom(batch, heads, d, grid, tile, shapes)


def gather(L, g, dt=V.BF16, raster=A, tiled=B_, strides=(4096 * 2 * 128, 2 * 128, 128), layout=0, inverse=0):
    return L.veda_tile_gather(g.ref if g is not None else None, dt, raster, *strides, tiled, layout, inverse, None)


def test_empty_geometries_are_refused(L):
    """An empty batch, head set or grid is a shape error on every geometry-taking call,
    returned before anything is launched (the top-k call alone takes rows = 0 as nothing to do)."""
    for kw in (dict(batch=0), dict(heads=0, shapes=((2, 8, 8),))):
        g = geom(**kw)
        assert L.veda_tiled_tokens(g.ref, V.BF16) == SHAPE
        assert L.veda_sparse_attn_fwd(g.ref, V.BF16, A, A, A, V.ROWS, A, None, 1, 0.088, A, None, None) == SHAPE
        assert gather(L, g) == SHAPE
    g = geom(grid=(0, 16, 32))
    assert L.veda_tiled_tokens(g.ref, V.BF16) == SHAPE
    assert L.veda_oracle_tilemap(g.ref, V.BF16, A, A, 0.088, A, 1, A, None, A, 1 << 40, None) == SHAPE


def test_padded_tile_counts(L):
    """Tiles per head on the grid padded up to whole tiles, and the tiled rows per head."""
    g = geom(grid=(20, 48, 80), shapes=((8, 4, 4), (2, 8, 8), (1, 8, 16)))
    assert [L.veda_head_tiles(g.ref, V.BF16, h) for h in range(3)] == [3 * 12 * 20, 600, 600]
    assert L.veda_tiled_tokens(g.ref, V.BF16) == 720 * 128
    assert [g.head_tiles(h) for h in range(3)] == [720, 600, 600] and g.padded and g.n_tiled == 720 * 128
    g = geom(grid=(8, 16, 31), shapes=((1, 8, 16),))          # w = 31: two tiles of 16 along w
    assert L.veda_head_tiles(g.ref, V.BF16, 0) == 8 * 2 * 2 and L.veda_tiled_tokens(g.ref, V.BF16) == 32 * 128
    g = geom()
    assert L.veda_tiled_tokens(g.ref, V.BF16) == 4096 and not g.padded and g.n_tiled == g.n_tokens
    assert L.veda_head_tiles(g.ref, V.BF16, 2) == SHAPE
    assert L.veda_tiled_tokens(geom(d=64).ref, V.BF16) == UNSUP
    assert L.veda_tiled_tokens(geom(d=64, tile=64, grid=(20, 8, 8), shapes=((8, 4, 2),)).ref, V.F32) == UNSUP


def test_padded_rejected_where_unsupported(L):
    """A padded tiling goes through the raster calls with K and V tiled (the raster attention
    and tile map refuse a raster K, the attention a raster V), and the all-tiles tile map
    needs an explicit list; each refusal comes before anything is launched."""
    g = geom(grid=(20, 16, 32), shapes=((8, 4, 4), (2, 8, 8)))
    n_t = g.n_tiles                                           # 3 * 4 * 8 = 96 > 80 (dividing head)
    st = (g.n_tokens * 2 * 128, 2 * 128, 128)
    RAS, big = V.RASTER, 1 << 40
    assert L.veda_sparse_attn_fwd_raster(g.ref, V.BF16, A, A, RAS, *st, A, V.COLS, A, None, 4, 0.088, A, *st, None,
                                         None) == UNSUP
    assert L.veda_sparse_attn_fwd_raster(g.ref, V.BF16, A, A, V.ROWS, *st, A, RAS, A, None, 4, 0.088, A, *st, None,
                                         None) == UNSUP                      # a raster V, likewise
    assert L.veda_oracle_tilemap_raster(g.ref, V.BF16, A, A, RAS, *st, 0.088, A, 4, A, None, A, big, None) == UNSUP
    assert L.veda_oracle_tilemap_raster(g.ref, V.BF16, A, A, V.ROWS, *st, 0.088, None, n_t, A, None, A, big,
                                        None) == SHAPE
    assert L.veda_oracle_tilemap(g.ref, V.BF16, A, A, 0.088, None, n_t, A, None, A, big, None) == SHAPE
    # k may not exceed the smallest per-head tile count (80 here), on every path
    assert L.veda_sparse_attn_fwd(g.ref, V.BF16, A, A, A, V.COLS, A, None, 81, 0.088, A, None, None) == SHAPE
    assert L.veda_sparse_attn_fwd_raster(g.ref, V.BF16, A, A, V.ROWS, *st, A, V.COLS, A, None, 81, 0.088, A, *st,
                                         None, None) == SHAPE
    assert L.veda_trippool_score(g.ref, V.BF16, A, A, A, A, A, A, 256, 64, 0.125, None, None, None, None, None, 81,
                                 A, A, big, None) == SHAPE
    assert L.veda_trippool_score_raster(g.ref, V.BF16, A, A, RAS, *st, A, A, A, A, 256, 64, 0.125, None, None, None,
                                        None, None, 81, A, None, None, None, A, big, None) == SHAPE
    assert L.veda_distill_step(g.ref, V.BF16, A, A, A, A, 256, 64, 0.125, A, n_t + 1, A, A, A, A, 0.0, A, big,
                               None) == SHAPE


def test_gather_validation(L):
    assert gather(L, None) == NULL
    assert gather(L, geom(), raster=None) == NULL
    assert gather(L, geom(), dt=7) == DTYPE
    assert gather(L, geom(d=64)) == UNSUP                      # bf16 needs d = 128
    assert gather(L, geom(d=128, tile=64, shapes=((1, 8, 8),) * 2), dt=V.F32) == UNSUP
    assert gather(L, geom(shapes=((2, 8, 4), (2, 8, 8)))) == SHAPE    # product != tile
    # padded tilings (a shape that does not divide the grid) are bf16-only
    assert gather(L, geom(d=64, tile=64, grid=(20, 8, 8), shapes=((8, 4, 2),)), dt=V.F32) == UNSUP
    assert gather(L, geom(), raster=MIS) == ALIGN
    assert gather(L, geom(), strides=(4096 * 256, 260, 128)) == ALIGN
    assert gather(L, geom(), layout=1, inverse=1) == UNSUP
    assert gather(L, geom(), layout=5) == SHAPE
    assert gather(L, geom(heads=200, shapes=((2, 8, 8),) * 200)) == SHAPE


def score(L, g, topk=6, idx=B_, scores=None, ws=A, ws_bytes=1 << 30, hidden=256, out=64):
    return L.veda_trippool_score(g.ref, V.BF16, A, A, A, A, A, A, hidden, out, 0.125, scores, None, None, None, None,
                                 topk, idx, ws, ws_bytes, None)


def test_score_validation(L):
    g = geom()
    assert score(L, g, topk=0, idx=None) == NULL               # nothing requested
    assert score(L, g, topk=0, idx=B_) == SHAPE
    assert score(L, g, topk=6, idx=None) == NULL
    assert score(L, g, topk=33) == SHAPE                       # n_t = 32
    assert score(L, g, hidden=512) == UNSUP
    assert score(L, g, hidden=128) == UNSUP
    assert score(L, g, out=128) == UNSUP
    assert score(L, g, ws=None) == WS
    need = L.veda_trippool_workspace_bytes(g.ref, 256, 64)
    assert need > 0
    assert score(L, g, ws_bytes=need - 1) == WS
    assert score(L, g, idx=MIS) == ALIGN
    big = geom(grid=(40, 48, 160), shapes=((2, 8, 8),))      # n_t = 2400 > fused-score limit
    assert score(L, big, topk=10) == UNSUP


def test_topk_validation(L):
    assert L.veda_topk_mask(4, 10, A, 0, B_, None, None) == SHAPE
    assert L.veda_topk_mask(4, 10, A, 11, B_, None, None) == SHAPE
    assert L.veda_topk_mask(4, 5000, A, 3, B_, None, None) == SHAPE
    assert L.veda_topk_mask(-1, 10, A, 3, B_, None, None) == SHAPE
    assert L.veda_topk_mask(4, 10, None, 3, B_, None, None) == NULL
    assert L.veda_topk_mask(4, 10, A, 3, None, None, None) == NULL
    assert L.veda_topk_mask(4, 10, ctypes.c_void_p(0x10002), 3, B_, None, None) == ALIGN
    assert L.veda_topk_mask(0, 10, A, 3, B_, None, None) == OK   # nothing to do: nothing launched


def test_attn_validation(L):
    g = geom()
    f = L.veda_sparse_attn_fwd
    C = V.COLS
    assert f(g.ref, V.BF16, A, A, None, C, A, None, 4, 0.088, A, None, None) == NULL
    assert f(g.ref, V.BF16, A, A, A, C, A, None, 0, 0.088, A, None, None) == SHAPE
    assert f(g.ref, V.BF16, A, A, A, C, A, None, 33, 0.088, A, None, None) == SHAPE
    assert f(g.ref, V.BF16, A, A, A, C, A, None, 4, 0.088, MIS, None, None) == ALIGN
    assert f(g.ref, V.BF16, A, A, A, C, A, None, 4, 0.088, A, MIS, None) == ALIGN
    assert f(geom(d=64).ref, V.BF16, A, A, A, C, A, None, 4, 0.088, A, None, None) == UNSUP
    assert f(g.ref, V.BF16, A, A, A, C, A, MIS, 4, 0.088, A, None, None) == ALIGN      # key-tile bounds
    for bad in (0.0, -0.088, float("inf"), float("nan")):                               # softmax scale
        assert f(g.ref, V.BF16, A, A, A, C, A, None, 4, bad, A, None, None) == SHAPE
        assert L.veda_oracle_tilemap(g.ref, V.BF16, A, A, bad, A, 4, A, None, A, 1 << 40, None) == SHAPE


def test_key_tile_bound_pointers(L):
    """The per-key-tile norm bounds (scoring output, attention input) are checked like every
    other device pointer, in all five calls that take them."""
    g = geom()
    st = (4096 * 2 * 128, 2 * 128, 128)
    RAS, C = V.RASTER, V.COLS
    assert L.veda_sparse_attn_fwd_raster(g.ref, V.BF16, A, A, RAS, *st, A, C, A, MIS, 4, 0.088, A, *st, None,
                                         None) == ALIGN
    assert L.veda_trippool_score(g.ref, V.BF16, A, A, A, A, A, A, 256, 64, 0.125, None, None, None, None, MIS, 6,
                                 B_, A, 1 << 30, None) == ALIGN
    assert L.veda_trippool_score_raster(g.ref, V.BF16, A, A, RAS, *st, A, A, A, A, 256, 64, 0.125, None, None, None,
                                        None, MIS, 6, B_, None, None, None, A, 1 << 30, None) == ALIGN
    assert L.veda_trippool_score_raster_noalloc(g.ref, V.BF16, A, A, RAS, *st, A, A, A, A, 256, 64, 0.125, None,
                                                None, None, None, MIS, 6, B_, None, None, None, None) == ALIGN


def test_attn_v_layout_validation(L):
    """V may be channel-major or tile-major in both calls and raster in the raster call; a
    raster V in the tiled call (no strides) and an unknown layout are refused with a status,
    never computed as if V were in another layout."""
    g = geom()
    assert L.veda_sparse_attn_fwd(g.ref, V.BF16, A, A, A, V.RASTER, A, None, 4, 0.088, A, None, None) == UNSUP
    assert L.veda_sparse_attn_fwd(g.ref, V.BF16, A, A, A, 7, A, None, 4, 0.088, A, None, None) == SHAPE
    st = (4096 * 2 * 128, 2 * 128, 128)
    assert L.veda_sparse_attn_fwd_raster(g.ref, V.BF16, A, A, V.RASTER, *st, A, 7, A, None, 4, 0.088, A, *st, None,
                                         None) == SHAPE


def test_tilemap_validation(L):
    g = geom()
    f = L.veda_oracle_tilemap
    big = 1 << 40
    assert f(g.ref, V.BF16, A, A, 0.088, None, 5, A, None, A, big, None) == SHAPE   # NULL list needs n_sel = n_t
    assert f(g.ref, V.BF16, A, A, 0.088, A, 0, A, None, A, big, None) == SHAPE
    assert f(g.ref, V.BF16, A, A, 0.088, A, 33, A, None, A, big, None) == SHAPE
    assert f(g.ref, V.BF16, A, None, 0.088, A, 4, A, None, A, big, None) == NULL
    assert f(g.ref, V.BF16, A, A, 0.088, MIS, 4, A, None, A, big, None) == ALIGN
    need = L.veda_oracle_tilemap_workspace_bytes(g.ref, 4)
    assert need == 1 * 2 * 4 * 32 * 128 * 4 + 1 * 2 * 4 * 4 * 128 * 8   # row maxima, then (m, l) for <= 4 key ranges
    assert f(g.ref, V.BF16, A, A, 0.088, A, 4, A, None, None, big, None) == WS
    assert f(g.ref, V.BF16, A, A, 0.088, A, 4, A, None, A, need - 1, None) == WS


def test_binding_fails_loudly_without_gpu_tensors():
    import torch
    g = geom()
    with pytest.raises(V.VedaError):
        V.veda_topk_mask(torch.zeros(4, 10), 3, torch.zeros(4, 3, dtype=torch.int32))


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    """No fallback: with libveda.so absent, the first call raises instead of computing."""
    monkeypatch.setattr(V, "_lib", None)
    monkeypatch.setattr(V, "LIB_PATH", str(tmp_path / "libveda.so"))
    with pytest.raises(V.VedaError, match="missing"):
        V.lib()
    import torch
    with pytest.raises(V.VedaError):
        V.veda_topk_mask(torch.zeros(4, 10), 3, torch.zeros(4, 3, dtype=torch.int32))


def test_head_error_validation(L):
    f = L.veda_head_sq_error
    wsb = L.veda_head_sq_error_workspace_bytes(1, 16, 2)
    assert wsb == 1 * 2 * 1 * 8                                      # one chunk of 16 tokens per head
    assert L.veda_head_sq_error_workspace_bytes(2, 76800, 40) == 2 * 40 * 256 * 8
    assert L.veda_head_sq_error_workspace_bytes(0, 16, 2) == 0
    W = (A, wsb)
    assert f(1, 16, 2, 128, 7, A, B_, A, None, None, *W, None) == DTYPE
    assert f(0, 16, 2, 128, V.BF16, A, B_, A, None, None, *W, None) == SHAPE
    assert f(1, 16, 2, 12, V.BF16, A, B_, A, None, None, *W, None) == SHAPE     # 24-byte rows
    assert f(1, 16, 2, 128, V.BF16, None, B_, A, None, None, *W, None) == NULL
    assert f(1, 16, 2, 128, V.BF16, A, B_, None, None, None, *W, None) == NULL
    assert f(1, 16, 2, 128, V.BF16, MIS, B_, A, None, None, *W, None) == ALIGN
    assert f(1, 16, 2, 128, V.BF16, A, B_, A, ctypes.c_void_p(0x10002), None, *W, None) == ALIGN   # batch sum
    assert f(1, 16, 2, 128, V.BF16, A, B_, A, None, None, None, wsb, None) == WS
    assert f(1, 16, 2, 128, V.BF16, A, B_, A, None, None, A, wsb - 1, None) == WS


def test_raster_validation(L):
    g = geom()
    f = L.veda_sparse_attn_fwd_raster
    st = (4096 * 2 * 128, 2 * 128, 128)
    RAS = V.RASTER
    C = V.COLS
    assert f(g.ref, V.BF16, A, A, RAS, 4096 * 256, 260, 128, A, C, A, None, 4, 0.088, A, *st, None, None) == ALIGN
    assert f(g.ref, V.BF16, A, None, RAS, *st, A, C, A, None, 4, 0.088, A, *st, None, None) == NULL
    assert f(g.ref, V.BF16, MIS, A, RAS, *st, A, C, A, None, 4, 0.088, A, *st, None, None) == ALIGN
    assert f(g.ref, V.BF16, A, A, V.COLS, *st, A, C, A, None, 4, 0.088, A, *st, None, None) == SHAPE   # K layout
    # O has strides of its own, checked like Q's
    assert f(g.ref, V.BF16, A, A, RAS, *st, A, C, A, None, 4, 0.088, A, 4096 * 256, 260, 128, None, None) == ALIGN
    assert f(g.ref, V.BF16, A, A, RAS, *st, A, C, A, None, 4, 0.088, A, -1, 256, 128, None, None) == SHAPE
    # in-tile token offset x token stride beyond 2^31 bytes (Q's or O's)
    assert f(geom(grid=(8, 16, 32), shapes=((8, 4, 4),) * 2).ref, V.BF16, A, A, RAS, 0, 1 << 20, 128, A, C, A, None, 4,
             0.088, A, *st, None, None) == UNSUP
    assert f(geom(grid=(8, 16, 32), shapes=((8, 4, 4),) * 2).ref, V.BF16, A, A, RAS, *st, A, C, A, None, 4,
             0.088, A, 0, 1 << 20, 128, None, None) == UNSUP
    s = L.veda_trippool_score_raster
    assert s(g.ref, V.BF16, A, A, RAS, *st, A, A, A, A, 256, 64, 0.125, None, None, None, None, None, 6, None, None,
             None, None, A, 1 << 30, None) == NULL
    # K's tiled copy comes only from a raster K, and must be aligned
    assert s(g.ref, V.BF16, A, A, V.ROWS, *st, A, A, A, A, 256, 64, 0.125, None, None, None, None, None, 6, A, B_, None,
             None, A, 1 << 30, None) == SHAPE
    assert s(g.ref, V.BF16, A, A, RAS, *st, A, A, A, A, 256, 64, 0.125, None, None, None, None, None, 6, A, MIS, None,
             None, A, 1 << 30, None) == ALIGN
    # V's tiled copy needs the raster V and the output together, both aligned
    assert s(g.ref, V.BF16, A, A, RAS, *st, A, A, A, A, 256, 64, 0.125, None, None, None, None, None, 6, A, None, A,
             None, A, 1 << 30, None) == NULL
    assert s(g.ref, V.BF16, A, A, RAS, *st, A, A, A, A, 256, 64, 0.125, None, None, None, None, None, 6, A, None, None,
             B_, A, 1 << 30, None) == NULL
    assert s(g.ref, V.BF16, A, A, RAS, *st, A, A, A, A, 256, 64, 0.125, None, None, None, None, None, 6, A, None, A,
             MIS, A, 1 << 30, None) == ALIGN
    t = L.veda_oracle_tilemap_raster
    assert t(g.ref, V.BF16, A, A, V.ROWS, *st, 0.088, A, 0, A, None, A, 1 << 40, None) == SHAPE


def test_binding_checks_sizes_before_taking_pointers():
    """The C ABI cannot see buffer sizes, so the binding checks dtype and size of every
    tensor against the geometry first: short, mistyped or misshapen CPU tensors raise with
    the size message, before the GPU check and before any pointer is taken."""
    import torch
    g = geom()                                    # B 1, H 2, N 4096, d 128, n_t 32
    n = 2 * 4096 * 128
    bf = lambda m: torch.zeros(m, dtype=torch.bfloat16)
    i32 = lambda m: torch.zeros(m, dtype=torch.int32)
    with pytest.raises(V.VedaError, match="at least"):
        V.veda_sparse_attn_fwd(g, bf(n), bf(n), bf(n), i32(2 * 32 * 4).view(1, 2, 32, 4), 4, 0.088, bf(n - 8))
    with pytest.raises(V.VedaError, match="does not match k"):
        V.veda_sparse_attn_fwd(g, bf(n), bf(n), bf(n), i32(2 * 32 * 5).view(1, 2, 32, 5), 4, 0.088, bf(n))
    with pytest.raises(V.VedaError, match="dtype"):
        V.veda_sparse_attn_fwd(g, bf(n), bf(n), bf(n), torch.zeros(1, 2, 32, 4, dtype=torch.int64), 4, 0.088, bf(n))
    with pytest.raises(V.VedaError, match="at least"):     # list of one head only
        V.veda_sparse_attn_fwd(g, bf(n), bf(n), bf(n), i32(32 * 4).view(1, 1, 32, 4), 4, 0.088, bf(n))
    with pytest.raises(V.VedaError, match="shape"):
        V.veda_tile_gather(g, torch.zeros(1, 4096, 3, 128, dtype=torch.bfloat16), bf(n))
    with pytest.raises(V.VedaError, match="at least"):
        V.veda_tile_gather(g, torch.zeros(1, 4096, 2, 128, dtype=torch.bfloat16), bf(n - 1))
    w1, w2 = torch.zeros(2, 384, 256), torch.zeros(2, 256, 64)
    with pytest.raises(V.VedaError, match="shape"):
        V.veda_trippool_score(g, bf(n), bf(n), torch.zeros(3, 384, 256), w2, topk=6, idx=i32(2 * 32 * 6))
    with pytest.raises(V.VedaError, match="at least"):
        V.veda_trippool_score(g, bf(n), bf(n), w1, w2, topk=6, idx=i32(2 * 32 * 6 - 1))
    with pytest.raises(V.VedaError, match="at least"):
        V.veda_trippool_score(g, bf(n), bf(n), w1, w2, scores=torch.zeros(2 * 32 * 31))
    with pytest.raises(V.VedaError, match="at least"):     # key-tile bounds: [B, H, n_t]
        V.veda_trippool_score(g, bf(n), bf(n), w1, w2, topk=6, idx=i32(2 * 32 * 6), k_bound=torch.zeros(2 * 32 - 1))
    with pytest.raises(V.VedaError, match="dtype"):
        V.veda_sparse_attn_fwd(g, bf(n), bf(n), bf(n), i32(2 * 32 * 4).view(1, 2, 32, 4), 4, 0.088, bf(n),
                               k_bound=torch.zeros(2 * 32, dtype=torch.float64))
    with pytest.raises(V.VedaError, match="at least"):
        V.veda_oracle_tilemap(g, bf(n), bf(n), 0.088, i32(2 * 4), 4, torch.zeros(2 * 4 * 32 - 1))
    with pytest.raises(V.VedaError, match="at least"):
        V.veda_topk_mask(torch.zeros(4, 10), 3, i32(11))
    with pytest.raises(V.VedaError, match="at least"):
        V.veda_head_sq_error(bf(2 * 16 * 128).view(1, 16, 2, 128), bf(2 * 16 * 128).view(1, 16, 2, 128),
                             torch.zeros(1))
    # well-formed CPU tensors get as far as the device check
    with pytest.raises(V.VedaError, match="GPU tensor"):
        V.veda_sparse_attn_fwd(g, bf(n), bf(n), bf(n), i32(2 * 32 * 4).view(1, 2, 32, 4), 4, 0.088, bf(n))


def test_noalloc_scoring_rejects_beyond_its_scratch(L):
    """The no-allocation scoring call holds the MLP outputs of at most 65536 tiles (32 MiB of
    static scratch): a larger geometry is refused with VEDA_ERR_SCRATCH before anything runs,
    and its own argument checks are those of the workspace call."""
    f = L.veda_trippool_score_raster_noalloc
    RAS = V.RASTER
    big = geom(grid=(40, 48, 80), shapes=((2, 8, 8),) * 56)        # 56 heads x 1200 tiles = 67200
    st = (153600 * 56 * 128, 56 * 128, 128)
    assert f(big.ref, V.BF16, A, A, RAS, *st, A, A, A, A, 256, 64, 0.125, None, None, None, None, None, 60, A, None,
             None, None, None) == -8
    assert b"scratch" in L.veda_status_str(-8)
    fits = geom(grid=(40, 48, 80), shapes=((2, 8, 8),) * 54)       # 64800 tiles: passes the size check,
    st = (153600 * 54 * 128, 54 * 128, 128)                         # then a NULL K is refused
    assert f(fits.ref, V.BF16, A, None, RAS, *st, A, A, A, A, 256, 64, 0.125, None, None, None, None, None, 60, A, None,
             None, None, None) == NULL
    g = geom()
    st = (4096 * 2 * 128, 2 * 128, 128)
    assert f(g.ref, V.BF16, A, A, RAS, *st, A, A, A, A, 256, 64, 0.125, None, None, None, None, None, 6, None, None,
             None, None, None) == NULL
    assert f(g.ref, V.BF16, A, A, RAS, *st, A, A, A, A, 512, 64, 0.125, None, None, None, None, None, 6, A, None,
             None, None, None) == UNSUP
    assert f(g.ref, V.BF16, A, A, RAS, *st, A, A, A, A, 256, 64, 0.125, None, None, None, None, None, 6, A, None,
             A, None, None) == NULL                                    # V's copy: both or neither
