// Host-side launchers of the gfx950 kernels (internal).  Each enqueues its kernels on
// `st` and returns hipGetLastError(); arguments are validated by the C ABI layer first.
#pragma once
#include "common.h"

namespace veda {

hipError_t launch_gather(const Geo &g, const HeadShapes &hs, veda_dtype dt, void *raster, int64_t rs_b,
                         int64_t rs_n, int64_t rs_h, void *tiled, veda_layout layout, int inverse, hipStream_t st);

// Scoring: pool -> MLP -> scores / softmax / top-k.  ws layout: see score.hip.  With rv
// (and hs) set, Q is a raster tensor read through each head's tiling, and K too if k_raster;
// k_tiled_out (raster K only) receives K's tile-major copy, written as K is pooled;
// v_tiled_out (raster Q only) receives the tile-major copy of the raster V v_raster (strides
// of Q), streamed in the same launch; k_bound [B][H][n_t] receives each key tile's row-norm
// bound (from its max and min descriptors).
size_t score_workspace_bytes(const Geo &g, int hidden, int mlp_out);
hipError_t launch_score(const Geo &g, veda_dtype dt, const void *q, const void *k, const float *w1q,
                        const float *w2q, const float *w1k, const float *w2k, int hidden, int mlp_out, float scale,
                        float *scores, float *probs, float *q_desc, float *k_desc, int topk, int32_t *idx,
                        void *ws, hipStream_t st, const HeadShapes *hs = nullptr, const RasterView *rv = nullptr,
                        bool k_raster = false, void *k_tiled_out = nullptr, const void *v_raster = nullptr,
                        void *v_tiled_out = nullptr, float *k_bound = nullptr);

// TripPool + MLP only: y [Q|K][B][H][n_t][64]; descriptors [B][H][n_t][3d] if non-NULL;
// the pre-activation hidden layer z [Q|K][B][H][n_t][256] if non-NULL.  With qlist
// ([B][H][nlist] tile indices), the Q rows are the listed tiles, rows 0 .. nlist-1 of each
// (b, h) block, instead of every tile.
hipError_t launch_pool_mlp(const Geo &g, veda_dtype dt, const void *q, const void *k, const float *w1q,
                           const float *w2q, const float *w1k, const float *w2k, float *y, float *q_desc,
                           float *k_desc, hipStream_t st, const HeadShapes *hs = nullptr,
                           const RasterView *rv = nullptr, bool k_raster = false, float *z = nullptr,
                           const int32_t *qlist = nullptr, int nlist = 0, void *k_tiled_out = nullptr,
                           const void *v_raster = nullptr, void *v_tiled_out = nullptr, float *k_bound = nullptr);

hipError_t launch_topk(int64_t rows, int n_cols, const float *scores, int k, int32_t *idx, uint8_t *mask,
                       hipStream_t st);

// V in v_layout: VEDA_TILE_COLS or VEDA_TILE_ROWS.  kbound: [B][H][n_t] key-tile row-norm
// bounds (the fixed exponent offset), or null (running offset).
hipError_t launch_sparse_attn(const Geo &g, const HeadShapes &hs, veda_dtype dt, const void *q, const void *k,
                              const void *v, veda_layout v_layout, const int32_t *kv_idx, const float *kbound, int kk,
                              float scale, void *o, float *lse, hipStream_t st);

// Q (element strides rs_*) and O (element strides os_*) in raster layout [B, N, H, d], K
// raster (Q's strides) or tile-major, V channel-major tiled, tile-major, or raster with Q's
// strides.
hipError_t launch_sparse_attn_raster(const Geo &g, const HeadShapes &hs, veda_dtype dt, const void *q, const void *k,
                                     bool k_raster, int64_t rs_b, int64_t rs_n, int64_t rs_h, const void *v,
                                     veda_layout v_layout, const int32_t *kv_idx, const float *kbound, int kk,
                                     float scale, void *o, int64_t os_b, int64_t os_n, int64_t os_h, float *lse,
                                     hipStream_t st);

size_t tilemap_workspace_bytes(const Geo &g, int n_sel);
hipError_t launch_tilemap(const Geo &g, veda_dtype dt, const void *q, const void *k, float scale,
                          const int32_t *q_tiles, int n_sel, float *tilemap, float *lse, void *ws, hipStream_t st,
                          const HeadShapes *hs = nullptr, const RasterView *rv = nullptr, bool k_raster = false);

// Distillation step (see distill.hip).
size_t distill_workspace_bytes(const Geo &g, int n_sel);
hipError_t launch_distill(const Geo &g, const HeadShapes &hs, veda_dtype dt, const void *q, const void *k, float *w1,
                          float *w2, float score_scale, const int32_t *q_tiles, int n_sel, const float *target,
                          float *loss, float *dw1, float *dw2, float lr, void *ws, hipStream_t st);

int head_sq_error_chunks(int n_tokens);  // token chunks per head (one partial pair each)
hipError_t launch_head_sq_error(int batch, int n_tokens, int heads, int head_dim, veda_dtype dt, const void *a,
                                const void *b, float *err, float *err_batch_sum, float *ref_sq, void *ws,
                                hipStream_t st);

}  // namespace veda
