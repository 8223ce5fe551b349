/*
 * veda.h - C ABI of the MI355X (gfx950) hot path of Veda's distilled sparse attention.
 *
 * The method ("Technical Summary: Veda - Scalable Video Diffusion via Distilled Sparse
 * Attention", gist.science; arXiv abstract on fugumt.com): each attention head tiles the
 * T x H x W video latent with its own (p_t, p_h, p_w) factorisation of the hardware tile
 * (§2.2 Head-Aware Tiling), scores every (query tile, key tile) pair with a per-head MLP
 * on TripPool [mean|max|min] tile descriptors (§2.1 Distilled Tile Scoring), keeps the
 * best key tiles of each query tile, and runs attention only over the kept tiles
 * (§2.3 Hardware-Efficient Implementation).  The full-attention max-pooled tile map
 * (§2.1 "Target Construction") is the reference the estimator is distilled toward.
 *
 * Conventions (all entry points):
 *  - Every device buffer is owned by the caller; the library never allocates or frees
 *    device memory.  Host arrays (veda_geom.tile_shapes) are read before the call returns.
 *  - Calls are asynchronous on the given HIP stream and never synchronise it.
 *  - All arguments are validated before anything is launched; on an error nothing is
 *    launched and the status says why.  A failed HIP launch returns VEDA_ERR_HIP and
 *    veda_last_hip_error() reports the hipError_t (per host thread).
 *  - Device pointers must be 16-byte aligned (veda_topk_mask: 4-byte).  Outputs must not
 *    alias inputs.
 *  - Supported element types: VEDA_F32 with head_dim 64 and tile 64; VEDA_BF16 with
 *    head_dim 128 and tile 128.  Scores, descriptors, weights, LSEs and maps are float32.
 *  - Stateless and thread-safe (apart from the per-thread last-error slot).
 *
 * Tiled layouts (per batch b and head h, N = t*h*w tokens, P = tile, n_t = N / P; for
 * padded tilings see below):
 *  - VEDA_TILE_ROWS: [B, H, N, d]; row r holds token perm_h[r] of the raster sequence,
 *    where tile r / P is numbered row-major over the tile grid (t/p_t, h/p_h, w/p_w) and
 *    r % P row-major over (p_t, p_h, p_w).  Q, K, V and the attention output use it.
 *  - VEDA_TILE_COLS: [B, H, n_t, d, P]; the same tiles, each stored channel-major:
 *    element (position p, channel c) of tile j at ((j*d + c)*P + p) holds token
 *    key(p) of the tile, where within every group of 16 positions the tokens are ordered
 *    0-3, 8-11, 4-7, 12-15 (key(p) = 16*(p/16) + {0,1,2,3,8,9,10,11,4,5,6,7,12,13,14,15}
 *    [p%16]).  The attention calls also take V in it: that is the order in which the
 *    attention kernel's probability fragments meet V in the MFMA, so every V operand is
 *    one contiguous 16-byte read (a VEDA_TILE_ROWS V takes two transposed 8-byte reads per
 *    operand instead, at the same speed; the results are bit-identical).
 * The raster layout is [B, N, H, d] with any element strides for b, n, h and d contiguous;
 * raster token n = (t*H + h)*W + w.
 *
 * Padded tilings (bf16).  A head's shape (p_t, p_h, p_w) need not divide
 * the grid: the grid is then padded up to whole tiles on every axis for that head, giving
 * n_t(h) = ceil(t/p_t) * ceil(h/p_h) * ceil(w/p_w) tiles, some of them partial; a row of
 * the padded grid outside the real grid is a padding row and holds no token.  Reading of
 * [Technical Summary §2.2 Head-Aware Tiling], whose tiles are blocks of the latent grid.
 *  - Tiled tensors then have N = n_t * P rows per head with n_t = max_h n_t(h)
 *    (veda_tiled_tokens); rows past a head's own tiles and padding rows are zero after
 *    the gather and skipped by the scatter.
 *  - TripPool pools only a tile's real rows; attention and the tile map give padding
 *    keys no weight; padding query rows produce values that the scatter drops.
 *  - Scores, top-k lists and maps have n_t columns per row; a head uses its first n_t(h)
 *    (top-k and maps never pick or fill the others: scores -inf, probabilities and map
 *    entries 0).  k must not exceed the smallest n_t(h).
 *  - VEDA_F32 returns VEDA_ERR_UNSUPPORTED for such a geometry.  The raster attention and
 *    tile-map calls read K tiled (k_layout VEDA_TILE_ROWS, else VEDA_ERR_UNSUPPORTED), and
 *    the raster attention V tiled too (a raster V: VEDA_ERR_UNSUPPORTED); the raster
 *    scoring call reads K raster or tiled, and its k_tiled_out and v_tiled_out copies have
 *    the zero rows too.  Raster outputs hold the real tokens only (padding rows have none).  Both
 *    tile-map calls need an explicit q_tiles list.  veda_distill_step takes each head's
 *    own n_t(h) key tiles (target columns past them are ignored and get no gradient).
 */
#ifndef VEDA_H
#define VEDA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t veda_status;
enum {
  VEDA_OK = 0,
  VEDA_ERR_NULL = -1,        /* a required pointer is NULL */
  VEDA_ERR_SHAPE = -2,       /* sizes inconsistent: tile shape product != tile, k out of
                                range, too many heads ... */
  VEDA_ERR_DTYPE = -3,       /* unknown element type */
  VEDA_ERR_UNSUPPORTED = -4, /* valid but not implemented (head_dim/tile for this dtype) */
  VEDA_ERR_WORKSPACE = -5,   /* workspace NULL or smaller than the *_workspace_bytes query */
  VEDA_ERR_ALIGN = -6,       /* a device pointer is not 16-byte aligned */
  VEDA_ERR_HIP = -7,         /* a HIP launch failed; see veda_last_hip_error() */
  VEDA_ERR_SCRATCH = -8      /* the problem needs more than the library's static scratch
                                (veda_trippool_score_raster_noalloc) */
};

typedef enum { VEDA_F32 = 0, VEDA_BF16 = 1 } veda_dtype;
typedef enum { VEDA_TILE_ROWS = 0, VEDA_TILE_COLS = 1, VEDA_RASTER = 2 } veda_layout;

#define VEDA_MAX_HEADS 128

/* Problem geometry.  [Technical Summary §2.2: the per-(layer, head) tiling
 * pi = (p_t, p_h, p_w) factorises the hardware tile.] */
typedef struct {
  int32_t batch, heads, head_dim;  /* B, H (<= VEDA_MAX_HEADS), d; all >= 1 */
  int32_t t, h, w;                 /* latent grid, each >= 1, t*h*w <= 2^30 (an empty
                                      problem is VEDA_ERR_SHAPE, not a no-op) */
  int32_t tile;                    /* P tokens per tile */
  const int32_t *tile_shapes;      /* HOST int32[heads][3] (p_t, p_h, p_w); each product
                                      == tile; a shape that does not divide (t, h, w)
                                      makes the tiling padded (see above) */
} veda_geom;

/* Tokens per head of the tiled layouts (N = n_t * P; t*h*w unless the tiling is padded),
 * or a negative veda_status when the geometry is rejected. */
int64_t veda_tiled_tokens(const veda_geom *g, veda_dtype dtype);

/* Tiles of one head, n_t(h) (n_t unless the tiling is padded), or a negative status. */
int32_t veda_head_tiles(const veda_geom *g, veda_dtype dtype, int32_t head);

/* Head-aware tiling (permutation of tokens into per-head tiles).
 * [Technical Summary §2.2 Head-Aware Tiling]
 * inverse = 0: raster -> tiled (gather); inverse = 1: tiled -> raster (scatter; only
 * with layout VEDA_TILE_ROWS).  raster element (b, n, h, c) is at
 * raster[b*rs_b + n*rs_n + h*rs_h + c] (strides in elements; each multiple of 8 for
 * bf16 / 4 for f32, so rows stay 16-byte aligned).  tiled: contiguous, `layout`. */
veda_status veda_tile_gather(const veda_geom *g, veda_dtype dtype,
                             void *raster, int64_t rs_b, int64_t rs_n, int64_t rs_h,
                             void *tiled, veda_layout layout, int32_t inverse,
                             hipStream_t stream);

/* Workspace (bytes) that veda_trippool_score needs for the given geometry. */
size_t veda_trippool_workspace_bytes(const veda_geom *g, int32_t mlp_hidden, int32_t mlp_out);

/* Distilled tile scoring.  [Technical Summary §2.1 Distilled Tile Scoring]
 * For every tile of q_tiled and k_tiled (VEDA_TILE_ROWS): TripPool descriptor
 * [mean | max | min] over the tile's P tokens per channel (3d floats); per-head MLP
 * y = GELU(desc @ W1[h]) @ W2[h] (exact-erf GELU, no bias); logits
 * S[b,h,i,j] = score_scale * <y_q[i], y_k[j]>; optional row softmax over j; optional
 * top-k of each row (the k largest S, ties to the lower j, ascending j) - the same
 * selection as veda_topk_mask applied to S.
 *   w1_q, w1_k: [H, 3d, mlp_hidden] f32; w2_q, w2_k: [H, mlp_hidden, mlp_out] f32
 *               (the K pointers may alias the Q pointers: one MLP per head)
 *   scores:     out [B, H, n_t, n_t] f32, nullable
 *   probs:      out [B, H, n_t, n_t] f32 row softmax, nullable
 *   q_desc, k_desc: out [B, H, n_t, 3d] f32, nullable
 *   k_bound:    out [B, H, n_t] f32, nullable: for each key tile j,
 *               sqrt(sum over channels c of max(max_c^2, min_c^2)) with max_c, min_c its
 *               max and min descriptors - an upper bound of the L2 norm of every key row
 *               of the tile (0 for tiles past a padded head's own n_t(h)); the attention
 *               calls take it to fix their softmax offset
 *   topk, idx:  topk in [1, n_t] with idx out [B, H, n_t, topk] int32; or topk = 0, idx NULL
 * At least one of scores / probs / idx must be requested.  Implemented for
 * mlp_hidden = 256 and mlp_out = 64.  workspace >= veda_trippool_workspace_bytes. */
veda_status veda_trippool_score(const veda_geom *g, veda_dtype dtype,
                                const void *q_tiled, const void *k_tiled,
                                const float *w1_q, const float *w2_q,
                                const float *w1_k, const float *w2_k,
                                int32_t mlp_hidden, int32_t mlp_out, float score_scale,
                                float *scores, float *probs, float *q_desc, float *k_desc,
                                float *k_bound, int32_t topk, int32_t *idx,
                                void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Tile selection at a sparsity level.  [Technical Summary §4: 90% / 95% of key tiles
 * skipped]  For each of `rows` rows of scores [rows, n_cols] (f32), write the indices of
 * the k largest values (ties to the lower index) in ascending order to idx [rows, k]
 * int32, and optionally a 0/1 mask [rows, n_cols] uint8.  1 <= k <= n_cols <= 4096. */
veda_status veda_topk_mask(int64_t rows, int32_t n_cols, const float *scores, int32_t k,
                           int32_t *idx, uint8_t *mask, hipStream_t stream);

/* Tile-skipping attention forward.  [Technical Summary §2.3: the kernel fetches only the
 * selected, non-contiguous key/value tiles]  For every query tile i of every (b, h):
 * O = softmax(Q_i K_sel^T * softmax_scale) V_sel over the keys of the tiles
 * kv_idx[b, h, i, 0..k-1], the softmax renormalised over those keys.
 *   q_tiled, k_tiled: VEDA_TILE_ROWS
 *   v_tiled, v_layout: V and the layout it is in: VEDA_TILE_ROWS (tile-major, as Q and K)
 *           or VEDA_TILE_COLS (channel-major tiles); both give bit-identical results.
 *           VEDA_RASTER returns VEDA_ERR_UNSUPPORTED (no strides here: see the raster
 *           call), any other value VEDA_ERR_SHAPE, with nothing launched
 *   kv_idx: [B, H, n_t, k] int32, each entry in [0, n_t), no repeats within a row
 *           (k == n_t with every tile listed is dense attention).  Entries outside
 *           [0, n_t) are clamped into it (no out-of-bounds access; the result is then
 *           not meaningful).
 *   k_bound: [B, H, n_t] f32 upper bounds of the key-row norms of each key tile of this
 *           K (the k_bound output of the scoring call that read it), nullable.  The bf16
 *           kernel offsets each row's exponentials by its first kept tile's row maximum m
 *           (log2 units: logits times softmax_scale * log2 e); without k_bound it takes
 *           every later tile's row maximum too and moves m when one exceeds it by more
 *           than 8.  With k_bound, the 32 rows of a wave keep m fixed and take no further
 *           row maximum when every row's b = log2 e * softmax_scale * |q| * max over its
 *           kept tiles of k_bound (at or above each of its scaled logits) lies at most 64
 *           above its m, so that no exponential exceeds 2^64; the result is then the same bit for bit unless a later tile's
 *           row maximum exceeds m by more than 8, and the same softmax up to rounding
 *           otherwise.  Rows whose first tile's maximum lies above b by more than 8 (a
 *           k_bound of another K) take the running maximum.  A k_bound below the true
 *           norms can still overflow the exponentials of later tiles: the output is then
 *           not meaningful, with no out-of-bounds access.  With the offset fixed, the
 *           fp32 sums of P V reach up to 2^64 * k * P * max |v| (k * P kept keys), which
 *           stays finite while max |v| < 3.4e38 / (2^64 * k * P), about 2.4e15 at
 *           k * P = 7680 and 1.2e14 at 153600; V with larger values needs k_bound = NULL
 *           (then p <= 2^8).  The fp32 kernel ignores it.
 *   softmax_scale: > 0 and finite (else VEDA_ERR_SHAPE)
 *   o_tiled: out VEDA_TILE_ROWS, same dtype
 *   lse:     out [B, H, N] f32 natural-log log-sum-exp of each query row, nullable */
veda_status veda_sparse_attn_fwd(const veda_geom *g, veda_dtype dtype,
                                 const void *q_tiled, const void *k_tiled, const void *v_tiled,
                                 veda_layout v_layout, const int32_t *kv_idx, const float *k_bound, int32_t k,
                                 float softmax_scale, void *o_tiled, float *lse, hipStream_t stream);

/* Workspace (bytes) that veda_oracle_tilemap needs: B*H*n_sel*n_t*P floats. */
size_t veda_oracle_tilemap_workspace_bytes(const veda_geom *g, int32_t n_sel);

/* Oracle tile map.  [Technical Summary §2.1 "Target Construction": max-pooling of the
 * full-attention matrix over query-key tile regions; §2.3: built in two passes on random
 * subsets of query tiles]  For each selected query tile a (q_tiles[b, h, a], or a itself
 * if q_tiles is NULL) and each key tile j:
 *   tilemap[b, h, a, j] = max over queries q of tile, keys x of tile j, of
 *                         exp(s(q, x) - lse(q)),  s = q.x * softmax_scale,
 *   lse(q) = log sum over all N keys of exp(s(q, x)).
 * Pass 1 sweeps the keys once, accumulating lse(q) and keeping the row max of s over each
 * key tile in `workspace`; pass 2 normalises those maxima and pools them over the queries.
 *   q_tiled, k_tiled: VEDA_TILE_ROWS
 *   q_tiles: DEVICE int32 [B, H, n_sel] in [0, n_t) (entries outside are clamped), or
 *            NULL (then n_sel must be n_t)
 *   softmax_scale: > 0 and finite (else VEDA_ERR_SHAPE)
 *   tilemap: out [B, H, n_sel, n_t] f32;  lse: out [B, H, n_sel * P] f32, nullable
 *   workspace: >= veda_oracle_tilemap_workspace_bytes(g, n_sel) bytes of device memory */
veda_status veda_oracle_tilemap(const veda_geom *g, veda_dtype dtype,
                                const void *q_tiled, const void *k_tiled, float softmax_scale,
                                const int32_t *q_tiles, int32_t n_sel,
                                float *tilemap, float *lse,
                                void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Raster-direct variants (no tiled copies of Q or O, and optionally none of K).
 * [Technical Summary §2.3 and the paper's future work on fusing the tiling into the
 * kernels]  They compute exactly what veda_trippool_score, veda_sparse_attn_fwd and
 * veda_oracle_tilemap compute (bit for bit; attention given the same k_bound), but read Q
 * (and write O) in the raster layout
 * [B, N, H, d] with element strides rs_b, rs_n, rs_h for Q (os_b, os_n, os_h for O; d
 * contiguous, 16-byte aligned rows and strides), going through each head's tiling in the
 * kernels: row r of tile j of head h
 * is raster token origin_h(j) + intra_h(r).  k_layout says where K is: VEDA_RASTER (with
 * the same strides as Q) or VEDA_TILE_ROWS (tile-major [B, H, N, d], from
 * veda_tile_gather; K tiles are then contiguous 32 KB copies, which the attention and
 * tile-map kernels prefer).  veda_sparse_attn_fwd_raster takes V as VEDA_TILE_ROWS,
 * VEDA_TILE_COLS or VEDA_RASTER (v_layout; a raster V has the strides of Q and is read
 * through the tiling like a raster K, bit-identical but slower than a tiled V, whose tiles
 * are contiguous 32 KB copies).  The output of veda_sparse_attn_fwd_raster is raster
 * [B, N, H, d] with its own element strides os_b, os_n, os_h (checked as rs_*; e.g. Q, K
 * and V views of one packed QKV tensor and a separate contiguous O) and its lse is
 * [B, H, t*h*w] in raster token order; the tile-map lse keeps its
 * [B, H, n_sel * P] tile-row order.  Extra status: VEDA_ERR_UNSUPPORTED if an in-tile
 * token offset times the token stride reaches 2^31 bytes.  Other arguments, outputs and
 * workspaces as in the tiled calls.
 * veda_trippool_score_raster also takes k_tiled_out (nullable; only with k_layout
 * VEDA_RASTER, else VEDA_ERR_SHAPE): [B, H, N, d] of `dtype`, which receives K's tile-major
 * copy (exactly what veda_tile_gather writes with VEDA_TILE_ROWS), written as K is read for
 * pooling, so that one pass over K both scores it and tiles it for the attention and
 * tile-map calls (the paper's future work on kernel fusion).  It also takes v_raster and
 * v_tiled_out (both NULL, or both set, else VEDA_ERR_NULL; any k_layout): a raster V with
 * the strides of Q, and [B, H, N, d] of `dtype` that receives V's VEDA_TILE_ROWS copy
 * (exactly what veda_tile_gather writes), streamed by workgroups of the same launch that
 * only copy, so that the scoring pass also leaves V tiled for the attention call. */
veda_status veda_trippool_score_raster(const veda_geom *g, veda_dtype dtype, const void *q_raster, const void *k,
                                       veda_layout k_layout, int64_t rs_b, int64_t rs_n, int64_t rs_h,
                                       const float *w1_q, const float *w2_q, const float *w1_k, const float *w2_k,
                                       int32_t mlp_hidden, int32_t mlp_out, float score_scale, float *scores,
                                       float *probs, float *q_desc, float *k_desc, float *k_bound, int32_t topk,
                                       int32_t *idx, void *k_tiled_out, const void *v_raster, void *v_tiled_out,
                                       void *workspace, size_t workspace_bytes, hipStream_t stream);
veda_status veda_sparse_attn_fwd_raster(const veda_geom *g, veda_dtype dtype, const void *q_raster, const void *k,
                                        veda_layout k_layout, int64_t rs_b, int64_t rs_n, int64_t rs_h,
                                        const void *v, veda_layout v_layout, const int32_t *kv_idx,
                                        const float *k_bound, int32_t k_kept, float softmax_scale, void *o_raster,
                                        int64_t os_b, int64_t os_n, int64_t os_h, float *lse, hipStream_t stream);
veda_status veda_oracle_tilemap_raster(const veda_geom *g, veda_dtype dtype, const void *q_raster, const void *k,
                                       veda_layout k_layout, int64_t rs_b, int64_t rs_n, int64_t rs_h,
                                       float softmax_scale, const int32_t *q_tiles, int32_t n_sel, float *tilemap,
                                       float *lse, void *workspace, size_t workspace_bytes, hipStream_t stream);

/* veda_trippool_score_raster without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  It allocates nothing: the MLP outputs go to a static device
 * array of 32 MiB inside the library (each GPU it runs on holds one until the process
 * ends), which bounds the problem to B * H * n_t <= 65536 tiles (e.g. 48 heads of 1200
 * tiles); a larger geometry returns VEDA_ERR_SCRATCH with nothing launched.  The first
 * call on a device looks up that device's copy (hipGetSymbolAddress); the stream must
 * belong to the current device.  Every call on one GPU shares its copy: calls that
 * overlap on one GPU (other streams, other host threads) race, so the caller orders
 * them.  Arguments, outputs and every other status as in veda_trippool_score_raster. */
veda_status veda_trippool_score_raster_noalloc(const veda_geom *g, veda_dtype dtype, const void *q_raster,
                                               const void *k, veda_layout k_layout, int64_t rs_b, int64_t rs_n,
                                               int64_t rs_h, const float *w1_q, const float *w2_q,
                                               const float *w1_k, const float *w2_k, int32_t mlp_hidden,
                                               int32_t mlp_out, float score_scale, float *scores, float *probs,
                                               float *q_desc, float *k_desc, float *k_bound, int32_t topk,
                                               int32_t *idx, void *k_tiled_out, const void *v_raster,
                                               void *v_tiled_out, hipStream_t stream);

/* Workspace (bytes) that veda_distill_step needs (descriptors, MLP activations and
 * gradients of the sampled Q tiles and of every K tile, per-row KL terms). */
size_t veda_distill_workspace_bytes(const veda_geom *g, int32_t n_sel);

/* One distillation step of the per-head tile-score estimator.  [Technical Summary §2.1
 * "Optimization": a row-wise KL divergence between the full-attention reference and the
 * predicted tile-score distribution; stop-gradient on the features feeding the estimator]
 * With one MLP per head shared by the Q-tile and K-tile descriptors (w1 [H, 3d, 256],
 * w2 [H, 256, 64] f32, as in veda_trippool_score with w*_k = w*_q), for each sampled query
 * tile a of (b, h), i = q_tiles[b, h, a] (clamped to [0, n_t)):
 *   p = target[b, h, a, :] / sum_j target[b, h, a, j]   (e.g. the veda_oracle_tilemap rows)
 *   s = score_scale * y_q[i] . y_k[j]  for every key tile j
 *   loss = mean over the B*H*n_sel rows of KL(p || softmax(s))   (out [1] f32)
 *   dw1, dw2 = d loss / d w1, w2 (out, same shapes as w1, w2); descriptors are constants.
 * If lr != 0 the weights are then updated in place: w -= lr * dw.  Deterministic.
 *   q_tiled, k_tiled: VEDA_TILE_ROWS;  q_tiles: DEVICE int32 [B, H, n_sel] (required; a
 *   tile sampled twice counts twice);  target: [B, H, n_sel, n_t] f32, rows with a
 *   positive sum;  workspace: >= veda_distill_workspace_bytes(g, n_sel) bytes. */
veda_status veda_distill_step(const veda_geom *g, veda_dtype dtype, const void *q_tiled, const void *k_tiled,
                              float *w1, float *w2, int32_t mlp_hidden, int32_t mlp_out, float score_scale,
                              const int32_t *q_tiles, int32_t n_sel, const float *target, float *loss,
                              float *dw1, float *dw2, float lr, void *workspace, size_t workspace_bytes,
                              hipStream_t stream);

/* Per-head squared output error, the objective of the tiling search.  [Technical Summary
 * §2.2 Head-Aware Tiling, "Offline Selection": each head's tiling is picked on calibration
 * data by the error between the full-attention and the sparse-attention output]
 *   a, b: raster [B, N, H, d] contiguous tensors of `dtype` (d = head_dim; d * element
 *         size a multiple of 16 bytes), e.g. a sparse output and the dense output
 *   err:    out [B, H] f32, err[b, h] = sum over tokens n and channels c of (a - b)^2
 *   err_batch_sum: out [H] f32, sum over b of err[b, h] (the search objective summed
 *         over the calibration batch, added in ascending b), nullable
 *   ref_sq: out [B, H] f32, sum of b^2 (for relative errors), nullable
 *   workspace: device scratch of >= veda_head_sq_error_workspace_bytes(B, N, H) bytes,
 *         8-byte aligned, caller-owned (one partial pair per head and token chunk)
 * fp32 accumulation in a fixed order (deterministic).  The shapes only need N >= 1;
 * veda_geom is not used because the error does not depend on the tiling.  Errors:
 * VEDA_ERR_WORKSPACE when the workspace is missing or short; VEDA_ERR_UNSUPPORTED when one
 * token chunk holds 2^31 or more 16-byte pieces. */
size_t veda_head_sq_error_workspace_bytes(int32_t batch, int32_t n_tokens, int32_t heads);
veda_status veda_head_sq_error(int32_t batch, int32_t n_tokens, int32_t heads, int32_t head_dim,
                               veda_dtype dtype, const void *a, const void *b, float *err,
                               float *err_batch_sum, float *ref_sq, void *workspace, size_t workspace_bytes,
                               hipStream_t stream);

const char *veda_status_str(veda_status s);
int veda_last_hip_error(void);
/* Library version string. */
const char *veda_version(void);

#ifdef __cplusplus
}
#endif
#endif /* VEDA_H */
