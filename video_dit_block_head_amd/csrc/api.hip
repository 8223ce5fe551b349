// C ABI of the library: argument validation (before anything is launched), status codes,
// and dispatch to the kernel launchers.  No exception crosses this boundary.
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "common.h"
#include "kernels.h"

using namespace veda;

static thread_local int g_last_hip_error = 0;

namespace {

constexpr int SCORE_MAX_NT = 1536;  // the score kernel holds a row of <= 1536 scores in registers
constexpr int DISTILL_MAX_NT = 1536;  // the KL row kernel holds a row of <= 1536 logits in registers
constexpr int TILEMAP_MAX_NT_F32 = 1280;  // the fp32 tile map keeps one row of maxima in LDS
constexpr int TILEMAP_MAX_NT = 1536;

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

veda_status hip_status(hipError_t e) {
  if (e == hipSuccess) return VEDA_OK;
  g_last_hip_error = (int)e;
  return VEDA_ERR_HIP;
}

// Tiles of every head on the grid padded up to whole tiles: the largest and smallest count,
// and whether some shape does not divide the grid.  Shapes are assumed valid.
void tile_counts(const veda_geom *g, int *nt_max, int *nt_min, bool *padded) {
  *nt_max = 0;
  *nt_min = INT32_MAX;
  *padded = false;
  for (int h = 0; h < g->heads; ++h) {
    const int pt = g->tile_shapes[3 * h], ph = g->tile_shapes[3 * h + 1], pw = g->tile_shapes[3 * h + 2];
    const int n = head_tiles(pt, ph, pw, g->t, g->h, g->w);
    *nt_max = n > *nt_max ? n : *nt_max;
    *nt_min = n < *nt_min ? n : *nt_min;
    *padded = *padded || g->t % pt || g->h % ph || g->w % pw;
  }
}

// Validates the geometry and dtype; fills Geo and per-head shapes.  Shapes that do not
// divide the grid pad it up to whole tiles per head (bf16 only); nt_min (optional) receives
// the smallest per-head tile count.
veda_status check_geom(const veda_geom *g, veda_dtype dt, Geo *out, HeadShapes *hs, int *nt_min = nullptr) {
  if (g == nullptr || g->tile_shapes == nullptr) return VEDA_ERR_NULL;
  if (dt != VEDA_F32 && dt != VEDA_BF16) return VEDA_ERR_DTYPE;
  if (g->batch < 1 || g->heads < 1 || g->heads > VEDA_MAX_HEADS || g->t < 1 || g->h < 1 || g->w < 1 ||
      g->tile < 1 || g->head_dim < 1)
    return VEDA_ERR_SHAPE;
  const int64_t n = (int64_t)g->t * g->h * g->w;
  if (n > (int64_t)1 << 30) return VEDA_ERR_SHAPE;
  if (dt == VEDA_BF16 && !(g->head_dim == 128 && g->tile == 128)) return VEDA_ERR_UNSUPPORTED;
  if (dt == VEDA_F32 && !(g->head_dim == 64 && g->tile == 64)) return VEDA_ERR_UNSUPPORTED;
  memset(hs, 0, sizeof(*hs));
  for (int h = 0; h < g->heads; ++h) {
    const int32_t pt = g->tile_shapes[3 * h], ph = g->tile_shapes[3 * h + 1], pw = g->tile_shapes[3 * h + 2];
    if (pt < 1 || ph < 1 || pw < 1) return VEDA_ERR_SHAPE;
    if ((int64_t)pt * ph * pw != g->tile) return VEDA_ERR_SHAPE;
    hs->s[h][0] = pt;
    hs->s[h][1] = ph;
    hs->s[h][2] = pw;
  }
  int nt_max, nt_lo;
  bool padded;
  tile_counts(g, &nt_max, &nt_lo, &padded);
  if ((int64_t)nt_max * g->tile > (int64_t)1 << 30) return VEDA_ERR_SHAPE;
  if (padded && dt != VEDA_BF16) return VEDA_ERR_UNSUPPORTED;
  out->B = g->batch;
  out->H = g->heads;
  out->d = g->head_dim;
  out->T = g->t;
  out->Hs = g->h;
  out->Ws = g->w;
  out->P = g->tile;
  out->N = nt_max * g->tile;  // tiled tokens per head (= t*h*w unless padded)
  out->nt = nt_max;
  out->padded = padded ? 1 : 0;
  if (nt_min != nullptr) *nt_min = nt_lo;
  return VEDA_OK;
}

// Tile count used to size buffers, from the geometry alone (0 when it is unusable).
int geom_tiles(const veda_geom *g) {
  if (g == nullptr || g->tile < 1 || g->heads < 1 || g->heads > VEDA_MAX_HEADS) return 0;
  if (g->tile_shapes == nullptr) return (int)((int64_t)g->t * g->h * g->w / g->tile);
  for (int h = 0; h < g->heads; ++h)
    if (g->tile_shapes[3 * h] < 1 || g->tile_shapes[3 * h + 1] < 1 || g->tile_shapes[3 * h + 2] < 1) return 0;
  int nt_max, nt_min;
  bool padded;
  tile_counts(g, &nt_max, &nt_min, &padded);
  return nt_max;
}

// Raster operands read through the tilings: 16-byte aligned rows and strides, and every
// in-tile token offset (the per-lane part of a copy address) below 2^31 bytes.
veda_status check_raster(const Geo &geo, const HeadShapes &hs, veda_dtype dt, int64_t rs_b, int64_t rs_n,
                         int64_t rs_h) {
  if (rs_b < 0 || rs_n < 0 || rs_h < 0) return VEDA_ERR_SHAPE;
  const int64_t epc = dt == VEDA_BF16 ? 8 : 4, eb = dt == VEDA_BF16 ? 2 : 4;
  if (rs_b % epc || rs_n % epc || rs_h % epc) return VEDA_ERR_ALIGN;
  for (int h = 0; h < geo.H; ++h) {
    const int64_t pt = hs.s[h][0], ph = hs.s[h][1], pw = hs.s[h][2];
    const int64_t intra_max = ((pt - 1) * geo.Hs + (ph - 1)) * geo.Ws + (pw - 1);
    if (intra_max * rs_n * eb >= ((int64_t)1 << 31)) return VEDA_ERR_UNSUPPORTED;
  }
  return VEDA_OK;
}

// A softmax scale the kernels handle: positive and finite (they take row maxima of the
// unscaled logits).
bool scale_ok(float x) { return x > 0.f && x <= 3.4028234663852886e38f; }

// Validation shared by the raster scoring calls: everything but the workspace.  Fills the
// kernels' geometry, shapes and raster byte strides.
veda_status check_score_raster(const veda_geom *g, veda_dtype dtype, const void *q_raster, const void *k_raster,
                               veda_layout k_layout, int64_t rs_b, int64_t rs_n, int64_t rs_h, const float *w1_q,
                               const float *w2_q, const float *w1_k, const float *w2_k, int32_t mlp_hidden,
                               int32_t mlp_out, const float *scores, const float *probs, const float *q_desc,
                               const float *k_desc, const float *k_bound, int32_t topk, const int32_t *idx,
                               const void *k_tiled_out,
                               const void *v_raster, const void *v_tiled_out, Geo *geo, HeadShapes *hs,
                               RasterView *rv) {
  int nt_min;
  veda_status s = check_geom(g, dtype, geo, hs, &nt_min);
  if (s != VEDA_OK) return s;
  if (!q_raster || !k_raster || !w1_q || !w2_q || !w1_k || !w2_k) return VEDA_ERR_NULL;
  if (scores == nullptr && probs == nullptr && idx == nullptr) return VEDA_ERR_NULL;
  if ((topk > 0) != (idx != nullptr)) return idx ? VEDA_ERR_SHAPE : VEDA_ERR_NULL;
  if (topk < 0 || topk > nt_min) return VEDA_ERR_SHAPE;
  if (mlp_hidden != 256 || mlp_out != 64) return VEDA_ERR_UNSUPPORTED;
  if (geo->nt > SCORE_MAX_NT) return VEDA_ERR_UNSUPPORTED;
  if ((v_raster == nullptr) != (v_tiled_out == nullptr)) return VEDA_ERR_NULL;  // V's copy: both or neither
  const void *ptrs[] = {q_raster, k_raster, w1_q, w2_q, w1_k,        w2_k,     scores,     probs,
                        q_desc,   k_desc,   k_bound, idx, k_tiled_out, v_raster, v_tiled_out};
  for (const void *p : ptrs)
    if (p && !aligned16(p)) return VEDA_ERR_ALIGN;
  if (k_layout != VEDA_RASTER && k_layout != VEDA_TILE_ROWS) return VEDA_ERR_SHAPE;
  if (k_tiled_out != nullptr && k_layout != VEDA_RASTER) return VEDA_ERR_SHAPE;  // the copy is of a raster K
  if ((s = check_raster(*geo, *hs, dtype, rs_b, rs_n, rs_h)) != VEDA_OK) return s;
  const int64_t eb = dtype == VEDA_BF16 ? 2 : 4;
  *rv = RasterView{rs_b * eb, rs_n * eb, rs_h * eb};
  return VEDA_OK;
}

// Static scratch of the no-allocation scoring call: the MLP outputs y_q, y_k of one call
// (2 * B * H * n_t * 64 floats; 32 MiB holds B * H * n_t <= 65536 tiles, e.g. 48 heads of
// 1200 tiles).  Each GPU the library runs on holds its own copy until the process ends.
// In host code `scratch` only names the symbol: its device address on the current device
// comes from hipGetSymbolAddress, once per device, and only that address is ever passed to
// a kernel.
constexpr size_t SCRATCH_BYTES = (size_t)32 << 20;
static __device__ __align__(256) uint8_t scratch[SCRATCH_BYTES];
constexpr int SCRATCH_MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[SCRATCH_MAX_DEVICES] = {};

// Device address of `scratch` on the current device (looked up on the first call there).
veda_status scratch_device_ptr(void **out) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= SCRATCH_MAX_DEVICES) return VEDA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    const hipError_t se = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (se != hipSuccess) return hip_status(se);
    if (p == nullptr) return VEDA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return VEDA_OK;
}

}  // namespace

extern "C" {

veda_status veda_tile_gather(const veda_geom *g, veda_dtype dtype, void *raster, int64_t rs_b, int64_t rs_n,
                             int64_t rs_h, void *tiled, veda_layout layout, int32_t inverse, hipStream_t stream) {
  Geo geo;
  HeadShapes hs;
  veda_status s = check_geom(g, dtype, &geo, &hs);
  if (s != VEDA_OK) return s;
  if (raster == nullptr || tiled == nullptr) return VEDA_ERR_NULL;
  if (!aligned16(raster) || !aligned16(tiled)) return VEDA_ERR_ALIGN;
  if (layout != VEDA_TILE_ROWS && layout != VEDA_TILE_COLS) return VEDA_ERR_SHAPE;
  if (inverse != 0 && inverse != 1) return VEDA_ERR_SHAPE;
  if (inverse && layout != VEDA_TILE_ROWS) return VEDA_ERR_UNSUPPORTED;
  if (rs_b < 0 || rs_n < 0 || rs_h < 0) return VEDA_ERR_SHAPE;
  const int64_t epc = dtype == VEDA_BF16 ? 8 : 4;  // elements per 16 bytes
  if (rs_b % epc || rs_n % epc || rs_h % epc) return VEDA_ERR_ALIGN;
  return hip_status(launch_gather(geo, hs, dtype, raster, rs_b, rs_n, rs_h, tiled, layout, inverse, stream));
}

size_t veda_trippool_workspace_bytes(const veda_geom *g, int32_t mlp_hidden, int32_t mlp_out) {
  if (g == nullptr || g->batch < 1 || g->heads < 1 || g->tile < 1 || mlp_out < 1) return 0;
  const int64_t n = (int64_t)g->t * g->h * g->w;
  Geo geo{};
  geo.B = g->batch;
  geo.H = g->heads;
  geo.d = g->head_dim;
  (void)n;
  geo.nt = geom_tiles(g);
  return score_workspace_bytes(geo, mlp_hidden, mlp_out);
}

veda_status veda_trippool_score(const veda_geom *g, veda_dtype dtype, const void *q_tiled, const void *k_tiled,
                                const float *w1_q, const float *w2_q, const float *w1_k, const float *w2_k,
                                int32_t mlp_hidden, int32_t mlp_out, float score_scale, float *scores, float *probs,
                                float *q_desc, float *k_desc, float *k_bound, int32_t topk, int32_t *idx,
                                void *workspace, size_t workspace_bytes, hipStream_t stream) {
  Geo geo;
  HeadShapes hs;
  int nt_min;
  veda_status s = check_geom(g, dtype, &geo, &hs, &nt_min);
  if (s != VEDA_OK) return s;
  if (!q_tiled || !k_tiled || !w1_q || !w2_q || !w1_k || !w2_k) return VEDA_ERR_NULL;
  if (scores == nullptr && probs == nullptr && idx == nullptr) return VEDA_ERR_NULL;
  if ((topk > 0) != (idx != nullptr)) return idx ? VEDA_ERR_SHAPE : VEDA_ERR_NULL;
  if (topk < 0 || topk > nt_min) return VEDA_ERR_SHAPE;
  if (mlp_hidden != 256 || mlp_out != 64) return VEDA_ERR_UNSUPPORTED;
  if (geo.nt > SCORE_MAX_NT) return VEDA_ERR_UNSUPPORTED;
  const void *ptrs[] = {q_tiled, k_tiled, w1_q, w2_q, w1_k, w2_k, scores, probs, q_desc, k_desc, k_bound, idx, workspace};
  for (const void *p : ptrs)
    if (p && !aligned16(p)) return VEDA_ERR_ALIGN;
  if (workspace == nullptr || workspace_bytes < score_workspace_bytes(geo, mlp_hidden, mlp_out))
    return VEDA_ERR_WORKSPACE;
  return hip_status(launch_score(geo, dtype, q_tiled, k_tiled, w1_q, w2_q, w1_k, w2_k, mlp_hidden, mlp_out,
                                 score_scale, scores, probs, q_desc, k_desc, topk, idx, workspace, stream, &hs,
                                 nullptr, false, nullptr, nullptr, nullptr, k_bound));
}

veda_status veda_trippool_score_raster(const veda_geom *g, veda_dtype dtype, const void *q_raster,
                                       const void *k_raster, veda_layout k_layout, int64_t rs_b, int64_t rs_n,
                                       int64_t rs_h,
                                       const float *w1_q, const float *w2_q, const float *w1_k, const float *w2_k,
                                       int32_t mlp_hidden, int32_t mlp_out, float score_scale, float *scores,
                                       float *probs, float *q_desc, float *k_desc, float *k_bound, int32_t topk,
                                       int32_t *idx, void *k_tiled_out, const void *v_raster, void *v_tiled_out,
                                       void *workspace, size_t workspace_bytes, hipStream_t stream) {
  Geo geo;
  HeadShapes hs;
  RasterView rv;
  veda_status s = check_score_raster(g, dtype, q_raster, k_raster, k_layout, rs_b, rs_n, rs_h, w1_q, w2_q, w1_k,
                                     w2_k, mlp_hidden, mlp_out, scores, probs, q_desc, k_desc, k_bound, topk, idx,
                                     k_tiled_out, v_raster, v_tiled_out, &geo, &hs, &rv);
  if (s != VEDA_OK) return s;
  if (workspace != nullptr && !aligned16(workspace)) return VEDA_ERR_ALIGN;
  if (workspace == nullptr || workspace_bytes < score_workspace_bytes(geo, mlp_hidden, mlp_out))
    return VEDA_ERR_WORKSPACE;
  return hip_status(launch_score(geo, dtype, q_raster, k_raster, w1_q, w2_q, w1_k, w2_k, mlp_hidden, mlp_out,
                                 score_scale, scores, probs, q_desc, k_desc, topk, idx, workspace, stream, &hs, &rv,
                                 k_layout == VEDA_RASTER, k_tiled_out, v_raster, v_tiled_out, k_bound));
}

veda_status veda_trippool_score_raster_noalloc(const veda_geom *g, veda_dtype dtype, const void *q_raster,
                                               const void *k_raster, veda_layout k_layout, int64_t rs_b,
                                               int64_t rs_n, int64_t rs_h, const float *w1_q, const float *w2_q,
                                               const float *w1_k, const float *w2_k, int32_t mlp_hidden,
                                               int32_t mlp_out, float score_scale, float *scores, float *probs,
                                               float *q_desc, float *k_desc, float *k_bound, int32_t topk,
                                               int32_t *idx, void *k_tiled_out, const void *v_raster,
                                               void *v_tiled_out, hipStream_t stream) {
  Geo geo;
  HeadShapes hs;
  RasterView rv;
  veda_status s = check_score_raster(g, dtype, q_raster, k_raster, k_layout, rs_b, rs_n, rs_h, w1_q, w2_q, w1_k,
                                     w2_k, mlp_hidden, mlp_out, scores, probs, q_desc, k_desc, k_bound, topk, idx,
                                     k_tiled_out, v_raster, v_tiled_out, &geo, &hs, &rv);
  if (s != VEDA_OK) return s;
  if (score_workspace_bytes(geo, mlp_hidden, mlp_out) > SCRATCH_BYTES) return VEDA_ERR_SCRATCH;
  void *ws = nullptr;
  if ((s = scratch_device_ptr(&ws)) != VEDA_OK) return s;
  // The MLP outputs are written whole before they are read: nothing needs clearing.
  return hip_status(launch_score(geo, dtype, q_raster, k_raster, w1_q, w2_q, w1_k, w2_k, mlp_hidden, mlp_out,
                                 score_scale, scores, probs, q_desc, k_desc, topk, idx, ws, stream, &hs, &rv,
                                 k_layout == VEDA_RASTER, k_tiled_out, v_raster, v_tiled_out, k_bound));
}

veda_status veda_topk_mask(int64_t rows, int32_t n_cols, const float *scores, int32_t k, int32_t *idx,
                           uint8_t *mask, hipStream_t stream) {
  if (rows < 0 || n_cols < 1 || n_cols > 4096 || k < 1 || k > n_cols) return VEDA_ERR_SHAPE;
  if (rows > ((int64_t)1 << 31) * 4 - 4) return VEDA_ERR_SHAPE;
  if (scores == nullptr || idx == nullptr) return VEDA_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(scores) & 3u) || (reinterpret_cast<uintptr_t>(idx) & 3u)) return VEDA_ERR_ALIGN;
  if (rows == 0) return VEDA_OK;
  return hip_status(launch_topk(rows, n_cols, scores, k, idx, mask, stream));
}

veda_status veda_sparse_attn_fwd(const veda_geom *g, veda_dtype dtype, const void *q_tiled, const void *k_tiled,
                                 const void *v_tiled, veda_layout v_layout, const int32_t *kv_idx,
                                 const float *k_bound, int32_t k, float softmax_scale, void *o_tiled, float *lse,
                                 hipStream_t stream) {
  Geo geo;
  HeadShapes hs;
  int nt_min;
  veda_status s = check_geom(g, dtype, &geo, &hs, &nt_min);
  if (s != VEDA_OK) return s;
  if (!q_tiled || !k_tiled || !v_tiled || !kv_idx || !o_tiled) return VEDA_ERR_NULL;
  if (v_layout == VEDA_RASTER) return VEDA_ERR_UNSUPPORTED;  // no raster strides in the tiled call
  if (v_layout != VEDA_TILE_ROWS && v_layout != VEDA_TILE_COLS) return VEDA_ERR_SHAPE;
  if (k < 1 || k > nt_min || !scale_ok(softmax_scale)) return VEDA_ERR_SHAPE;
  const void *ptrs[] = {q_tiled, k_tiled, v_tiled, kv_idx, k_bound, o_tiled, lse};
  for (const void *p : ptrs)
    if (p && !aligned16(p)) return VEDA_ERR_ALIGN;
  return hip_status(launch_sparse_attn(geo, hs, dtype, q_tiled, k_tiled, v_tiled, v_layout, kv_idx, k_bound, k,
                                       softmax_scale, o_tiled, lse, stream));
}

veda_status veda_sparse_attn_fwd_raster(const veda_geom *g, veda_dtype dtype, const void *q_raster,
                                        const void *k_raster, veda_layout k_layout, int64_t rs_b, int64_t rs_n,
                                        int64_t rs_h,
                                        const void *v, veda_layout v_layout, const int32_t *kv_idx,
                                        const float *k_bound, int32_t k, float softmax_scale, void *o_raster,
                                        int64_t os_b, int64_t os_n, int64_t os_h, float *lse, hipStream_t stream) {
  Geo geo;
  HeadShapes hs;
  int nt_min;
  veda_status s = check_geom(g, dtype, &geo, &hs, &nt_min);
  if (s != VEDA_OK) return s;
  if (!q_raster || !k_raster || !v || !kv_idx || !o_raster) return VEDA_ERR_NULL;
  if (k < 1 || k > nt_min || !scale_ok(softmax_scale)) return VEDA_ERR_SHAPE;
  const void *ptrs[] = {q_raster, k_raster, v, kv_idx, k_bound, o_raster, lse};
  for (const void *p : ptrs)
    if (p && !aligned16(p)) return VEDA_ERR_ALIGN;
  if (k_layout != VEDA_RASTER && k_layout != VEDA_TILE_ROWS) return VEDA_ERR_SHAPE;
  if (v_layout != VEDA_RASTER && v_layout != VEDA_TILE_ROWS && v_layout != VEDA_TILE_COLS) return VEDA_ERR_SHAPE;
  if ((s = check_raster(geo, hs, dtype, rs_b, rs_n, rs_h)) != VEDA_OK) return s;
  if ((s = check_raster(geo, hs, dtype, os_b, os_n, os_h)) != VEDA_OK) return s;
  // padded tilings: K and V tiled (the copies read whole tiles)
  if (geo.padded && (k_layout != VEDA_TILE_ROWS || v_layout == VEDA_RASTER)) return VEDA_ERR_UNSUPPORTED;
  return hip_status(launch_sparse_attn_raster(geo, hs, dtype, q_raster, k_raster, k_layout == VEDA_RASTER, rs_b, rs_n,
                                              rs_h, v, v_layout, kv_idx, k_bound, k, softmax_scale, o_raster, os_b,
                                              os_n, os_h, lse, stream));
}

size_t veda_oracle_tilemap_workspace_bytes(const veda_geom *g, int32_t n_sel) {
  if (g == nullptr || g->batch < 1 || g->heads < 1 || g->tile < 1 || n_sel < 1) return 0;
  Geo geo{};
  geo.B = g->batch;
  geo.H = g->heads;
  geo.P = g->tile;
  geo.nt = geom_tiles(g);
  return tilemap_workspace_bytes(geo, n_sel);
}

veda_status veda_oracle_tilemap(const veda_geom *g, veda_dtype dtype, const void *q_tiled, const void *k_tiled,
                                float softmax_scale, const int32_t *q_tiles, int32_t n_sel, float *tilemap,
                                float *lse, void *workspace, size_t workspace_bytes, hipStream_t stream) {
  Geo geo;
  HeadShapes hs;
  veda_status s = check_geom(g, dtype, &geo, &hs);
  if (s != VEDA_OK) return s;
  if (!q_tiled || !k_tiled || !tilemap) return VEDA_ERR_NULL;
  if (n_sel < 1 || n_sel > geo.nt || (q_tiles == nullptr && (n_sel != geo.nt || geo.padded))) return VEDA_ERR_SHAPE;
  if (!scale_ok(softmax_scale)) return VEDA_ERR_SHAPE;
  if (geo.nt > (dtype == VEDA_F32 ? TILEMAP_MAX_NT_F32 : TILEMAP_MAX_NT)) return VEDA_ERR_UNSUPPORTED;
  const void *ptrs[] = {q_tiled, k_tiled, q_tiles, tilemap, lse, workspace};
  for (const void *p : ptrs)
    if (p && !aligned16(p)) return VEDA_ERR_ALIGN;
  if (workspace == nullptr || workspace_bytes < tilemap_workspace_bytes(geo, n_sel)) return VEDA_ERR_WORKSPACE;
  return hip_status(
      launch_tilemap(geo, dtype, q_tiled, k_tiled, softmax_scale, q_tiles, n_sel, tilemap, lse, workspace, stream, &hs));
}

size_t veda_distill_workspace_bytes(const veda_geom *g, int32_t n_sel) {
  if (g == nullptr || g->batch < 1 || g->heads < 1 || g->tile < 1 || g->head_dim < 1 || n_sel < 1) return 0;
  Geo geo{};
  geo.B = g->batch;
  geo.H = g->heads;
  geo.d = g->head_dim;
  geo.P = g->tile;
  geo.nt = geom_tiles(g);
  return distill_workspace_bytes(geo, n_sel);
}

veda_status veda_oracle_tilemap_raster(const veda_geom *g, veda_dtype dtype, const void *q_raster,
                                       const void *k_raster, veda_layout k_layout, int64_t rs_b, int64_t rs_n,
                                       int64_t rs_h,
                                       float softmax_scale, const int32_t *q_tiles, int32_t n_sel, float *tilemap,
                                       float *lse, void *workspace, size_t workspace_bytes, hipStream_t stream) {
  Geo geo;
  HeadShapes hs;
  veda_status s = check_geom(g, dtype, &geo, &hs);
  if (s != VEDA_OK) return s;
  if (!q_raster || !k_raster || !tilemap) return VEDA_ERR_NULL;
  if (n_sel < 1 || n_sel > geo.nt || (q_tiles == nullptr && (n_sel != geo.nt || geo.padded))) return VEDA_ERR_SHAPE;
  if (!scale_ok(softmax_scale)) return VEDA_ERR_SHAPE;
  if (geo.nt > (dtype == VEDA_F32 ? TILEMAP_MAX_NT_F32 : TILEMAP_MAX_NT)) return VEDA_ERR_UNSUPPORTED;
  const void *ptrs[] = {q_raster, k_raster, q_tiles, tilemap, lse, workspace};
  for (const void *p : ptrs)
    if (p && !aligned16(p)) return VEDA_ERR_ALIGN;
  if (k_layout != VEDA_RASTER && k_layout != VEDA_TILE_ROWS) return VEDA_ERR_SHAPE;
  if ((s = check_raster(geo, hs, dtype, rs_b, rs_n, rs_h)) != VEDA_OK) return s;
  if (geo.padded && k_layout != VEDA_TILE_ROWS) return VEDA_ERR_UNSUPPORTED;  // padded: K tiled
  if (workspace == nullptr || workspace_bytes < tilemap_workspace_bytes(geo, n_sel)) return VEDA_ERR_WORKSPACE;
  const int64_t eb = dtype == VEDA_BF16 ? 2 : 4;
  const RasterView rv{rs_b * eb, rs_n * eb, rs_h * eb};
  return hip_status(launch_tilemap(geo, dtype, q_raster, k_raster, softmax_scale, q_tiles, n_sel, tilemap, lse,
                                   workspace, stream, &hs, &rv, k_layout == VEDA_RASTER));
}

veda_status veda_distill_step(const veda_geom *g, veda_dtype dtype, const void *q_tiled, const void *k_tiled,
                              float *w1, float *w2, int32_t mlp_hidden, int32_t mlp_out, float score_scale,
                              const int32_t *q_tiles, int32_t n_sel, const float *target, float *loss, float *dw1,
                              float *dw2, float lr, void *workspace, size_t workspace_bytes, hipStream_t stream) {
  Geo geo;
  HeadShapes hs;
  veda_status s = check_geom(g, dtype, &geo, &hs);
  if (s != VEDA_OK) return s;
  if (!q_tiled || !k_tiled || !w1 || !w2 || !q_tiles || !target || !loss || !dw1 || !dw2) return VEDA_ERR_NULL;
  if (n_sel < 1 || n_sel > geo.nt) return VEDA_ERR_SHAPE;
  if (mlp_hidden != 256 || mlp_out != 64) return VEDA_ERR_UNSUPPORTED;
  if (geo.nt > DISTILL_MAX_NT) return VEDA_ERR_UNSUPPORTED;
  const void *ptrs[] = {q_tiled, k_tiled, w1, w2, q_tiles, target, loss, dw1, dw2, workspace};
  for (const void *p : ptrs)
    if (p && !aligned16(p)) return VEDA_ERR_ALIGN;
  if (workspace == nullptr || workspace_bytes < distill_workspace_bytes(geo, n_sel)) return VEDA_ERR_WORKSPACE;
  return hip_status(launch_distill(geo, hs, dtype, q_tiled, k_tiled, w1, w2, score_scale, q_tiles, n_sel, target,
                                   loss, dw1, dw2, lr, workspace, stream));
}

size_t veda_head_sq_error_workspace_bytes(int32_t batch, int32_t n_tokens, int32_t heads) {
  if (batch < 1 || n_tokens < 1 || heads < 1) return 0;
  return (size_t)batch * heads * head_sq_error_chunks(n_tokens) * 2 * sizeof(float);
}

veda_status veda_head_sq_error(int32_t batch, int32_t n_tokens, int32_t heads, int32_t head_dim, veda_dtype dtype,
                               const void *a, const void *b, float *err, float *err_batch_sum, float *ref_sq,
                               void *workspace, size_t workspace_bytes, hipStream_t stream) {
  if (dtype != VEDA_F32 && dtype != VEDA_BF16) return VEDA_ERR_DTYPE;
  if (batch < 1 || n_tokens < 1 || heads < 1 || head_dim < 1 || batch > 65535 || heads > 65535)
    return VEDA_ERR_SHAPE;
  const int eb = dtype == VEDA_BF16 ? 2 : 4;
  if (((int64_t)head_dim * eb) % 16 != 0) return VEDA_ERR_SHAPE;
  if (!a || !b || !err) return VEDA_ERR_NULL;
  if (!aligned16(a) || !aligned16(b) || (reinterpret_cast<uintptr_t>(err) & 3u) ||
      (reinterpret_cast<uintptr_t>(ref_sq) & 3u) || (reinterpret_cast<uintptr_t>(err_batch_sum) & 3u) ||
      (reinterpret_cast<uintptr_t>(workspace) & 7u))
    return VEDA_ERR_ALIGN;
  // one chunk's 16-byte pieces are counted in 32 bits
  const int64_t chunk_rows = ((int64_t)n_tokens + head_sq_error_chunks(n_tokens) - 1) / head_sq_error_chunks(n_tokens);
  if (chunk_rows * ((int64_t)head_dim * eb / 16) >= (int64_t)1 << 31) return VEDA_ERR_UNSUPPORTED;
  if (workspace == nullptr || workspace_bytes < veda_head_sq_error_workspace_bytes(batch, n_tokens, heads))
    return VEDA_ERR_WORKSPACE;
  return hip_status(
      launch_head_sq_error(batch, n_tokens, heads, head_dim, dtype, a, b, err, err_batch_sum, ref_sq, workspace,
                           stream));
}

int64_t veda_tiled_tokens(const veda_geom *g, veda_dtype dtype) {
  Geo geo;
  HeadShapes hs;
  const veda_status s = check_geom(g, dtype, &geo, &hs);
  return s != VEDA_OK ? (int64_t)s : (int64_t)geo.N;
}

int32_t veda_head_tiles(const veda_geom *g, veda_dtype dtype, int32_t head) {
  Geo geo;
  HeadShapes hs;
  const veda_status s = check_geom(g, dtype, &geo, &hs);
  if (s != VEDA_OK) return s;
  if (head < 0 || head >= geo.H) return VEDA_ERR_SHAPE;
  return head_tiles(hs.s[head][0], hs.s[head][1], hs.s[head][2], geo.T, geo.Hs, geo.Ws);
}

const char *veda_status_str(veda_status s) {
  switch (s) {
    case VEDA_OK: return "ok";
    case VEDA_ERR_NULL: return "required pointer is NULL";
    case VEDA_ERR_SHAPE: return "inconsistent sizes or tile shapes";
    case VEDA_ERR_DTYPE: return "unknown element type";
    case VEDA_ERR_UNSUPPORTED: return "unsupported configuration";
    case VEDA_ERR_WORKSPACE: return "workspace missing or too small";
    case VEDA_ERR_ALIGN: return "pointer or stride not 16-byte aligned";
    case VEDA_ERR_HIP: return "HIP launch failed";
    case VEDA_ERR_SCRATCH: return "problem too large for the library's 32 MiB static scratch";
    default: return "unknown status";
  }
}

int veda_last_hip_error(void) { return g_last_hip_error; }

const char *veda_version(void) { return "veda-mi355x 0.1 (gfx950)"; }

}  // extern "C"
