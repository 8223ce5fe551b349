// Oracle tile map: max-pooling of the full-attention probabilities over each
// (query tile x key tile) region.  [Technical Summary: Veda, §2.1 "Target Construction";
// §2.3: ground-truth heatmaps in two passes, on subsets of query tiles]
//
// bf16 path: one workgroup (4 waves x 64 queries) per two selected query tiles of a head and
// one of S contiguous ranges of its key tiles (S chosen so that the workgroups fill whole
// rounds of the chip; a last round left half empty cost about a sixth of the time).
//  pass 1 (a sweep over the range's keys): S^T = K Q^T per key tile (MFMA, same blocking as
//          the attention kernel; K tiles double-buffered in LDS through direct-to-LDS
//          copies); per query row the range's log-sum-exp terms (log2 domain, lazy max: the
//          running max m and sum l) and the row max of each key tile, m[q][j] = max_x
//          s(q, x) * c, written to the workspace;
//  pass 2 (tilemap_pool_kernel): lse2[q] from the S (m, l) pairs, then M[j] = exp2(max over
//          the tile's queries of m[q][j] - lse2[q]) from the workspace (no second Q K^T).
// exp is monotone, so this is the max over the region of exp(s - lse).
#include "common.h"
#include "kernels.h"

namespace veda {

static constexpr float TM_LOG2E = 1.4426950408889634f;
static constexpr float TM_LN2 = 0.6931471805599453f;
static constexpr float TM_SLACK = 8.0f;  // lazy running-max slack (log2 units)
static constexpr int TM_MAX_NT = 1280;

static constexpr int TM_MAX_SPLITS = 4;

static inline size_t tm_align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Row maxima [B, H, n_sel, nt, P] f32, then the per-range (m, l) pairs [B, H, n_sel, S, P].
size_t tilemap_workspace_bytes(const Geo &g, int n_sel) {
  return tm_align256((size_t)g.B * g.H * n_sel * (size_t)g.nt * g.P * sizeof(float)) +
         (size_t)g.B * g.H * n_sel * TM_MAX_SPLITS * g.P * sizeof(float2);
}

// Two selected query tiles (of one head) per workgroup: they sweep the same K tiles, so wave
// w takes 64 queries of query tile w/2 as two 32-query blocks that share every K operand
// read (half the LDS traffic per MFMA) and every K tile is copied once for both tiles.
static constexpr int TM_QT = 2;

// RQ (RK): Q (K) is a raster [B, N, H, d] tensor (byte strides in rv) read through the
// head's tiling (token of row r of tile j = origin(j) + intra(r)); otherwise tile-major.
// PAD: padded tiling: per-head tile counts, partial tiles (K tiled); with RQ the padding
// query rows of a partial tile are not read (Q taken as zero, as the gather stores it).
// Maximum of v over lanes l and l ^ 32, the two halves of a query row's lane pair, with
// v_permlane32_swap (a VALU op; a shuffle would go through the LDS and its latency).
__device__ __forceinline__ float pair_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

template <bool RQ, bool RK, bool PAD>
__global__ void __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2, 2)))
tilemap_bf16_kernel(const __bf16 *__restrict__ q, const __bf16 *__restrict__ k, float c2,
                    const int32_t *__restrict__ q_tiles, int n_sel, int splits, float *__restrict__ rowmax,
                    float2 *__restrict__ part, Geo g, HeadShapes hs, RasterView rv) {
  // items ordered (b, h, key range, query-tile pair): each XCD walks consecutive pairs that
  // sweep the same key tiles
  const int ngrp = (n_sel + TM_QT - 1) / TM_QT;
  const int L = xcd_tile(blockIdx.x, gridDim.x);
  const int a0 = (L % ngrp) * TM_QT;
  const int sp = (L / ngrp) % splits;
  const int64_t bh = L / (ngrp * splits);
  const int t = threadIdx.x, lane = t & 63, lr = lane & 31, hi = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int qt = w >> 1;                     // which of the workgroup's query tiles
  const int a = min(a0 + qt, n_sel - 1);     // an odd tail repeats the last tile (not written twice)
  const bool owner = a0 + qt < n_sel;
  const int hh = (int)(bh % g.H), bb = (int)(bh / g.H);
  const int pt = hs.s[hh][0], ph = hs.s[hh][1], pw = hs.s[hh][2];
  // this head's tiles (fewer than nt for a head of a padded tiling with fewer tiles)
  const int nth = PAD ? head_tiles(pt, ph, pw, g.T, g.Hs, g.Ws) : g.nt;
  const int i = q_tiles ? min(max(q_tiles[bh * n_sel + a], 0), nth - 1) : a;  // clamped
  const int j0 = (int)((int64_t)nth * sp / splits), j1 = (int)((int64_t)nth * (sp + 1) / splits);  // key range
  const int64_t rhead = (int64_t)bb * rv.sb + (int64_t)hh * rv.sh;
  const __bf16 *qh = q + bh * (int64_t)g.N * 128;
  const char *kh = RK ? reinterpret_cast<const char *>(k) + rhead
                          : reinterpret_cast<const char *>(k + bh * (int64_t)g.N * 128);
  auto k_tile = [&](int j) -> const char * {
    return RK ? kh + tile_origin(j, pt, ph, pw, g.Hs, g.Ws) * rv.sn : kh + (int64_t)j * 32768;
  };
  float *rm = rowmax + (bh * n_sel + a) * (int64_t)g.nt * 128;   // [j][128 queries]

  __shared__ uint4 Kb[2][128 * 16];

  bf16x8_t qf[2][8];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int r = 64 * (w & 1) + 32 * qb + lr;
    // origin + intra names a real token unless the row is padding of a partial tile
    const bool real = !(RQ && PAD) || row_real(i, r, pt, ph, pw, g.T, g.Hs, g.Ws);
    const __bf16 *qp =
        RQ ? reinterpret_cast<const __bf16 *>(reinterpret_cast<const char *>(q) + rhead +
                                                  (tile_origin(i, pt, ph, pw, g.Hs, g.Ws) +
                                                   tile_intra(r, ph, pw, g.Hs, g.Ws)) * rv.sn)
               : qh + ((int64_t)i * 128 + r) * 128;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      if (real) {
        qf[qb][s] = *reinterpret_cast<const bf16x8_t *>(qp + 16 * s + 8 * hi);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[qb][s][e] = (__bf16)0.0f;
      }
    }
  }
  asm volatile("" ::"v"(qf[0][0]), "v"(qf[0][1]), "v"(qf[0][2]), "v"(qf[0][3]), "v"(qf[0][4]), "v"(qf[0][5]),
               "v"(qf[0][6]), "v"(qf[0][7]));
  asm volatile("" ::"v"(qf[1][0]), "v"(qf[1][1]), "v"(qf[1][2]), "v"(qf[1][3]), "v"(qf[1][4]), "v"(qf[1][5]),
               "v"(qf[1][6]), "v"(qf[1][7]));

  uint32_t off[8];
  if (RK)
    tile_dma_offsets_raster(w, lane, ph, pw, g.Hs, g.Ws, rv.sn, off);
  else
    tile_dma_offsets(w, lane, off);
  const uint32_t kb_lds[2] = {lds_addr(Kb[0]), lds_addr(Kb[1])};
  if (j0 < j1) tile_to_lds(k_tile(j0), kb_lds[0], w, off);
  if (j0 + 1 < j1) tile_to_lds(k_tile(j0 + 1), kb_lds[1], w, off);

  float m_run[2] = {-1e30f, -1e30f}, l_run[2] = {0.f, 0.f};
  for (int j = j0; j < j1; ++j) {
    const int buf = (j - j0) & 1;
    if (j + 1 < j1)
      wait_vmem<8>();  // tile j+1's copies may still be in flight
    else
      wait_vmem<0>();
    barrier();
    f32x16_t acc[2][4];
    const uint4 *Ks = Kb[buf];
    // A padding key of a partial tile (padded tilings only) starts at -inf: its K row is
    // zero, so the MFMAs leave it there and it gets no probability.  Entry (kb, r) of this
    // lane is key row 32 kb + 8 (r / 4) + 4 hi + r % 4 of the tile.
    const TileBox bx = PAD ? tile_box(j, pt, ph, pw, g.T, g.Hs, g.Ws) : TileBox{128, 1, 1};
    if (box_rows(bx) < 128) {
      uint32_t wd[4];
      tile_row_words(bx, ph, pw, lane, wd);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float z = (wd[kb] >> (8 * (r >> 2) + (r & 3))) & 1u ? 0.f : -INFINITY;
          acc[0][kb][r] = z;
          acc[1][kb][r] = z;
        }
    } else {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          acc[0][kb][r] = 0.f;
          acc[1][kb][r] = 0.f;
        }
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int row = 32 * kb + lr;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const bf16x8_t av = *reinterpret_cast<const bf16x8_t *>(&Ks[row * 16 + ((2 * s + hi) ^ (row & 15))]);
        acc[0][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qf[0][s], acc[0][kb], 0, 0, 0);
        acc[1][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qf[1][s], acc[1][kb], 0, 0, 0);
      }
    }
    wait_lds();
    barrier();  // every wave has read this buffer
    if (j + 2 < j1) tile_to_lds(k_tile(j + 2), kb_lds[buf], w, off);

#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float mx = -1e30f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc[qb][kb][r]);
      mx = pair_max(mx) * c2;
      if (hi == 0 && owner) rm[(int64_t)j * 128 + 64 * (w & 1) + 32 * qb + lr] = mx;
      if (__ballot(mx > m_run[qb] + TM_SLACK)) {
        const float m_new = fmaxf(m_run[qb], mx);
        l_run[qb] *= __builtin_amdgcn_exp2f(m_run[qb] - m_new);
        m_run[qb] = m_new;
      }
      float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) ls[r & 3] += __builtin_amdgcn_exp2f(fmaf(acc[qb][kb][r], c2, -m_run[qb]));
      l_run[qb] += (ls[0] + ls[1]) + (ls[2] + ls[3]);
    }
  }
  // this range's (m, l) per query row: l summed over both halves of the lane pair
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float l = l_run[qb] + __shfl_xor(l_run[qb], 32);
    const int qi = 64 * (w & 1) + 32 * qb + lr;
    if (hi == 0 && owner) part[((bh * n_sel + a) * splits + sp) * 128 + qi] = make_float2(m_run[qb], l);
  }
}

// Pass 2, one workgroup per selected query tile: lse2[q] = log2 of the sum over the ranges of
// l * 2^m, then M[j] = exp2(max over the tile's queries of rowmax[j][q] - lse2[q]).
template <bool PAD>
__global__ void __launch_bounds__(256) tilemap_pool_kernel(const float *__restrict__ rowmax,
                                                           const float2 *__restrict__ part, int splits,
                                                           const int32_t *__restrict__ q_tiles, int n_sel,
                                                           float *__restrict__ out, float *__restrict__ lse_out,
                                                           Geo g, HeadShapes hs) {
  const int64_t bh = blockIdx.x;
  const int a = blockIdx.y;
  const int t = threadIdx.x, hh = (int)(bh % g.H);
  const int pt = hs.s[hh][0], ph = hs.s[hh][1], pw = hs.s[hh][2];
  const int nth = PAD ? head_tiles(pt, ph, pw, g.T, g.Hs, g.Ws) : g.nt;
  __shared__ float lse_s[128];
  if (t < 128) {
    const float2 *pp = part + (bh * n_sel + a) * splits * 128 + t;
    float m = -1e30f;
    for (int s = 0; s < splits; ++s) m = fmaxf(m, pp[s * 128].x);
    float l = 0.f;
    for (int s = 0; s < splits; ++s) l += pp[s * 128].y * __builtin_amdgcn_exp2f(pp[s * 128].x - m);
    const float lse2 = m + log2f(l);
    if (lse_out != nullptr) lse_out[(bh * n_sel + a) * 128 + t] = lse2 * TM_LN2;
    bool real = true;
    if (PAD) {  // a padding query row of a padded tiling stays out of the pooled maximum
      const int i = q_tiles ? min(max(q_tiles[bh * n_sel + a], 0), nth - 1) : a;
      real = row_real(i, t, pt, ph, pw, g.T, g.Hs, g.Ws);
    }
    lse_s[t] = real ? lse2 : INFINITY;
  }
  __syncthreads();
  for (int j = t; j < g.nt; j += 256) {
    float *o = out + (bh * n_sel + a) * (int64_t)g.nt + j;
    if (j >= nth) {  // past this head's tiles
      *o = 0.f;
      continue;
    }
    const float4 *src = reinterpret_cast<const float4 *>(rowmax + ((bh * n_sel + a) * (int64_t)g.nt + j) * 128);
    float x = -INFINITY;
#pragma unroll 8
    for (int c = 0; c < 32; ++c) {
      const float4 v = src[c];
      x = fmaxf(x, fmaxf(fmaxf(v.x - lse_s[4 * c], v.y - lse_s[4 * c + 1]),
                         fmaxf(v.z - lse_s[4 * c + 2], v.w - lse_s[4 * c + 3])));
    }
    *o = __builtin_amdgcn_exp2f(x);
  }
}

// fp32 path (d = 64, P = 64): one thread per query row.
template <bool RQ, bool RK>
__global__ void __launch_bounds__(64) tilemap_f32_kernel(const float *__restrict__ q, const float *__restrict__ k,
                                                         float scale, const int32_t *__restrict__ q_tiles, int n_sel,
                                                         float *__restrict__ out, float *__restrict__ lse_out, Geo g,
                                                         HeadShapes hs, RasterView rv) {
  const int a = blockIdx.x, h = blockIdx.y, b = blockIdx.z, t = threadIdx.x;
  const int64_t bh = (int64_t)b * g.H + h;
  const int i = q_tiles ? min(max(q_tiles[bh * n_sel + a], 0), g.nt - 1) : a;
  const float *qh = q + bh * (int64_t)g.N * 64, *kh = k + bh * (int64_t)g.N * 64;
  const int pt = hs.s[h][0], ph = hs.s[h][1], pw = hs.s[h][2];
  const int64_t rhead = (int64_t)b * rv.sb + (int64_t)h * rv.sh;
  // element index of (tiled row, channel) of Q or K in either layout
  auto at = [&](bool raster, int row, int c) -> int64_t {
    if (!raster) return (int64_t)row * 64 + c;
    const int64_t tok = tile_origin(row / 64, pt, ph, pw, g.Hs, g.Ws) + tile_intra(row % 64, ph, pw, g.Hs, g.Ws);
    return (rhead + tok * rv.sn) / 4 + c;
  };
  const float *qb = RQ ? q : qh, *kb = RK ? k : kh;
  float qr[64];
#pragma unroll
  for (int c = 0; c < 64; ++c) qr[c] = qb[at(RQ, i * 64 + t, c)];
  __shared__ float Ks[64][65];
  __shared__ float wm[TM_MAX_NT];
  float m = -1e30f, l = 0.f;
  for (int pass = 0; pass < 2; ++pass) {
    const float lse = m + logf(l);
    for (int j = 0; j < g.nt; ++j) {
      __syncthreads();
      for (int e = t; e < 64 * 64; e += 64) Ks[e >> 6][e & 63] = kb[at(RK, j * 64 + (e >> 6), e & 63)];
      __syncthreads();
      float tmax = -1e30f;
      for (int x = 0; x < 64; ++x) {
        float s = 0.f;
#pragma unroll
        for (int c = 0; c < 64; ++c) s = fmaf(qr[c], Ks[x][c], s);
        s *= scale;
        if (pass == 0) {
          const float m_new = fmaxf(m, s);
          l = l * expf(m - m_new) + expf(s - m_new);
          m = m_new;
        } else {
          tmax = fmaxf(tmax, s);
        }
      }
      if (pass == 1) {
        const float x = wave_max(tmax - lse);
        if (t == 0) wm[j] = x;
      }
    }
    if (pass == 0 && lse_out != nullptr) lse_out[bh * (int64_t)n_sel * 64 + (int64_t)a * 64 + t] = m + logf(l);
  }
  __syncthreads();
  for (int j = t; j < g.nt; j += 64) out[(bh * n_sel + a) * (int64_t)g.nt + j] = expf(wm[j]);
}

// Key ranges per query-tile pair: the S in 1..TM_MAX_SPLITS for which the workgroups
// (two per CU) fill their last round best; at most the smallest per-head tile count.
static int tilemap_splits(int groups, const Geo &g, const HeadShapes &hs) {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) n = 256;
    cus[dev] = n;
  }
  const int64_t slots = 2 * (int64_t)cus[dev];
  int nt_min = g.nt;
  if (g.padded)
    for (int h = 0; h < g.H; ++h) nt_min = std::min(nt_min, head_tiles(hs.s[h][0], hs.s[h][1], hs.s[h][2], g.T, g.Hs, g.Ws));
  int best = 1;
  double best_cost = (double)((groups + slots - 1) / slots);
  for (int s = 2; s <= TM_MAX_SPLITS && s <= nt_min; ++s) {
    const double cost = (double)(((int64_t)groups * s + slots - 1) / slots) / s;  // rounds, in whole-sweep units
    if (cost < best_cost - 1e-9) {
      best = s;
      best_cost = cost;
    }
  }
  return best;
}

template <bool RQ, bool RK>
static void launch_tilemap_t(const Geo &g, const HeadShapes &hs, const RasterView &rv, veda_dtype dt, const void *q,
                             const void *k, float scale, const int32_t *q_tiles, int n_sel, float *tilemap,
                             float *lse, void *ws, hipStream_t st) {
  if (dt == VEDA_BF16) {
    const int groups = ((n_sel + TM_QT - 1) / TM_QT) * g.H * g.B;
    const int splits = tilemap_splits(groups, g, hs);
    float *rowmax = static_cast<float *>(ws);
    float2 *part = reinterpret_cast<float2 *>(static_cast<char *>(ws) +
                                              tm_align256((size_t)g.B * g.H * n_sel * (size_t)g.nt * g.P * sizeof(float)));
    const dim3 grid(groups * splits), pgrid(g.H * g.B, n_sel);
    const __bf16 *qq = (const __bf16 *)q, *kk = (const __bf16 *)k;
    if (!RK && g.padded) {  // padded tilings read K tiled (the C ABI refuses a raster K)
      tilemap_bf16_kernel<RQ, false, true><<<grid, 256, 0, st>>>(qq, kk, scale * TM_LOG2E, q_tiles, n_sel, splits,
                                                                 rowmax, part, g, hs, rv);
      tilemap_pool_kernel<true><<<pgrid, 256, 0, st>>>(rowmax, part, splits, q_tiles, n_sel, tilemap, lse, g, hs);
    } else {
      tilemap_bf16_kernel<RQ, RK, false><<<grid, 256, 0, st>>>(qq, kk, scale * TM_LOG2E, q_tiles, n_sel, splits,
                                                               rowmax, part, g, hs, rv);
      tilemap_pool_kernel<false><<<pgrid, 256, 0, st>>>(rowmax, part, splits, q_tiles, n_sel, tilemap, lse, g, hs);
    }
  } else
    tilemap_f32_kernel<RQ, RK><<<dim3(n_sel, g.H, g.B), 64, 0, st>>>((const float *)q, (const float *)k, scale,
                                                                     q_tiles, n_sel, tilemap, lse, g, hs, rv);
}

hipError_t launch_tilemap(const Geo &g, veda_dtype dt, const void *q, const void *k, float scale,
                          const int32_t *q_tiles, int n_sel, float *tilemap, float *lse, void *ws, hipStream_t st,
                          const HeadShapes *hs, const RasterView *rv, bool k_raster) {
  if (rv == nullptr)
    launch_tilemap_t<false, false>(g, hs != nullptr ? *hs : HeadShapes{}, RasterView{0, 0, 0}, dt, q, k, scale, q_tiles, n_sel, tilemap,
                                   lse, ws, st);
  else if (k_raster)
    launch_tilemap_t<true, true>(g, *hs, *rv, dt, q, k, scale, q_tiles, n_sel, tilemap, lse, ws, st);
  else
    launch_tilemap_t<true, false>(g, *hs, *rv, dt, q, k, scale, q_tiles, n_sel, tilemap, lse, ws, st);
  return hipGetLastError();
}

}  // namespace veda
