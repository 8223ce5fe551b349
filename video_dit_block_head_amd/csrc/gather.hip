// Head-aware tiling: permutation of raster tokens into per-head (p_t, p_h, p_w) tiles.
// [Technical Summary: Veda, §2.2 Head-Aware Tiling]
//
// HBM-bound copies.  One workgroup per (tile, head, batch); every access moves 16 bytes.
// Padded tilings (shapes that do not divide the grid): the forward copy writes zero rows for
// padding rows and for the tiles past the head's own count; the inverse skips them.
#include "common.h"
#include "kernels.h"

namespace veda {

// Row layout: each 256-byte token row is copied as 16 chunks of 16 bytes; the 256 threads
// cover 16 rows per step.  EB = element bytes (2 or 4); d*EB must be 256.
template <bool INVERSE>
__global__ void __launch_bounds__(256) gather_rows_kernel(uint8_t *__restrict__ raster, int64_t rs_b, int64_t rs_n,
                                                          int64_t rs_h, uint8_t *__restrict__ tiled, Geo g,
                                                          HeadShapes hs, int eb) {
  const int j = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int pt = hs.s[h][0], ph = hs.s[h][1], pw = hs.s[h][2];
  const int chunk = threadIdx.x & 15, r0 = threadIdx.x >> 4;
  const int64_t row_bytes = (int64_t)g.d * eb;
  uint8_t *tbase = tiled + (((int64_t)b * g.H + h) * g.N + (int64_t)j * g.P) * row_bytes;
  const int64_t rb = (int64_t)b * rs_b * eb, rh = (int64_t)h * rs_h * eb;
  const bool in_head = !g.padded || j < head_tiles(pt, ph, pw, g.T, g.Hs, g.Ws);
  for (int o = r0; o < g.P; o += 16) {
    uint4 *dst_t = reinterpret_cast<uint4 *>(tbase + o * row_bytes) + chunk;
    if (g.padded && !(in_head && row_real(j, o, pt, ph, pw, g.T, g.Hs, g.Ws))) {
      if (!INVERSE) *dst_t = make_uint4(0u, 0u, 0u, 0u);
      continue;
    }
    const int64_t n = tile_row_token(j, o, pt, ph, pw, g.Hs, g.Ws);
    uint4 *src_r = reinterpret_cast<uint4 *>(raster + rb + n * rs_n * eb + rh) + chunk;
    if (INVERSE)
      *src_r = *dst_t;
    else
      *dst_t = *src_r;
  }
}

// Column layout, bf16, through LDS so that both sides are coalesced: the 256 threads first
// copy the tile's 128 token rows into LDS (16 lanes per 256-byte row, chunk c of row o at slot
// c ^ cols_slot(o)); then each thread gathers one 8-position x 8-channel block (eight 16-byte
// LDS reads), transposes it in registers and writes 8 channel rows; the 16 lanes that share a
// channel row write it whole (256 contiguous bytes).  The swizzle gives the 16 rows that one
// read instruction touches per channel block 16 different slots, so neither the copy in nor
// the reads out have bank conflicts.  Each tile is written channel-major ([d][P]) with the
// key order of cols_key().
__device__ __forceinline__ int cols_slot(int o) { return (((o >> 4) << 1) | ((o >> 2) & 1)) & 15; }

__global__ void __launch_bounds__(256) gather_cols_bf16_kernel(const uint16_t *__restrict__ raster, int64_t rs_b,
                                                               int64_t rs_n, int64_t rs_h,
                                                               uint16_t *__restrict__ tiled, Geo g, HeadShapes hs) {
  const int j = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int pt = hs.s[h][0], ph = hs.s[h][1], pw = hs.s[h][2];
  const int t = threadIdx.x;
  const bool in_head = !g.padded || j < head_tiles(pt, ph, pw, g.T, g.Hs, g.Ws);
  __shared__ uint4 tile[128 * 16];
  {
    const int c = t & 15, r0 = t >> 4;
    uint4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int o = r0 + 16 * i;
      v[i] = make_uint4(0u, 0u, 0u, 0u);  // padding rows are zero
      if (!g.padded || (in_head && row_real(j, o, pt, ph, pw, g.T, g.Hs, g.Ws))) {
        const int64_t n = tile_row_token(j, o, pt, ph, pw, g.Hs, g.Ws);
        v[i] = *reinterpret_cast<const uint4 *>(raster + b * rs_b + n * rs_n + h * rs_h + c * 8);
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int o = r0 + 16 * i;
      tile[o * 16 + (c ^ cols_slot(o))] = v[i];
    }
  }
  __syncthreads();
  const int tb = t & 15, cb = t >> 4;  // position block (8 keys), channel block (8 channels)
  uint32_t in[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int o = cols_key(tb * 8 + i);
    const uint4 v = tile[o * 16 + (cb ^ cols_slot(o))];
    in[i][0] = v.x;
    in[i][1] = v.y;
    in[i][2] = v.z;
    in[i][3] = v.w;
  }
  uint16_t *tbase = tiled + (((int64_t)b * g.H + h) * g.nt + j) * (int64_t)g.d * g.P;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int w = c >> 1;
    uint32_t o[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t a = in[2 * p][w], bb = in[2 * p + 1][w];
      o[p] = (c & 1) ? ((a >> 16) | (bb & 0xFFFF0000u)) : ((a & 0xFFFFu) | (bb << 16));
    }
    *reinterpret_cast<uint4 *>(tbase + (int64_t)(cb * 8 + c) * g.P + tb * 8) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// Column layout, f32 (small problems only): one thread per element.
__global__ void __launch_bounds__(256) gather_cols_f32_kernel(const float *__restrict__ raster, int64_t rs_b,
                                                              int64_t rs_n, int64_t rs_h, float *__restrict__ tiled,
                                                              Geo g, HeadShapes hs) {
  const int j = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int pt = hs.s[h][0], ph = hs.s[h][1], pw = hs.s[h][2];
  float *tbase = tiled + (((int64_t)b * g.H + h) * g.nt + j) * (int64_t)g.d * g.P;
  const bool in_head = !g.padded || j < head_tiles(pt, ph, pw, g.T, g.Hs, g.Ws);
  for (int e = threadIdx.x; e < g.P * g.d; e += blockDim.x) {
    const int p = e % g.P, c = e / g.P, o = cols_key(p);
    if (g.padded && !(in_head && row_real(j, o, pt, ph, pw, g.T, g.Hs, g.Ws))) {
      tbase[(int64_t)c * g.P + p] = 0.f;
      continue;
    }
    const int64_t n = tile_row_token(j, o, pt, ph, pw, g.Hs, g.Ws);
    tbase[(int64_t)c * g.P + p] = raster[b * rs_b + n * rs_n + h * rs_h + c];
  }
}

hipError_t launch_gather(const Geo &g, const HeadShapes &hs, veda_dtype dt, void *raster, int64_t rs_b,
                         int64_t rs_n, int64_t rs_h, void *tiled, veda_layout layout, int inverse,
                         hipStream_t st) {
  const dim3 grid(g.nt, g.H, g.B), block(256);
  const int eb = dt == VEDA_BF16 ? 2 : 4;
  if (layout == VEDA_TILE_ROWS) {
    if (inverse)
      gather_rows_kernel<true><<<grid, block, 0, st>>>((uint8_t *)raster, rs_b, rs_n, rs_h, (uint8_t *)tiled, g, hs,
                                                       eb);
    else
      gather_rows_kernel<false><<<grid, block, 0, st>>>((uint8_t *)raster, rs_b, rs_n, rs_h, (uint8_t *)tiled, g,
                                                        hs, eb);
  } else if (dt == VEDA_BF16) {
    gather_cols_bf16_kernel<<<grid, block, 0, st>>>((const uint16_t *)raster, rs_b, rs_n, rs_h, (uint16_t *)tiled,
                                                    g, hs);
  } else {
    gather_cols_f32_kernel<<<grid, block, 0, st>>>((const float *)raster, rs_b, rs_n, rs_h, (float *)tiled, g, hs);
  }
  return hipGetLastError();
}

}  // namespace veda
