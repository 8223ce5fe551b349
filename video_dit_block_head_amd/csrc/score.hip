// Distilled tile scoring: TripPool descriptors -> per-head MLP -> tile scores -> row
// softmax / top-k.  [Technical Summary: Veda, §2.1 Distilled Tile Scoring]
//
//  pool_mlp_kernel   32 tiles of one (head, batch, Q|K) per workgroup.  Each wave streams 8
//                    tiles (HBM-bound: non-temporal 16-byte loads, 32 per lane in flight, so
//                    the stream does not evict the MLP weights from L2) into their
//                    [mean|max|min] descriptors, then the workgroup runs the MLP on fp32
//                    MFMA: layer 1 32x3d @ 3d x256 (v_mfma_f32_32x32x2f32, 64 hidden units
//                    per wave), exact-erf GELU, layer 2 32x256 @ 256x64
//                    (v_mfma_f32_16x16x4f32, 16 outputs per wave).  Three workgroups per
//                    CU, so other workgroups' streaming overlaps one's MFMA work.  For the
//                    distillation step it can take a list of Q tiles and also keep the
//                    pre-activation hidden layer.  Reading a raster K, it can also write
//                    K's tile-major copy as it streams it (the K gather fused into pooling),
//                    and with raster Q, workgroups of a third kind stream a raster V into
//                    its tile-major copy (the V gather in the same launch, filling the HBM
//                    time that the others spend in the MLP).
//  score_topk_kernel 16 query-tile rows per workgroup: S = y_q y_k^T on fp32 MFMA
//                    (v_mfma_f32_16x16x4f32) into an LDS row block, then one wave per row
//                    for softmax and top-k (ballot/popcount; deterministic); 4, 8 or 16
//                    waves per workgroup by row length.
//  topk_kernel       standalone top-k, one wave per row.
#include "common.h"
#include "kernels.h"

namespace veda {

static constexpr int PM_ROWS = 32;    // descriptors per workgroup
static constexpr int PM_DS = 385;     // LDS row stride (floats) of the descriptor block
static constexpr int PM_HS = 257;     // LDS row stride (floats) of the hidden block
static constexpr int MLP_HIDDEN = 256, MLP_OUT = 64;

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t score_workspace_bytes(const Geo &g, int hidden, int mlp_out) {
  (void)hidden;
  const size_t nt = (size_t)g.B * g.H * g.nt;
  return align256(2 * nt * mlp_out * sizeof(float));
}

__device__ __forceinline__ float gelu_erf(float x) { return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f)); }

// ---------------------------------------------------------------------------------------
// TripPool + MLP on 32 tiles of one (Q|K, batch, head) per workgroup (4 waves; three
// workgroups fit a CU, so other workgroups stream while one runs its MLP).
//   pooling: wave w pools tiles 8w .. 8w + 7, 32 16-byte loads per lane in flight;
//   layer 1: fp32 MFMA 32x32x2 (A[m = lane%32][k = lane/32], B[k = lane/32][n = lane%32]),
//            64 hidden units per wave (two per lane column, so one 8-byte weight load per
//            lane and step), weights prefetched PF steps ahead in registers;
//   GELU (exact erf) into the hidden block, in place of the descriptors;
//   layer 2: fp32 MFMA 16x16x4, 16 outputs per wave for all 32 rows (no cross-wave sum).
// EB: element bytes (2: bf16 with d = P = 128; 4: f32 with d = P = 64).  Rows are 256 bytes.
static constexpr int PM_HST = 260;    // hidden block row stride (floats)

// RQ (RK): Q (K) is a raster [B, N, H, d] tensor (byte strides in rv) read through each
// head's tiling (token of row r of tile j = origin(j) + intra(r)); otherwise tile-major.
// PAD: padded tiling: per-head tile counts, partial tiles (their real rows only).
// vout (RQ only, else null): the items are (b, h, Q|K|V, group), and a V item copies its 32
// tiles of the raster V vsrc (strides of Q) to their tile-major place in vout, as the K
// items write kout (zero rows where the tiling has no token), and does nothing else.
// kbound (nullable): [B, H, nt], for each key tile sqrt(sum over channels of
// max(max^2, min^2)) from its max and min descriptors, an upper bound of the norm of each
// of its key rows (0 for tiles past a padded head's own count).
template <int EB, bool RQ, bool RK, bool PAD>
__global__ void __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(3, 3)))
pool_mlp_kernel(const uint8_t *__restrict__ q, const uint8_t *__restrict__ k, const float *__restrict__ w1q,
                const float *__restrict__ w2q, const float *__restrict__ w1k, const float *__restrict__ w2k,
                float *__restrict__ y, float *__restrict__ qdesc, float *__restrict__ kdesc, float *__restrict__ zout,
                const int32_t *__restrict__ qlist, int nlist, Geo g, HeadShapes hs, RasterView rv,
                uint8_t *__restrict__ kout, const uint8_t *__restrict__ vsrc, uint8_t *__restrict__ vout,
                float *__restrict__ kbound) {
  constexpr int EPC = 16 / EB;            // channels per 16-byte chunk
  constexpr int P = EB == 2 ? 128 : 64;   // tokens per tile
  constexpr int D = EB == 2 ? 128 : 64;   // head dim
  constexpr int D3 = 3 * D;
  constexpr int PF = 8;                   // weight prefetch distance (MFMA steps)
  // Items ordered (b, h, Q|K[|V], group); each XCD walks a contiguous range, so the
  // workgroups that share a head's weights share that XCD's L2.
  const int ngrp = (g.nt + PM_ROWS - 1) / PM_ROWS;
  const int nwh = (RQ && vout != nullptr) ? 3 : 2;
  const int L = xcd_tile(blockIdx.x, gridDim.x);
  const int r0 = (L % ngrp) * PM_ROWS, which = (L / ngrp) % nwh, h = (L / (nwh * ngrp)) % g.H,
            b = L / (nwh * ngrp * g.H);
  const bool vcopy = which == 2;  // uniform: a V item (copy only)
  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);  // wave index (uniform)
  __shared__ float Ds[PM_ROWS * PM_DS];   // descriptors, then the hidden layer

  // ---- TripPool: lane (rg = lane/16, c = lane%16) accumulates rows rg, rg + 4, ... of its
  // 16-byte channel chunk c; the 4 row groups are combined as (g0 + g1) + (g2 + g3).
  const int pt = hs.s[h][0], ph = hs.s[h][1], pw = hs.s[h][2];
  const bool rast = which == 0 ? RQ : (which == 1 ? RK : true);  // uniform over the workgroup
  const int nth = PAD ? head_tiles(pt, ph, pw, g.T, g.Hs, g.Ws) : g.nt;  // this head's tiles
  // With a query-tile list, the Q rows are its entries (row r pools tile qlist[b, h, r]) and
  // there are nlist of them; groups past the list have nothing to do.
  const bool listed = qlist != nullptr && which == 0;
  if (listed && r0 >= nlist) return;  // whole workgroup, before any barrier
  const int32_t *qrow = listed ? qlist + ((int64_t)b * g.H + h) * nlist : nullptr;
  const uint8_t *base = which == 0 ? q : (which == 1 ? k : vsrc);
  const uint8_t *src0 = rast ? base + (int64_t)b * rv.sb + (int64_t)h * rv.sh
                             : base + ((int64_t)b * g.H + h) * (int64_t)g.N * D * EB;
  const int rg = lane >> 4, c = lane & 15;
#pragma unroll 1
  for (int tt = 0; tt < 8; ++tt) {
    const int row = 8 * w + tt;
    // the tile this row pools; nth (no tile) past the end
    const int j = listed ? (r0 + row < nlist ? min(max(qrow[r0 + row], 0), nth - 1) : nth) : r0 + row;
    float s[EPC], mx[EPC], mn[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      s[e] = 0.f;
      mx[e] = -INFINITY;
      mn[e] = INFINITY;
    }
    const TileBox bx = PAD ? tile_box(j, pt, ph, pw, g.T, g.Hs, g.Ws) : TileBox{P, 1, 1};
    auto accum = [&](const uint4 &v) {
      float x[EPC];
      const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
      if (EB == 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[2 * e] = __uint_as_float(wd[e] << 16);
          x[2 * e + 1] = __uint_as_float(wd[e] & 0xFFFF0000u);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = __uint_as_float(wd[e]);
      }
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        s[e] += x[e];
        mx[e] = fmaxf(mx[e], x[e]);
        mn[e] = fminf(mn[e], x[e]);
      }
    };
    // K's (raster K only) or V's tile-major copy, if asked for: rows as loaded; zero rows
    // for the padding rows of a partial tile and for the tiles past this head's own count
    uint8_t *cdst = (RK && which == 1) ? kout : (vcopy ? vout : nullptr);
    uint8_t *kdst = cdst != nullptr
                        ? cdst + ((int64_t)b * g.H + h) * (int64_t)g.N * 256 + (int64_t)j * P * 256 + c * 16
                        : nullptr;
    if (j < nth && PAD && box_rows(bx) < P) {
      // a partial tile of a padded tiling: its real rows only (raster rows at origin +
      // intra, which names a real token only inside the tile's box), eight loads in flight
      // per lane; each lane still takes its rows in increasing order
      const uint8_t *src = rast ? src0 + tile_origin(j, pt, ph, pw, g.Hs, g.Ws) * rv.sn + c * 16
                                : src0 + (int64_t)j * P * 256 + c * 16;
      const int64_t rstride = rast ? rv.sn : 256;
#pragma unroll 1
      for (int o0 = rg; o0 < P; o0 += 32) {
        uint4 v[8];
        bool real[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int o = o0 + 4 * i;
          real[i] = in_box(o, ph, pw, bx);
          v[i] = make_uint4(0u, 0u, 0u, 0u);
          if (real[i]) {
            const int64_t ro = rast ? (int64_t)tile_intra(o, ph, pw, g.Hs, g.Ws) * rstride : (int64_t)o * 256;
            v[i] = load_stream16(src + ro);
          }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          if (real[i] && !vcopy) accum(v[i]);
          if (kdst != nullptr) store_stream16(kdst + (o0 + 4 * i) * 256, v[i]);  // zero rows for padding
        }
      }
    } else if (PAD && j >= nth && j < g.nt) {
      if (kdst != nullptr)
        for (int o = rg; o < P; o += 4) store_stream16(kdst + o * 256, make_uint4(0u, 0u, 0u, 0u));
    } else if (j < nth) {
      // raster rows: 32-bit offsets from the tile's origin, half a tile (16 loads) at a time
      constexpr int NL = (RQ || RK) ? P / 8 : P / 4;
#pragma unroll 1
      for (int part = 0; part < P / 4 / NL; ++part) {
        uint4 v[NL];
        if ((RQ || RK) && rast) {
          const uint8_t *src = src0 + tile_origin(j, pt, ph, pw, g.Hs, g.Ws) * rv.sn + c * 16;
#pragma unroll
          for (int i = 0; i < NL; ++i)
            v[i] = load_stream16(src + (uint32_t)(tile_intra(rg + 4 * (NL * part + i), ph, pw, g.Hs, g.Ws) * (int)rv.sn));
          if (kdst != nullptr) {  // uniform: K's tile-major copy, rows as loaded
#pragma unroll
            for (int i = 0; i < NL; ++i) store_stream16(kdst + (rg + 4 * (NL * part + i)) * 256, v[i]);
          }
        } else {
          const uint8_t *src = src0 + (int64_t)j * P * 256 + c * 16;
#pragma unroll
          for (int i = 0; i < NL; ++i) v[i] = load_stream16(src + (rg + 4 * (NL * part + i)) * 256);
        }
        if (!vcopy) {
#pragma unroll
          for (int i = 0; i < NL; ++i) accum(v[i]);
        }
      }
    }
    if (vcopy) continue;  // a V item only copies
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      s[e] += __shfl_xor(s[e], 16);
      mx[e] = fmaxf(mx[e], __shfl_xor(mx[e], 16));
      mn[e] = fminf(mn[e], __shfl_xor(mn[e], 16));
      s[e] += __shfl_xor(s[e], 32);
      mx[e] = fmaxf(mx[e], __shfl_xor(mx[e], 32));
      mn[e] = fminf(mn[e], __shfl_xor(mn[e], 32));
    }
    if (rg == 0) {
      const bool ok = j < nth;
      // mean over the tile's real rows (all P of them unless the tiling is padded)
      const float inv_cnt = 1.0f / (float)(PAD && ok ? box_rows(bx) : P);  // exact for P = 2^n
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        Ds[row * PM_DS + c * EPC + e] = ok ? s[e] * inv_cnt : 0.f;
        Ds[row * PM_DS + D + c * EPC + e] = ok ? mx[e] : 0.f;
        Ds[row * PM_DS + 2 * D + c * EPC + e] = ok ? mn[e] : 0.f;
      }
    }
  }
  if (vcopy) return;  // whole workgroup, before any barrier
  __syncthreads();
  float *dout = which ? kdesc : qdesc;
  if (dout != nullptr) {
    for (int e = t; e < PM_ROWS * D3; e += 256) {
      const int row = e / D3, col = e % D3;
      if (r0 + row < g.nt) dout[(((int64_t)b * g.H + h) * g.nt + r0 + row) * D3 + col] = Ds[row * PM_DS + col];
    }
  }
  if (which == 1 && kbound != nullptr) {  // uniform: each key tile's row-norm bound, 8 lanes per row
    const int row = t >> 3, part = t & 7, j = r0 + row;
    float nb = 0.f;
#pragma unroll
    for (int c = part * (D / 8); c < (part + 1) * (D / 8); ++c) {
      const float a = fmaxf(fabsf(Ds[row * PM_DS + D + c]), fabsf(Ds[row * PM_DS + 2 * D + c]));
      nb = fmaf(a, a, nb);
    }
    nb += __shfl_xor(nb, 4);
    nb += __shfl_xor(nb, 2);
    nb += __shfl_xor(nb, 1);
    if (part == 0 && j < g.nt) kbound[((int64_t)b * g.H + h) * g.nt + j] = j < nth ? sqrtf(nb) : 0.f;
  }

  // ---- layer 1: hidden units 64 w .. 64 w + 63; column m of the two accumulator blocks is
  // hidden unit 64 w + 2 m (acc0) and 64 w + 2 m + 1 (acc1), so that each lane takes both of
  // its weights of a step with one 8-byte load
  {
    const int m = lane & 31, kh = lane >> 5;
    const float *W1 = (which ? w1k : w1q) + (int64_t)h * D3 * MLP_HIDDEN + 64 * w + 2 * m;
    f32x16_t acc0, acc1;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      acc0[r] = 0.f;
      acc1[r] = 0.f;
    }
    float2 wr[PF];
#pragma unroll
    for (int pp = 0; pp < PF; ++pp) wr[pp] = *reinterpret_cast<const float2 *>(W1 + (2 * pp + kh) * MLP_HIDDEN);
#pragma unroll 1
    for (int sb = 0; sb < D3 / 2; sb += PF) {
#pragma unroll
      for (int pp = 0; pp < PF; ++pp) {
        const int kk = 2 * (sb + pp) + kh;
        const float2 bw = wr[pp];
        // unconditional prefetch (row clamped in range): no branch, so the waits stay exact
        const int kn = min(kk + 2 * PF, D3 - 2 + kh);
        const float av = Ds[m * PM_DS + kk];
        acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bw.x, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bw.y, acc1, 0, 0, 0);
        wr[pp] = *reinterpret_cast<const float2 *>(W1 + kn * MLP_HIDDEN);
        __builtin_amdgcn_sched_barrier(0);  // keep each step's prefetch a full ring ahead of its use
      }
    }
    __syncthreads();  // descriptors consumed: the block now holds the hidden layer
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 8 * (r >> 2) + 4 * kh + (r & 3);
      *reinterpret_cast<float2 *>(&Ds[row * PM_HST + 64 * w + 2 * m]) = make_float2(gelu_erf(acc0[r]), gelu_erf(acc1[r]));
    }
    if (zout != nullptr) {  // the pre-activation layer, for the estimator's backward pass
      float *zo = zout + ((((int64_t)which * g.B + b) * g.H + h) * g.nt + r0) * MLP_HIDDEN + 64 * w + 2 * m;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 8 * (r >> 2) + 4 * kh + (r & 3);
        if (r0 + row < g.nt) *reinterpret_cast<float2 *>(&zo[(int64_t)row * MLP_HIDDEN]) = make_float2(acc0[r], acc1[r]);
      }
    }
  }
  __syncthreads();

  // ---- layer 2: outputs 16 w .. 16 w + 15, rows in two 16-row blocks, all 256 hidden units;
  // A[m = lane%16][k = lane/16], B[k = lane/16][n = lane%16], D[m = 4*(lane/16) + r][n].
  {
    const int m = lane & 15, kq = lane >> 4;
    const float *W2 = (which ? w2k : w2q) + (int64_t)h * MLP_HIDDEN * MLP_OUT + 16 * w + m;
    f32x4_t a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
    float wr[PF];
#pragma unroll
    for (int pp = 0; pp < PF; ++pp) wr[pp] = W2[(4 * pp + kq) * MLP_OUT];
#pragma unroll 1
    for (int sb = 0; sb < MLP_HIDDEN / 4; sb += PF) {
#pragma unroll
      for (int pp = 0; pp < PF; ++pp) {
        const int kk = 4 * (sb + pp) + kq;
        const float bv = wr[pp];
        a0 = __builtin_amdgcn_mfma_f32_16x16x4f32(Ds[m * PM_HST + kk], bv, a0, 0, 0, 0);
        a1 = __builtin_amdgcn_mfma_f32_16x16x4f32(Ds[(16 + m) * PM_HST + kk], bv, a1, 0, 0, 0);
        wr[pp] = W2[min(kk + 4 * PF, MLP_HIDDEN - 4 + kq) * MLP_OUT];
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    float *yo = y + (((int64_t)which * g.B + b) * g.H + h) * (int64_t)g.nt * MLP_OUT + 16 * w + m;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row0 = r0 + 4 * kq + r, row1 = row0 + 16;
      if (row0 < g.nt) yo[(int64_t)row0 * MLP_OUT] = a0[r];
      if (row1 < g.nt) yo[(int64_t)row1 * MLP_OUT] = a1[r];
    }
  }
}

// ---------------------------------------------------------------------------------------
// Scores for 16 query-tile rows: S = scale * y_q y_k^T on 16x16x4 fp32 MFMA (A[m = lane%16]
// [k = lane/16], B[k = lane/16][n = lane%16], D[m = 4*(lane/16) + r][n = lane%16]); two
// accumulation chains (even / odd k steps) summed at the end.  Then one wave per row: NW
// waves take 16 / NW rows each.  Long rows (large MAXM) make the row block big enough that
// only one workgroup fits a CU, so they use 16 waves, one row each, to keep every SIMD busy
// through the latency-bound top-k.
template <int MAXM, int NW, int NC>
__global__ void __launch_bounds__(64 * NW) score_topk_kernel(const float *__restrict__ y, Geo g, float scale,
                                                             float *__restrict__ scores, float *__restrict__ probs,
                                                             int topk, int32_t *__restrict__ idx, HeadShapes hs) {
  constexpr int SW = 64 * MAXM + 1;
  __shared__ float S[16 * SW];
  const int nt = g.nt, nrb = (nt + 15) >> 4;
  const int L = xcd_tile(blockIdx.x, gridDim.x);  // each XCD walks contiguous heads
  const int i0 = (L % nrb) * 16, h = (L / nrb) % g.H, b = L / (nrb * g.H);
  const int t = threadIdx.x, lane = t & 63, w = __builtin_amdgcn_readfirstlane(t >> 6);
  // rows and columns of this head (fewer than nt for a head of a padded tiling with fewer tiles)
  const int nth = g.padded ? head_tiles(hs.s[h][0], hs.s[h][1], hs.s[h][2], g.T, g.Hs, g.Ws) : nt;
  const float *yq = y + (((int64_t)b * g.H + h) * nt) * MLP_OUT;
  const float *yk = y + ((((int64_t)g.B + b) * g.H + h) * nt) * MLP_OUT;
  // The contraction slot kq of step s carries channel 16 kq + s, so each lane's 16 operand
  // values are one contiguous 64-byte run (four 16-byte loads).
  const int m = lane & 15, kq = lane >> 4;
  float4 qa[4];
  {
    const float4 *qr = reinterpret_cast<const float4 *>(yq + (int64_t)min(i0 + m, nt - 1) * MLP_OUT + 16 * kq);
#pragma unroll
    for (int e = 0; e < 4; ++e) qa[e] = qr[e];
  }
  const int nblk = (nt + 15) >> 4;
  // Key blocks w, w + NW, w + 2 NW, ... of this wave, loaded SD blocks ahead (a ring of SD
  // register buffers indexed by constants: the loop is unrolled SD times).
  constexpr int SD = 3;
  float4 kv[SD][4];
#pragma unroll
  for (int u = 0; u < SD; ++u) {
    const int kb = w + NW * u;
    const float4 *kr = reinterpret_cast<const float4 *>(yk + (int64_t)min(16 * kb + m, nt - 1) * MLP_OUT + 16 * kq);
#pragma unroll
    for (int e = 0; e < 4; ++e) kv[u][e] = kr[e];   // clamped rows: always in bounds
  }
#pragma unroll 1
  for (int kb0 = w; kb0 < nblk; kb0 += NW * SD) {
#pragma unroll
    for (int u = 0; u < SD; ++u) {
      const int kb = kb0 + NW * u;
      if (kb < nblk) {  // wave-uniform
        f32x4_t a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a0 = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[e].x, kv[u][e].x, a0, 0, 0, 0);
          a1 = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[e].y, kv[u][e].y, a1, 0, 0, 0);
          a0 = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[e].z, kv[u][e].z, a0, 0, 0, 0);
          a1 = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[e].w, kv[u][e].w, a1, 0, 0, 0);
        }
        const int key = 16 * kb + m;
#pragma unroll
        for (int r = 0; r < 4; ++r) S[(4 * kq + r) * SW + key] = (a0[r] + a1[r]) * scale;
        const int kn = kb + NW * SD;
        if (kn < nblk) {
          const float4 *kr = reinterpret_cast<const float4 *>(yk + (int64_t)(16 * kn + m < nt ? 16 * kn + m : nt - 1) *
                                                                       MLP_OUT + 16 * kq);
#pragma unroll
          for (int e = 0; e < 4; ++e) kv[u][e] = kr[e];
        }
      }
    }
  }
  __syncthreads();
#pragma unroll 1
  for (int rr = 0; rr < 16 / NW; ++rr) {
    const int row = (16 / NW) * w + rr, i = i0 + row;
    if (i >= nth) break;  // wave-uniform
    const int64_t grow = ((int64_t)b * g.H + h) * nt + i;
    float sc[MAXM];
#pragma unroll
    for (int mm = 0; mm < MAXM; ++mm) sc[mm] = S[row * SW + min(64 * mm + lane, 64 * MAXM - 1)];
    if (scores != nullptr) {  // columns past the head's tiles: -inf
#pragma unroll
      for (int mm = 0; mm < MAXM; ++mm)
        if (64 * mm + lane < nt) scores[grow * nt + 64 * mm + lane] = 64 * mm + lane < nth ? sc[mm] : -INFINITY;
    }
    if (probs != nullptr) {
      float mx = -INFINITY;
#pragma unroll
      for (int mm = 0; mm < MAXM; ++mm)
        if (64 * mm + lane < nth) mx = fmaxf(mx, sc[mm]);
      mx = wave_max(mx);
      float e[MAXM], sum = 0.f;
#pragma unroll
      for (int mm = 0; mm < MAXM; ++mm) {
        e[mm] = (64 * mm + lane < nth) ? expf(sc[mm] - mx) : 0.f;
        sum += e[mm];
      }
      sum = wave_sum(sum);
      const float inv = 1.0f / sum;
#pragma unroll
      for (int mm = 0; mm < MAXM; ++mm)
        if (64 * mm + lane < nt) probs[grow * nt + 64 * mm + lane] = e[mm] * inv;
    }
    if (topk > 0) {
      uint32_t key[MAXM];
#pragma unroll
      for (int mm = 0; mm < MAXM; ++mm) key[mm] = (64 * mm + lane < nth) ? float_key(sc[mm]) : 0u;
      // the row is in registers now: its LDS words serve as the wave's top-k scratch
      wave_topk<MAXM, NC>(key, nth, topk, lane, idx + grow * topk, nullptr,
                                             reinterpret_cast<uint32_t *>(&S[row * SW]));
    }
  }
}

template <int MAXM>
__global__ void __launch_bounds__(256) topk_kernel(const float *__restrict__ scores, int64_t rows, int n_cols, int k,
                                                   int32_t *__restrict__ idx, uint8_t *__restrict__ mask) {
  __shared__ uint32_t tk_scratch[4][128];  // per wave
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;  // whole wave
  const float *src = scores + row * n_cols;
  uint32_t key[MAXM];
#pragma unroll
  for (int m = 0; m < MAXM; ++m) {
    const int j = 64 * m + lane;
    key[m] = (j < n_cols) ? float_key(src[j]) : 0u;
  }
  wave_topk<MAXM>(key, n_cols, k, lane, idx + row * k, mask ? mask + row * n_cols : nullptr, tk_scratch[threadIdx.x >> 6]);
}

// ---------------------------------------------------------------------------------------
template <int MAXM>
static void launch_score_t(const Geo &g, const float *y, float scale, float *scores, float *probs, int topk,
                           int32_t *idx, const HeadShapes &hs, hipStream_t st) {
  constexpr int NW = MAXM >= 16 ? 16 : (MAXM >= 10 ? 8 : 4);
  // Top-k compaction width (candidates kept in NC registers per lane once at most 64 NC
  // remain): wide enough that the search reaches the compacted phase soon, narrow enough
  // that each later bit costs few ballots.  The bounds on k come from counting the ballots
  // of the search on normally distributed rows; the selection does not depend on NC.
  const dim3 grid(((g.nt + 15) / 16) * g.H * g.B), block(64 * NW);
  if constexpr (MAXM >= 16) {
    if (topk > 160)
      score_topk_kernel<MAXM, NW, 8><<<grid, block, 0, st>>>(y, g, scale, scores, probs, topk, idx, hs);
    else
      score_topk_kernel<MAXM, NW, 4><<<grid, block, 0, st>>>(y, g, scale, scores, probs, topk, idx, hs);
  } else if constexpr (MAXM >= 10) {
    if (topk > 100)
      score_topk_kernel<MAXM, NW, 6><<<grid, block, 0, st>>>(y, g, scale, scores, probs, topk, idx, hs);
    else
      score_topk_kernel<MAXM, NW, 2><<<grid, block, 0, st>>>(y, g, scale, scores, probs, topk, idx, hs);
  } else {
    score_topk_kernel<MAXM, NW, 2><<<grid, block, 0, st>>>(y, g, scale, scores, probs, topk, idx, hs);
  }
}

template <int EB, bool RQ, bool RK>
static void launch_pool_mlp_t(const Geo &g, const HeadShapes &hs, const RasterView &rv, const void *q, const void *k,
                              const float *w1q, const float *w2q, const float *w1k, const float *w2k, float *y,
                              float *q_desc, float *k_desc, float *z, const int32_t *qlist, int nlist,
                              uint8_t *kout, const uint8_t *vsrc, uint8_t *vout, float *kbound, hipStream_t st) {
  if (!RQ) vout = nullptr;  // a V copy comes only with raster Q (its strides)
  const int nwh = vout != nullptr ? 3 : 2;
  const dim3 pg(((g.nt + PM_ROWS - 1) / PM_ROWS) * g.H * nwh * g.B);
  if (g.padded)
    pool_mlp_kernel<EB, RQ, RK, true><<<pg, 256, 0, st>>>((const uint8_t *)q, (const uint8_t *)k, w1q, w2q, w1k, w2k,
                                                          y, q_desc, k_desc, z, qlist, nlist, g, hs, rv, kout, vsrc,
                                                          vout, kbound);
  else
    pool_mlp_kernel<EB, RQ, RK, false><<<pg, 256, 0, st>>>((const uint8_t *)q, (const uint8_t *)k, w1q, w2q, w1k, w2k,
                                                           y, q_desc, k_desc, z, qlist, nlist, g, hs, rv, kout, vsrc,
                                                           vout, kbound);
}

hipError_t launch_pool_mlp(const Geo &g, veda_dtype dt, const void *q, const void *k, const float *w1q,
                           const float *w2q, const float *w1k, const float *w2k, float *y, float *q_desc,
                           float *k_desc, hipStream_t st, const HeadShapes *hs, const RasterView *rv,
                           bool k_raster, float *z, const int32_t *qlist, int nlist, void *k_tiled_out,
                           const void *v_raster, void *v_tiled_out, float *k_bound) {
  uint8_t *kout = static_cast<uint8_t *>(k_tiled_out);
  const uint8_t *vsrc = static_cast<const uint8_t *>(v_raster);
  uint8_t *vout = static_cast<uint8_t *>(v_tiled_out);
  const HeadShapes hs0 = hs != nullptr ? *hs : HeadShapes{};  // tiled operands: shapes matter only when padded
  const RasterView rv0{0, 0, 0};
  const bool bf = dt == VEDA_BF16;
  if (rv == nullptr) {
    if (bf)
      launch_pool_mlp_t<2, false, false>(g, hs0, rv0, q, k, w1q, w2q, w1k, w2k, y, q_desc, k_desc, z, qlist, nlist, kout, vsrc, vout, k_bound, st);
    else
      launch_pool_mlp_t<4, false, false>(g, hs0, rv0, q, k, w1q, w2q, w1k, w2k, y, q_desc, k_desc, z, qlist, nlist, kout, vsrc, vout, k_bound, st);
  } else if (k_raster) {
    if (bf)
      launch_pool_mlp_t<2, true, true>(g, *hs, *rv, q, k, w1q, w2q, w1k, w2k, y, q_desc, k_desc, z, qlist, nlist, kout, vsrc, vout, k_bound, st);
    else
      launch_pool_mlp_t<4, true, true>(g, *hs, *rv, q, k, w1q, w2q, w1k, w2k, y, q_desc, k_desc, z, qlist, nlist, kout, vsrc, vout, k_bound, st);
  } else {
    if (bf)
      launch_pool_mlp_t<2, true, false>(g, *hs, *rv, q, k, w1q, w2q, w1k, w2k, y, q_desc, k_desc, z, qlist, nlist, kout, vsrc, vout, k_bound, st);
    else
      launch_pool_mlp_t<4, true, false>(g, *hs, *rv, q, k, w1q, w2q, w1k, w2k, y, q_desc, k_desc, z, qlist, nlist, kout, vsrc, vout, k_bound, st);
  }
  return hipGetLastError();
}

hipError_t launch_score(const Geo &g, veda_dtype dt, const void *q, const void *k, const float *w1q,
                        const float *w2q, const float *w1k, const float *w2k, int hidden, int mlp_out, float scale,
                        float *scores, float *probs, float *q_desc, float *k_desc, int topk, int32_t *idx,
                        void *ws, hipStream_t st, const HeadShapes *hs, const RasterView *rv, bool k_raster,
                        void *k_tiled_out, const void *v_raster, void *v_tiled_out, float *k_bound) {
  (void)hidden;
  (void)mlp_out;
  float *y = (float *)ws;
  const HeadShapes hsv = hs != nullptr ? *hs : HeadShapes{};
  const hipError_t pe = launch_pool_mlp(g, dt, q, k, w1q, w2q, w1k, w2k, y, q_desc, k_desc, st, hs, rv, k_raster,
                                        nullptr, nullptr, 0, k_tiled_out, v_raster, v_tiled_out, k_bound);
  if (pe != hipSuccess) return pe;
  if (g.nt <= 64)
    launch_score_t<1>(g, y, scale, scores, probs, topk, idx, hsv, st);
  else if (g.nt <= 256)
    launch_score_t<4>(g, y, scale, scores, probs, topk, idx, hsv, st);
  else if (g.nt <= 640)
    launch_score_t<10>(g, y, scale, scores, probs, topk, idx, hsv, st);
  else if (g.nt <= 768)   // the row block in LDS grows with the bound: keep it tight
    launch_score_t<12>(g, y, scale, scores, probs, topk, idx, hsv, st);
  else if (g.nt <= 1024)
    launch_score_t<16>(g, y, scale, scores, probs, topk, idx, hsv, st);
  else if (g.nt <= 1280)
    launch_score_t<20>(g, y, scale, scores, probs, topk, idx, hsv, st);
  else
    launch_score_t<24>(g, y, scale, scores, probs, topk, idx, hsv, st);
  return hipGetLastError();
}

hipError_t launch_topk(int64_t rows, int n_cols, const float *scores, int k, int32_t *idx, uint8_t *mask,
                       hipStream_t st) {
  const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
  if (n_cols <= 64)
    topk_kernel<1><<<grid, block, 0, st>>>(scores, rows, n_cols, k, idx, mask);
  else if (n_cols <= 256)
    topk_kernel<4><<<grid, block, 0, st>>>(scores, rows, n_cols, k, idx, mask);
  else if (n_cols <= 640)
    topk_kernel<10><<<grid, block, 0, st>>>(scores, rows, n_cols, k, idx, mask);
  else if (n_cols <= 1280)
    topk_kernel<20><<<grid, block, 0, st>>>(scores, rows, n_cols, k, idx, mask);
  else if (n_cols <= 2048)
    topk_kernel<32><<<grid, block, 0, st>>>(scores, rows, n_cols, k, idx, mask);
  else
    topk_kernel<64><<<grid, block, 0, st>>>(scores, rows, n_cols, k, idx, mask);
  return hipGetLastError();
}

}  // namespace veda
