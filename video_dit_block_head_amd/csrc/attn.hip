// Tile-skipping attention forward.  [Technical Summary: Veda, §2.3 Hardware-Efficient
// Implementation: only the selected, non-contiguous key/value tiles are fetched]
//
// bf16 path (d = 128, P = 128), gfx950 MFMA v_mfma_f32_32x32x16_bf16:
//  - one workgroup (4 waves) per query tile, two workgroups per CU; wave w owns queries
//    32w .. 32w+31;
//  - the kept K tile ([key][d]) and V tile are copied straight into LDS (global_load_lds,
//    no register staging) with an XOR swizzle of the 16-byte chunks of each row, which
//    makes every MFMA operand read conflict-free; the reads are issued four MFMAs ahead of
//    their use (scheduling groups: the default schedule read one ahead).  K and V have
//    their own buffers: the next K tile streams in during softmax + P V, the next V tile
//    during the next Q K^T.  Three barriers per key tile: K(t) read (K buffer free), V(t)
//    complete, and V(t) read with K(t+1) complete;
//  - V comes in one of three layouts.  Channel-major tiles ([d][key], keys in the order in
//    which the probabilities reach the MFMA) make each V operand one 16-byte row read.
//    Tile-major rows ([key][d], like K) and the raster tensor itself are read with
//    ds_read_b64_tr_b16: two transposed 8-byte reads per operand, each giving a lane one
//    channel of four consecutive keys; their rows use the quad swizzle, which keeps these
//    reads conflict-free too (K then uses it as well, so both copies share offsets);
//  - S^T = K Q^T (32 keys x 32 queries per MFMA block) puts one query per lane column, so
//    the row max needs one exchange between lane halves; O^T = V^T P^T keeps each lane's
//    accumulators on its own query, so the online-softmax rescale is lane-local;
//  - softmax in fp32 in the log2 domain (scale * log2 e folded into one FMA); P rounded to
//    bf16 (nearest even) for P V; 1/l applied in fp32 at the end.  The exponent offset m
//    in p = exp2(s c - m) starts at the first kept tile's row max.  Running offset: it
//    only moves when a later tile's row max exceeds it by more than 2^8 (the rescale of O
//    is then rare; p <= 256 stays exact in fp32 and bf16 range).  Fixed offset, when
//    per-key-tile norm bounds are given: b = c |q| max over the kept tiles of the bound is
//    at or above every logit of the row (Cauchy-Schwarz); if b - m <= 64 for every row of
//    the wave, no later p can exceed 2^64 (far inside fp32 and bf16 range, and so are l
//    and O), so m stays where it is and no later tile needs a row max.  That gives the
//    running offset's result bit for bit unless a later row max exceeds m by more than
//    2^8 (where the running offset rescales instead);
//  - workgroups are mapped so that each XCD walks consecutive query tiles of one head,
//    sharing that head's K/V tiles in its L2.
//
// MFMA 32x32x16 operand layout (lane l, 0..63): A[m = l%32][k = 8*(l/32) + 0..7],
// B[k = 8*(l/32) + 0..7][n = l%32], D[m = 8*(r/4) + 4*(l/32) + r%4][n = l%32], r = 0..15.
#include "common.h"
#include "kernels.h"

namespace veda {

static constexpr float LOG2E = 1.4426950408889634f;
static constexpr float LN2 = 0.6931471805599453f;
static constexpr float RESCALE_SLACK = 8.0f;  // log2 units
static constexpr float BOUND_SLACK = 64.0f;   // log2 units: fixed offset while every later p <= 2^64

__device__ __forceinline__ f32x16_t mfma32(const bf16x8_t &a, const bf16x8_t &b, const f32x16_t &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Combine lanes l and l ^ 32 with v_permlane32_swap (a VALU op, no LDS round trip): with both
// operands = v, the two results hold v[l % 32] and v[32 + l % 32] in every lane.
__device__ __forceinline__ float half_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// V layouts of the attention kernels: channel-major tiles, tile-major rows, raster.
enum { VM_COLS = 0, VM_ROWS = 1, VM_RAST = 2 };

// RQ: Q and O are raster [B, N, H, d] tensors (byte strides in rv and ro) read and written
// through the head's tiling (token of row r of tile j = origin(j) + intra(r)), and LSE is in
// raster order; RK: the same for K (strides rv).  Otherwise tile-major.  VM: V's layout (VM_RAST with the
// strides of Q).  PAD: padded tiling: per-head tile counts and partial key tiles (K and V
// tiled); with RQ the padding query rows of a partial query tile are neither read (Q taken
// as zero, as the gather stores it) nor written.
// kbound: [B, H, nt] upper bounds of the key-row norms of each key tile, or null (running
// offset throughout).
template <bool RQ, bool RK, bool PAD, int VM>
__global__ void __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2, 2)))
attn_bf16_kernel(const __bf16 *__restrict__ q, const __bf16 *__restrict__ k, const __bf16 *__restrict__ vt,
                 const int32_t *__restrict__ kv_idx, const float *__restrict__ kbound, int kk, float c2,
                 __bf16 *__restrict__ o, float *__restrict__ lse, Geo g, HeadShapes hs, RasterView rv, RasterView ro) {
  constexpr bool VROW = VM != VM_COLS;          // V read with transposed reads
  constexpr int SW = VROW ? SWZ_QUAD : SWZ_ROW;  // swizzle of both LDS tiles
  const int L = xcd_tile(blockIdx.x, gridDim.x);
  const int i = L % g.nt;
  const int64_t bh = L / g.nt;
  const int hh = (int)(bh % g.H), bb = (int)(bh / g.H);
  const int t = threadIdx.x, lane = t & 63, lr = lane & 31, hi = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);  // wave index (uniform)
  const int64_t head = bh * (int64_t)g.N * 128;
  const int pt = hs.s[hh][0], ph = hs.s[hh][1], pw = hs.s[hh][2];
  // raster: byte offset of (b, n = 0, h); a tile's rows are origin(j) + intra(r) tokens on
  const int64_t rhead = (int64_t)bb * rv.sb + (int64_t)hh * rv.sh;
  const char *kh = RK ? reinterpret_cast<const char *>(k) + rhead : reinterpret_cast<const char *>(k + head);
  const char *vh = VM == VM_RAST ? reinterpret_cast<const char *>(vt) + rhead : reinterpret_cast<const char *>(vt + head);
  const int32_t *list = kv_idx + (bh * g.nt + i) * kk;
  // this head's tiles (fewer than nt for a head of a padded tiling with fewer tiles)
  const int nth = PAD ? head_tiles(hs.s[hh][0], hs.s[hh][1], hs.s[hh][2], g.T, g.Hs, g.Ws) : g.nt;
  if (i >= nth) return;  // whole workgroup, before any barrier
  const int last = nth - 1;
  auto k_tile = [&](int j) -> const char * {
    return RK ? kh + tile_origin(j, pt, ph, pw, g.Hs, g.Ws) * rv.sn : kh + (int64_t)j * 32768;
  };
  auto v_tile = [&](int j) -> const char * {
    return VM == VM_RAST ? vh + tile_origin(j, pt, ph, pw, g.Hs, g.Ws) * rv.sn : vh + (int64_t)j * 32768;
  };

  __shared__ uint4 Ks[128 * 16];
  __shared__ uint4 Vs[128 * 16];

  // The kept list is read 64 entries at a time into one register (lane l holds entry 64c + l)
  // and each step takes its entry with a readlane: no scalar load waits inside the loop.
  int lchunk = list[min(lane, kk - 1)];
  // The bound on this row's logits for a fixed offset: |c| |q| max over the kept tiles of
  // kbound (list entries clamped as in the loop).  The first 64 kept tiles' bounds load
  // beside the Q fragments (one unconditional load, pinned with them by the empty asm below,
  // so that the wait for Q covers it); longer lists read the rest first.
  bool lazy = kbound == nullptr;  // uniform: running offset for the whole query tile
  float km = 0.f;
  if (!lazy)
    for (int c0 = 64; c0 < kk; c0 += 64)
      km = fmaxf(km, kbound[bh * g.nt + min(max(list[min(c0 + lane, kk - 1)], 0), last)]);
  const uint32_t *km0_src = lazy ? reinterpret_cast<const uint32_t *>(list)  // any valid word when unused
                                 : reinterpret_cast<const uint32_t *>(kbound + bh * g.nt + min(max(lchunk, 0), last));
  const uint32_t km0 = *km0_src;

  // Q fragments, consumed by an empty asm so that they have arrived before the first copy
  // is issued (otherwise the compiler sinks the loads and waits for them in the loop, or
  // after the copies, which it does not count).
  const int qrow = i * 128 + 32 * w + lr;
  // this lane's query row: tiled row qrow, or its raster token (a real token unless the row
  // is padding of a partial tile of a padded tiling)
  const int64_t qtok = RQ ? tile_origin(i, pt, ph, pw, g.Hs, g.Ws) + tile_intra(32 * w + lr, ph, pw, g.Hs, g.Ws) : 0;
  const bool qreal = !(RQ && PAD) || row_real(i, 32 * w + lr, pt, ph, pw, g.T, g.Hs, g.Ws);
  const __bf16 *qp = RQ ? reinterpret_cast<const __bf16 *>(reinterpret_cast<const char *>(q) + rhead + qtok * rv.sn)
                        : q + head + (int64_t)qrow * 128;
  bf16x8_t qf[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    if (qreal) {
      qf[s] = *reinterpret_cast<const bf16x8_t *>(qp + 16 * s + 8 * hi);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[s][e] = (__bf16)0.0f;
    }
  }
  asm volatile("" ::"v"(qf[0]), "v"(qf[1]), "v"(qf[2]), "v"(qf[3]), "v"(qf[4]), "v"(qf[5]), "v"(qf[6]), "v"(qf[7]),
               "v"(km0));

  // copy offsets of a tile-major tile and of a raster one (computed only if K or V is raster)
  uint32_t toff[8], roff[8];
  tile_dma_offsets<SW>(w, lane, toff);
  if (RK || VM == VM_RAST)
    tile_dma_offsets_raster<SW>(w, lane, ph, pw, g.Hs, g.Ws, rv.sn, roff);
  else
#pragma unroll
    for (int e = 0; e < 8; ++e) roff[e] = toff[e];
  const uint32_t(&koff)[8] = RK ? roff : toff;
  const uint32_t(&voff)[8] = VM == VM_RAST ? roff : toff;
  const uint32_t ks_lds = lds_addr(Ks), vs_lds = lds_addr(Vs);
  // Transposed V reads (VROW): for MFMA block (s, db) lane l needs channel 32 db + l % 32 of
  // keys 16 s + 4 hi + {0..3} (k-slots 0-3) and 16 s + 8 + 4 hi + {0..3} (slots 4-7), the
  // keys whose probabilities sit in those slots of pb[s].  Within each 16-lane group lane i
  // reads key row (first key) + i / 4, 8 bytes at channel 16 c' + 4 (i % 4), and the
  // instruction hands lane i channel 16 c' + i of the four rows.  Byte offset in the V tile
  // of read (p, db), before the key-block term (16 s + 8 p) * 256 that goes into the
  // instruction's offset: (4 hi + i/4) * 256 + 16 * (chunk ^ swz) + 8 (i & 1) with chunk =
  // 4 db + 2 ((l / 16) & 1) + (i % 4) / 2 and swz = g(i / 4) ^ (2 p + hi).
  uint32_t vrd[2][4];
  if (VROW) {
    const int i16 = lane & 15, rq = i16 >> 2;
    const int cb = 2 * ((lane >> 4) & 1) + ((i16 & 3) >> 1);
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int slot = (4 * db + cb) ^ row_swz<SWZ_QUAD>(8 * p + 4 * hi + rq);
        vrd[p][db] = vs_lds + (uint32_t)((4 * hi + rq) * 256 + 16 * slot + 8 * (i16 & 1));
      }
  }
  int jn = min(max(__builtin_amdgcn_readlane(lchunk, 0), 0), last);  // out-of-range entries are clamped
  tile_to_lds(k_tile(jn), ks_lds, w, koff);
  tile_to_lds(v_tile(jn), vs_lds, w, voff);
  float m_bound = 0.f;
  if (!lazy) {  // the lane pair of a query row holds 64 of its channels each
    float qn = 0.f;
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) qn = fmaf((float)qf[s][e], (float)qf[s][e], qn);
    qn = half_sum(qn);
    km = fmaxf(km, __uint_as_float(km0));
#pragma unroll
    for (int x = 32; x >= 1; x >>= 1) km = fmaxf(km, __shfl_xor(km, x));
    m_bound = fabsf(c2) * sqrtf(qn) * km;
  }
  wait_vmem<8>();
  barrier();  // K(0) is complete

  f32x16_t acc_o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_o[db][r] = 0.f;
  float m_run = -1e30f, l_run = 0.f;

  for (int tt = 0; tt < kk; ++tt) {
    const bool more = tt + 1 < kk;
    const int jc = jn;  // this step's key tile (jn moves on to the next one below)
    // ---- S^T = K Q^T on the K tile in LDS (its loads were issued before the V loads)
    f32x16_t acc_s[4];
    // A padding key of a partial tile (padded tilings only) starts at -inf: its K row is
    // zero, so the MFMAs leave it there and it gets no weight.  Entry (kb, r) of this lane
    // is key row 32 kb + 8 (r / 4) + 4 hi + r % 4 of the tile.
    const TileBox bx = PAD ? tile_box(jc, pt, ph, pw, g.T, g.Hs, g.Ws) : TileBox{128, 1, 1};
    if (box_rows(bx) < 128) {
      uint32_t wd[4];
      tile_row_words(bx, ph, pw, lane, wd);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_s[kb][r] = (wd[kb] >> (8 * (r >> 2) + (r & 3))) & 1u ? 0.f : -INFINITY;
    } else {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_s[kb][r] = 0.f;
    }
    // the four key blocks' accumulations in rotation, so that consecutive MFMAs are
    // independent; operand reads run four MFMAs ahead
#pragma unroll
    for (int f = 0; f < 32; ++f) {
      const int kb = f & 3, s = f >> 2, row = 32 * kb + lr;
      const bf16x8_t a = *reinterpret_cast<const bf16x8_t *>(&Ks[row * 16 + ((2 * s + hi) ^ row_swz<SW>(lr))]);
      acc_s[kb] = mfma32(a, qf[s], acc_s[kb]);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int f = 0; f < 28; ++f) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    wait_lds();
    barrier();  // every wave has its K operands: the buffer may be refilled
    if (more) {
      const int tn = tt + 1;
      int e;
      if ((tn & 63) == 0) {  // uniform, once per 64 steps (the load is waited for only here)
        lchunk = list[min(tn + lane, kk - 1)];
        e = __builtin_amdgcn_readlane(lchunk, 0);
      } else {
        e = __builtin_amdgcn_readlane(lchunk, tn & 63);
      }
      jn = min(max(e, 0), last);
      tile_to_lds(k_tile(jn), ks_lds, w, koff);
    }

    // ---- online softmax (log2 domain): the row max of the first tile (it sets the offset),
    // and of every later tile with the running offset
    if (tt == 0 || lazy) {  // uniform
      float mx = -1e30f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc_s[kb][r]);
      mx = half_max(mx) * c2;
      // tt == 0 with bounds: the offset stays fixed unless a row's bound lies more than 2^64
      // above its first tile's max (or that max above the bound: the bounds are not this K's)
      if (!lazy) lazy = __ballot(mx < m_bound - BOUND_SLACK || mx > m_bound + RESCALE_SLACK) != 0;
      if (__ballot(mx > m_run + RESCALE_SLACK)) {  // always at tt == 0 (m_run starts at -1e30)
        const float m_new = fmaxf(m_run, mx);
        const float alpha = fast_exp2(m_run - m_new);
        l_run *= alpha;
        m_run = m_new;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc_o[db][r] *= alpha;
      }
    }
    // P = exp2(s * c - m) rounded to bf16; l sums the rounded values, so that the weights
    // that multiply V are exactly the ones normalised (matters for near one-hot rows).
    bf16x8_t pb[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[s][e] = (__bf16)fast_exp2(fmaf(acc_s[s >> 1][8 * (s & 1) + e], c2, -m_run));
    }
    const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
    float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      ls[0] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[s], pb[s], 0, 1), ones, ls[0], false);
      ls[1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[s], pb[s], 2, 3), ones, ls[1], false);
      ls[2] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[s], pb[s], 4, 5), ones, ls[2], false);
      ls[3] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[s], pb[s], 6, 7), ones, ls[3], false);
    }
    l_run += (ls[0] + ls[1]) + (ls[2] + ls[3]);

    // ---- O^T += V^T P^T on the V tile in LDS
    if (more)
      wait_vmem<8>();
    else
      wait_vmem<0>();
    barrier();
#pragma unroll
    for (int s = 0; s < 8; ++s) {
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        bf16x8_t a;
        if (VROW) {
          typedef __attribute__((address_space(3))) bf16x4_t lds_v4;
          const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4 *)(uintptr_t)(vrd[0][db] + 4096 * s));
          const bf16x4_t up = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4 *)(uintptr_t)(vrd[1][db] + 4096 * s + 2048));
          a = __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7);
        } else {
          const int drow = 32 * db + lr;
          a = *reinterpret_cast<const bf16x8_t *>(&Vs[drow * 16 + ((2 * s + hi) ^ (drow & 15))]);
        }
        acc_o[db] = mfma32(a, pb[s], acc_o[db]);
      }
    }
    constexpr int NRD = VROW ? 2 : 1;  // LDS reads per MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 4 * NRD, 0);  // operand reads four MFMAs ahead
#pragma unroll
    for (int f = 0; f < 28; ++f) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, NRD, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    wait_lds();
    wait_vmem<0>();  // this wave's part of K(t+1) has landed
    barrier();       // every wave is done with V(t), and K(t+1) is complete
    if (more) tile_to_lds(v_tile(jn), vs_lds, w, voff);
  }

  const float l_tot = half_sum(l_run);
  const float inv = 1.0f / l_tot;
  __bf16 *orow = RQ ? reinterpret_cast<__bf16 *>(reinterpret_cast<char *>(o) + (int64_t)bb * ro.sb +
                                                   (int64_t)hh * ro.sh + qtok * ro.sn)
                    : o + head + (int64_t)qrow * 128;
  if (qreal) {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = 32 * db + 8 * r4 + 4 * hi;
        bf16x4_t v;
        v[0] = (__bf16)(acc_o[db][4 * r4 + 0] * inv);
        v[1] = (__bf16)(acc_o[db][4 * r4 + 1] * inv);
        v[2] = (__bf16)(acc_o[db][4 * r4 + 2] * inv);
        v[3] = (__bf16)(acc_o[db][4 * r4 + 3] * inv);
        *reinterpret_cast<bf16x4_t *>(orow + d0) = v;
      }
  }
  // LSE: [B, H, tiled rows], or [B, H, real tokens] in raster order
  const int64_t lse_stride = RQ ? (int64_t)g.T * g.Hs * g.Ws : (int64_t)g.N;
  if (lse != nullptr && hi == 0 && qreal)
    lse[bh * lse_stride + (RQ ? qtok : (int64_t)qrow)] = (m_run + log2f(l_tot)) * LN2;
}

// fp32 path (d = 64, P = 64): one thread per query row, keys one at a time from LDS.
template <bool RQ, bool RK, int VM>
__global__ void __launch_bounds__(64) attn_f32_kernel(const float *__restrict__ q, const float *__restrict__ k,
                                                      const float *__restrict__ vt, const int32_t *__restrict__ kv_idx,
                                                      int kk, float scale, float *__restrict__ o,
                                                      float *__restrict__ lse, Geo g, HeadShapes hs, RasterView rv,
                                                      RasterView ro) {
  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z, t = threadIdx.x;
  const int64_t head = ((int64_t)b * g.H + h) * (int64_t)g.N * 64;
  const int32_t *list = kv_idx + (((int64_t)b * g.H + h) * g.nt + i) * kk;
  const int pt = hs.s[h][0], ph = hs.s[h][1], pw = hs.s[h][2];
  // element index of (tiled row, channel) of Q or K (raster if RQ / RK, strides rv), or of
  // O (raster if RQ, strides ro)
  auto at_v = [&](bool raster, const RasterView &r, int row, int c) -> int64_t {
    if (!raster) return head + (int64_t)row * 64 + c;
    const int64_t tok = tile_origin(row / 64, pt, ph, pw, g.Hs, g.Ws) + tile_intra(row % 64, ph, pw, g.Hs, g.Ws);
    return ((int64_t)b * r.sb + (int64_t)h * r.sh + tok * r.sn) / 4 + c;
  };
  auto at = [&](bool raster, int row, int c) -> int64_t { return at_v(raster, rv, row, c); };
  const int qrow = i * 64 + t;
  float qr[64], acc[64];
#pragma unroll
  for (int c = 0; c < 64; ++c) {
    qr[c] = q[at(RQ, qrow, c)];
    acc[c] = 0.f;
  }
  __shared__ float Ks[64][65];
  __shared__ float Vs[64][65];
  float m = -1e30f, l = 0.f;
  for (int tt = 0; tt < kk; ++tt) {
    const int j = min(max(list[tt], 0), g.nt - 1);
    __syncthreads();
    for (int e = t; e < 64 * 64; e += 64) {
      const int r = e >> 6, c = e & 63;
      Ks[r][c] = k[at(RK, j * 64 + r, c)];  // row r = key, c = channel
      if (VM == VM_COLS)
        Vs[cols_key(c)][r] = vt[head + ((int64_t)j * 64 + r) * 64 + c];  // channel-major: r = channel, c = position
      else
        Vs[r][c] = vt[at(VM == VM_RAST, j * 64 + r, c)];
    }
    __syncthreads();
    for (int x = 0; x < 64; ++x) {
      float s = 0.f;
#pragma unroll
      for (int c = 0; c < 64; ++c) s = fmaf(qr[c], Ks[x][c], s);
      s *= scale;
      const float m_new = fmaxf(m, s);
      const float a = expf(m - m_new), p = expf(s - m_new);
      l = l * a + p;
#pragma unroll
      for (int c = 0; c < 64; ++c) acc[c] = fmaf(p, Vs[x][c], acc[c] * a);
      m = m_new;
    }
  }
  const float inv = 1.0f / l;
#pragma unroll
  for (int c = 0; c < 64; ++c) o[at_v(RQ, ro, qrow, c)] = acc[c] * inv;
  if (lse != nullptr) {
    const int64_t pos = RQ ? tile_origin(i, pt, ph, pw, g.Hs, g.Ws) + tile_intra(t, ph, pw, g.Hs, g.Ws) : qrow;
    lse[((int64_t)b * g.H + h) * g.N + pos] = m + logf(l);
  }
}

template <bool RQ, bool RK, int VM>
static void launch_attn_t(const Geo &g, const HeadShapes &hs, const RasterView &rv, const RasterView &ro, veda_dtype dt,
                          const void *q, const void *k, const void *v, const int32_t *kv_idx, const float *kbound,
                          int kk, float scale, void *o, float *lse, hipStream_t st) {
  if (dt == VEDA_BF16) {
    constexpr bool PADDABLE = !RK && VM != VM_RAST;  // padded tilings read K and V tiled (the C ABI checks)
    if (PADDABLE && g.padded)
      attn_bf16_kernel<RQ, false, PADDABLE, VM><<<dim3(g.nt * g.H * g.B), 256, 0, st>>>(
          (const __bf16 *)q, (const __bf16 *)k, (const __bf16 *)v, kv_idx, kbound, kk, scale * LOG2E, (__bf16 *)o, lse,
          g, hs, rv, ro);
    else
      attn_bf16_kernel<RQ, RK, false, VM><<<dim3(g.nt * g.H * g.B), 256, 0, st>>>(
          (const __bf16 *)q, (const __bf16 *)k, (const __bf16 *)v, kv_idx, kbound, kk, scale * LOG2E, (__bf16 *)o, lse,
          g, hs, rv, ro);
  } else
    attn_f32_kernel<RQ, RK, VM><<<dim3(g.nt, g.H, g.B), 64, 0, st>>>((const float *)q, (const float *)k,
                                                                     (const float *)v, kv_idx, kk, scale, (float *)o,
                                                                     lse, g, hs, rv, ro);
}

template <bool RQ, bool RK>
static void launch_attn_v(int vm, const Geo &g, const HeadShapes &hs, const RasterView &rv, const RasterView &ro,
                          veda_dtype dt, const void *q, const void *k, const void *v, const int32_t *kv_idx,
                          const float *kbound, int kk, float scale, void *o, float *lse, hipStream_t st) {
  if (vm == VM_COLS)
    launch_attn_t<RQ, RK, VM_COLS>(g, hs, rv, ro, dt, q, k, v, kv_idx, kbound, kk, scale, o, lse, st);
  else if (vm == VM_ROWS)
    launch_attn_t<RQ, RK, VM_ROWS>(g, hs, rv, ro, dt, q, k, v, kv_idx, kbound, kk, scale, o, lse, st);
  else if constexpr (RQ)  // a raster V comes only with raster Q (its strides)
    launch_attn_t<RQ, RK, VM_RAST>(g, hs, rv, ro, dt, q, k, v, kv_idx, kbound, kk, scale, o, lse, st);
}

static int v_mode(veda_layout v_layout) {
  return v_layout == VEDA_TILE_COLS ? VM_COLS : v_layout == VEDA_RASTER ? VM_RAST : VM_ROWS;
}

hipError_t launch_sparse_attn(const Geo &g, const HeadShapes &hs, veda_dtype dt, const void *q, const void *k,
                              const void *v, veda_layout v_layout, const int32_t *kv_idx, const float *kbound, int kk,
                              float scale, void *o, float *lse, hipStream_t st) {
  launch_attn_v<false, false>(v_mode(v_layout), g, hs, RasterView{0, 0, 0}, RasterView{0, 0, 0}, dt, q, k, v, kv_idx,
                              kbound, kk, scale, o, lse, st);
  return hipGetLastError();
}

hipError_t launch_sparse_attn_raster(const Geo &g, const HeadShapes &hs, veda_dtype dt, const void *q, const void *k,
                                     bool k_raster, int64_t rs_b, int64_t rs_n, int64_t rs_h, const void *v,
                                     veda_layout v_layout, const int32_t *kv_idx, const float *kbound, int kk,
                                     float scale, void *o, int64_t os_b, int64_t os_n, int64_t os_h, float *lse,
                                     hipStream_t st) {
  const int64_t eb = dt == VEDA_BF16 ? 2 : 4;
  const RasterView rv{rs_b * eb, rs_n * eb, rs_h * eb}, ro{os_b * eb, os_n * eb, os_h * eb};
  if (k_raster)
    launch_attn_v<true, true>(v_mode(v_layout), g, hs, rv, ro, dt, q, k, v, kv_idx, kbound, kk, scale, o, lse, st);
  else
    launch_attn_v<true, false>(v_mode(v_layout), g, hs, rv, ro, dt, q, k, v, kv_idx, kbound, kk, scale, o, lse, st);
  return hipGetLastError();
}

}  // namespace veda
