// Shared device-side definitions of the gfx950 kernels (internal; not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "veda.h"

namespace veda {

// Number of compute units of the current device (cached per device; host side).
inline int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// Per-head tile shapes, passed to kernels by value (1.5 KB of kernel arguments).
struct HeadShapes {
  int32_t s[VEDA_MAX_HEADS][3];
};

// Geometry as the kernels see it.
// Shapes that do not divide the grid pad it up to whole tiles per head: N and nt are then the
// tiled per-head length and tile count of the head with the most tiles, and `padded` is 1.
struct Geo {
  int32_t B, H, d, T, Hs, Ws, P, N, nt;
  int32_t padded;
};

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Raster token index of row `o` of tile `j` for tile shape (pt, ph, pw): tiles row-major
// over the tile grid, tokens row-major inside the tile.
// The tile grid covers the grid padded up to whole tiles (ceil per axis); the token of a
// padding row lies outside the real grid (row_real is false) and is never accessed.
__device__ __forceinline__ int64_t tile_row_token(int j, int o, int pt, int ph, int pw, int Hs, int Ws) {
  const int ntw = (Ws + pw - 1) / pw, nth = (Hs + ph - 1) / ph;
  const int jw = j % ntw, jh = (j / ntw) % nth, jt = j / (ntw * nth);
  const int ow = o % pw, oh = (o / pw) % ph, ot = o / (pw * ph);
  return ((int64_t)(jt * pt + ot) * Hs + (jh * ph + oh)) * Ws + (jw * pw + ow);
}

// Tiles of a head on the grid padded up to whole tiles.
__host__ __device__ __forceinline__ int head_tiles(int pt, int ph, int pw, int T, int Hs, int Ws) {
  return ((T + pt - 1) / pt) * ((Hs + ph - 1) / ph) * ((Ws + pw - 1) / pw);
}

// Real extent of tile j along (t, h, w): the part of the tile inside the real grid (the
// whole shape unless the tile sticks out of a padded grid).  Uniform over a tile.
struct TileBox {
  int vt, vh, vw;
};
__device__ __forceinline__ TileBox tile_box(int j, int pt, int ph, int pw, int T, int Hs, int Ws) {
  const int ntw = (Ws + pw - 1) / pw, nth = (Hs + ph - 1) / ph;
  const int jw = j % ntw, jh = (j / ntw) % nth, jt = j / (ntw * nth);
  return TileBox{min(pt, T - jt * pt), min(ph, Hs - jh * ph), min(pw, Ws - jw * pw)};
}
__device__ __forceinline__ int box_rows(const TileBox &b) { return b.vt * b.vh * b.vw; }
// Whether row o of a tile with extent b is real; ph and pw are powers of two (their
// product with pt is the tile, 64 or 128 tokens), so the in-tile coordinates are shifts.
__device__ __forceinline__ bool in_box(int o, int ph, int pw, const TileBox &b) {
  const int lw = __builtin_ctz(pw), lh = __builtin_ctz(ph);
  return (o >> (lw + lh)) < b.vt && ((o >> lw) & (ph - 1)) < b.vh && (o & (pw - 1)) < b.vw;
}
__device__ __forceinline__ bool row_real(int j, int o, int pt, int ph, int pw, int T, int Hs, int Ws) {
  return in_box(o, ph, pw, tile_box(j, pt, ph, pw, T, Hs, Ws));
}

// Real rows of a 128-row tile as four 32-bit words (word kb: rows 32 kb .. 32 kb + 31),
// each shifted right by 4 * (lane / 32): bit 8 (r / 4) + r % 4 of word kb is then row
// 32 kb + 8 (r / 4) + 4 (lane / 32) + r % 4, the key of MFMA 32x32 output entry (kb, r).
// Built from the tile's box by two ballots, so nothing per lane outlives the tile.
__device__ __forceinline__ void tile_row_words(const TileBox &bx, int ph, int pw, int lane, uint32_t (&wd)[4]) {
  const uint64_t m0 = __ballot(in_box(lane, ph, pw, bx)), m1 = __ballot(in_box(64 + lane, ph, pw, bx));
  const int sh = 4 * (lane >> 5);
  wd[0] = (uint32_t)m0 >> sh;
  wd[1] = (uint32_t)(m0 >> 32) >> sh;
  wd[2] = (uint32_t)m1 >> sh;
  wd[3] = (uint32_t)(m1 >> 32) >> sh;
}

// The same token as origin(j) + intra(o): the first is uniform over a tile, the second is
// the same for row o of every tile of a head.  Tiles are numbered over the grid padded up
// to whole tiles; on a padded tiling origin + intra names a real token only for the rows
// inside the tile's box (in_box), and the others must not be read or written.
__device__ __forceinline__ int64_t tile_origin(int j, int pt, int ph, int pw, int Hs, int Ws) {
  const int ntw = (Ws + pw - 1) / pw, nth = (Hs + ph - 1) / ph;
  const int jw = j % ntw, jh = (j / ntw) % nth, jt = j / (ntw * nth);
  return ((int64_t)(jt * pt) * Hs + jh * ph) * Ws + jw * pw;
}
// ph and pw are powers of two (they divide the tile, 64 or 128 tokens).
__device__ __forceinline__ int tile_intra(int o, int ph, int pw, int Hs, int Ws) {
  const int lw = __builtin_ctz(pw), lh = __builtin_ctz(ph);
  return ((o >> (lw + lh)) * Hs + ((o >> lw) & (ph - 1))) * Ws + (o & (pw - 1));
}

// Raster [B, N, H, d] tensor seen by a kernel: byte strides of batch, token and head (the
// d elements of a token's head row are contiguous).
struct RasterView {
  int64_t sb, sn, sh;
};

// Channel-major tiles (VEDA_TILE_COLS) store, in each group of 16 consecutive positions,
// the tile's tokens (keys) 0-3, 8-11, 4-7, 12-15 of that group: key at position p.  This is
// the order in which the S^T accumulator of a 32x32 MFMA block reaches the k-slots of the
// next MFMA's B operand, so the matching V^T operand is one contiguous 16-byte read.
__host__ __device__ __forceinline__ int cols_key(int p) {
  const int q = p & 15;
  return (p & ~15) | (q < 4 || q >= 12 ? q : (q < 8 ? q + 4 : q - 4));
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t h16) { return __uint_as_float(h16 << 16); }

// Order-preserving map of a float to uint32 (larger float -> larger key); -0 maps like +0.
// 16-byte load marked non-temporal: read-once streams do not displace reused data in L2.
__device__ __forceinline__ uint4 load_stream16(const void *p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// 16-byte store marked non-temporal: a write-once copy does not displace reused data in L2.
__device__ __forceinline__ void store_stream16(void *p, const uint4 &v) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4 *>(p));
}

__device__ __forceinline__ uint32_t float_key(float x) {
  uint32_t u = __float_as_uint(x + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ uint64_t lanemask_lt(int lane) { return (lane == 0) ? 0ull : ((~0ull) >> (64 - lane)); }

// Top-k of one row held by a wave: lane `lane` holds columns j = 64*m + lane, m < MAXM,
// as order-preserving keys (0 for columns >= n_cols).  Writes the indices of the k largest
// keys, ties to the lower index, ascending, to idx[0..k); optional 0/1 mask[0..n_cols).
// The k-th largest key is found bit by bit (largest T with count(key >= T) >= k), starting
// below the bits that every valid key of the row shares, and stopping as soon as exactly k
// keys are >= the candidate (that set is then the answer, whatever lies below).  Every later
// candidate exceeds T, so only keys >= T can still be counted: once at most 64 NC of them
// are left they are compacted (through `scratch`, 64 NC words of the wave's own LDS) into NC
// registers per lane, and the remaining bits cost NC ballots instead of MAXM.
template <int MAXM, int NC = 2>
__device__ __forceinline__ void wave_topk(const uint32_t (&key)[MAXM], int n_cols, int k, int lane,
                                          int32_t *__restrict__ idx, uint8_t *__restrict__ mask,
                                          uint32_t *scratch) {
  static_assert(NC >= 1 && NC <= 8, "compaction registers");
  uint32_t kmax = 0u, kmin = 0xFFFFFFFFu;
#pragma unroll
  for (int m = 0; m < MAXM; ++m) {
    kmax = max(kmax, key[m]);
    if (64 * m + lane < n_cols) kmin = min(kmin, key[m]);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o));
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o));
  }
  kmax = __builtin_amdgcn_readfirstlane(kmax);
  kmin = __builtin_amdgcn_readfirstlane(kmin);
  const uint32_t diff = kmax ^ kmin;
  const uint64_t lt = lanemask_lt(lane);
  uint32_t T = kmax;  // every valid key equal: T is the k-th largest already
  if (diff != 0u) {
    const int b0 = 31 - __builtin_clz(diff);
    T = b0 == 31 ? 0u : (kmax & ~((2u << b0) - 1u));
    // keys >= T: all valid keys (they share T's bits), and the padding too when T = 0
    int alive = T != 0u ? n_cols : 64 * MAXM;
    bool done = false;
    int b = b0;
    for (; b >= 0 && (MAXM <= NC || alive > 64 * NC); --b) {
      const uint32_t cand = T | (1u << b);
      int cnt = 0;
#pragma unroll
      for (int m = 0; m < MAXM; ++m) cnt += __popcll(__ballot(key[m] >= cand));
      if (cnt >= k) {
        T = cand;
        alive = cnt;
      }
      if (cnt == k) {
        done = true;
        break;
      }
    }
    if (MAXM > NC && !done && b >= 0) {
      int base = 0;
#pragma unroll
      for (int m = 0; m < MAXM; ++m) {
        const bool a = key[m] >= T;
        const uint64_t am = __ballot(a);
        if (a) scratch[base + __popcll(am & lt)] = key[m];  // base + rank < alive <= 64 NC
        base += __popcll(am);
      }
      // padding 0 is never counted: every candidate is >= 1
      uint32_t c[NC];
#pragma unroll
      for (int j = 0; j < NC; ++j) c[j] = 64 * j + lane < base ? scratch[64 * j + lane] : 0u;
      for (; b >= 0; --b) {
        const uint32_t cand = T | (1u << b);
        int cnt = 0;
#pragma unroll
        for (int j = 0; j < NC; ++j) cnt += __popcll(__ballot(c[j] >= cand));
        if (cnt >= k) T = cand;
        if (cnt == k) break;
      }
    }
  }
  int n_gt = 0;
#pragma unroll
  for (int m = 0; m < MAXM; ++m) n_gt += __popcll(__ballot(key[m] > T));
  const int need = k - n_gt;
  int base = 0, ties = 0;
#pragma unroll
  for (int m = 0; m < MAXM; ++m) {
    const int j = 64 * m + lane;
    const bool gt = key[m] > T;
    const bool eq = key[m] == T;
    const uint64_t eqm = __ballot(eq);
    const int tie_rank = ties + __popcll(eqm & lt);
    const bool sel = gt || (eq && tie_rank < need);
    const uint64_t selm = __ballot(sel);
    if (sel) idx[base + __popcll(selm & lt)] = j;
    if (mask != nullptr && j < n_cols) mask[j] = sel ? 1 : 0;
    base += __popcll(selm);
    ties += __popcll(eqm);
  }
}

// LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// Direct-to-LDS copy of 16 bytes per lane: lane i's bytes at base + off land at LDS byte
// m0_addr + 16 * i.  Issued as inline asm so that the compiler does not treat the pending
// LDS write as aliasing every LDS read (it would wait for all copies before each read);
// completion is tracked by the explicit vmcnt waits below.  No output registers; M0 is
// set by the compiler through the "{m0}" operand.
__device__ __forceinline__ void dma16(const char *base, uint32_t off, uint32_t m0_addr) {
  // s_nop: one wait state between the SALU write of M0 and an LDS-DMA load that reads it.
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(off), "s"(base), "{m0}"(m0_addr) : "memory");
}

// Row swizzles of a 128 x 256-byte tile in LDS: 16-byte chunk c of row r sits at slot
// c ^ swz(r).
//  - SWZ_ROW, swz(r) = r & 15: sixteen consecutive rows read at one chunk (16-byte reads,
//    one row per lane) hit sixteen different slots.
//  - SWZ_QUAD, swz(r) = g(r & 3) ^ ((r >> 2) & 3) with g = {0, 10, 12, 6}: still a
//    permutation of the sixteen slots over any sixteen aligned rows, and in addition, within
//    every aligned quad of rows, bits 1-2 and bits 2-3 of swz take four different values.
//    Transposed 8-byte reads of four rows x 32 or 64 contiguous bytes then fall on
//    different banks (two or four chunks of each row side by side).
enum { SWZ_ROW = 0, SWZ_QUAD = 1 };
template <int SW>
__host__ __device__ __forceinline__ int row_swz(int r) {
  return SW == SWZ_ROW ? (r & 15) : (((0x6CA0 >> (4 * (r & 3))) & 15) ^ ((r >> 2) & 3));
}

// The calling wave copies rows [32w, 32w+32) of a 128 x 256-byte tile into LDS, 4 rows per
// instruction; LDS slot (r, s) receives global chunk (r, s ^ swz(r)).  off[e] is the lane's
// byte offset in the tile for instruction e.
__device__ __forceinline__ void tile_to_lds(const char *src, uint32_t lds_base, int w, const uint32_t (&off)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) dma16(src, off[e], lds_base + (uint32_t)((32 * w + 4 * e) * 256));
}

// Per-lane byte offsets of tile_to_lds for wave w: instruction e covers rows 32w+4e .. +3,
// lane -> (row 32w + 4e + lane/16, slot lane%16), source chunk slot ^ swz(row).
template <int SW = SWZ_ROW>
__device__ __forceinline__ void tile_dma_offsets(int w, int lane, uint32_t (&off)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int r = 32 * w + 4 * e + (lane >> 4);
    off[e] = (uint32_t)(r * 256 + (((lane & 15) ^ row_swz<SW>(r)) << 4));
  }
}

// The same copy from a raster tensor: row r of the tile is the token at intra(r) tokens
// from the tile's origin, so the per-lane offsets are those of tile_dma_offsets with the
// row's byte offset replaced by intra(row) * (token stride); the tile's origin goes into
// the scalar base address.  Offsets stay below 4 GiB for every supported grid.
template <int SW = SWZ_ROW>
__device__ __forceinline__ void tile_dma_offsets_raster(int w, int lane, int ph, int pw, int Hs, int Ws,
                                                        int64_t sn, uint32_t (&off)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int r = 32 * w + 4 * e + (lane >> 4);
    const int chunk = (lane & 15) ^ row_swz<SW>(r);
    off[e] = (uint32_t)((int64_t)tile_intra(r, ph, pw, Hs, Ws) * sn + chunk * 16);
  }
}

// Explicit waits for the copies above (the compiler does not know about them).
template <int N>
__device__ __forceinline__ void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void wait_lds() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void barrier() {
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// blockIdx.x -> logical tile: XCD x (= blockIdx.x % 8) takes a contiguous range.
__device__ __forceinline__ int xcd_tile(int bid, int nb) {
  const int per = nb >> 3;
  return bid < (per << 3) ? (bid & 7) * per + (bid >> 3) : bid;
}

}  // namespace veda
