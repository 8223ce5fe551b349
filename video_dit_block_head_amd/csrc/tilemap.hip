// Oracle tile map: max-pooling of the full-attention probabilities over each
// (query tile x key tile) region.  [Technical Summary: Veda, §2.1 "Target Construction";
// §2.3: ground-truth heatmaps in two passes, on subsets of query tiles]
//
// One workgroup per selected query tile, two passes over all N keys inside one launch:
//  pass 1: per query row, running max and sum of exp2 -> log2-domain LSE;
//  pass 2: S^T recomputed bit-identically; per key tile the row max of s*c - lse, then the
//          max over the tile's 128 queries (kept per wave in LDS, combined at the end);
//          M = exp2 of that.
// bf16 path uses the same MFMA S^T = K Q^T blocking as the attention kernel.
#include "common.h"
#include "kernels.h"

namespace veda {

static constexpr float TM_LOG2E = 1.4426950408889634f;
static constexpr float TM_LN2 = 0.6931471805599453f;
static constexpr int TM_MAX_NT = 1280;

__device__ __forceinline__ void stage_k(const uint4 *__restrict__ ksrc, uint4 *Ks, int t) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int ci = t + 256 * e;
    const int r = ci >> 4, c = ci & 15;
    Ks[r * 16 + (c ^ (r & 15))] = ksrc[ci];
  }
}

// Row max (over this lane's 64 keys and its partner lane's) of S^T for the wave's queries.
__device__ __forceinline__ void tile_scores_t(const uint4 *Ks, const bf16x8_t (&qf)[8], int lr, int hi,
                                              f32x16_t (&acc)[4]) {
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[kb][r] = 0.f;
    const int row = 32 * kb + lr;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int c = 2 * s + hi;
      const bf16x8_t a = *reinterpret_cast<const bf16x8_t *>(&Ks[row * 16 + (c ^ (row & 15))]);
      acc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], acc[kb], 0, 0, 0);
    }
  }
}

__global__ void __launch_bounds__(256) tilemap_bf16_kernel(const __bf16 *__restrict__ q, const __bf16 *__restrict__ k,
                                                           float c2, const int32_t *__restrict__ q_tiles, int n_sel,
                                                           float *__restrict__ out, float *__restrict__ lse_out,
                                                           Geo g) {
  const int a = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, lr = lane & 31, hi = lane >> 5;
  const int64_t bh = (int64_t)b * g.H + h;
  const int i = q_tiles ? min(max(q_tiles[bh * n_sel + a], 0), g.nt - 1) : a;  // clamped
  const __bf16 *qh = q + bh * (int64_t)g.N * 128, *kh = k + bh * (int64_t)g.N * 128;

  __shared__ uint4 Ks[128 * 16];
  __shared__ float wmax[4][TM_MAX_NT];

  const int qrow = i * 128 + 32 * w + lr;
  bf16x8_t qf[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) qf[s] = *reinterpret_cast<const bf16x8_t *>(qh + (int64_t)qrow * 128 + 16 * s + 8 * hi);

  f32x16_t acc[4];
  float m_run = -1e30f, l_run = 0.f;
  for (int j = 0; j < g.nt; ++j) {  // pass 1
    __syncthreads();
    stage_k(reinterpret_cast<const uint4 *>(kh + (int64_t)j * 128 * 128), Ks, t);
    __syncthreads();
    tile_scores_t(Ks, qf, lr, hi, acc);
    float mx = -1e30f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc[kb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx * c2);
    float lsum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) lsum += exp2f(fmaf(acc[kb][r], c2, -m_new));
    l_run = fmaf(l_run, exp2f(m_run - m_new), lsum);
    m_run = m_new;
  }
  const float lse2 = m_run + log2f(l_run + __shfl_xor(l_run, 32));
  if (lse_out != nullptr && hi == 0) lse_out[bh * (int64_t)n_sel * 128 + (int64_t)a * 128 + 32 * w + lr] = lse2 * TM_LN2;

  for (int j = 0; j < g.nt; ++j) {  // pass 2
    __syncthreads();
    stage_k(reinterpret_cast<const uint4 *>(kh + (int64_t)j * 128 * 128), Ks, t);
    __syncthreads();
    tile_scores_t(Ks, qf, lr, hi, acc);
    float mx = -1e30f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc[kb][r]);
    float x = fmaf(mx, c2, -lse2);
    x = wave_max(x);
    if (lane == 0) wmax[w][j] = x;
  }
  __syncthreads();
  float *dst = out + (bh * n_sel + a) * (int64_t)g.nt;
  for (int j = t; j < g.nt; j += 256)
    dst[j] = exp2f(fmaxf(fmaxf(wmax[0][j], wmax[1][j]), fmaxf(wmax[2][j], wmax[3][j])));
}

// fp32 path (d = 64, P = 64): one thread per query row.
__global__ void __launch_bounds__(64) tilemap_f32_kernel(const float *__restrict__ q, const float *__restrict__ k,
                                                         float scale, const int32_t *__restrict__ q_tiles, int n_sel,
                                                         float *__restrict__ out, float *__restrict__ lse_out, Geo g) {
  const int a = blockIdx.x, h = blockIdx.y, b = blockIdx.z, t = threadIdx.x;
  const int64_t bh = (int64_t)b * g.H + h;
  const int i = q_tiles ? min(max(q_tiles[bh * n_sel + a], 0), g.nt - 1) : a;
  const float *qh = q + bh * (int64_t)g.N * 64, *kh = k + bh * (int64_t)g.N * 64;
  float qr[64];
#pragma unroll
  for (int c = 0; c < 64; ++c) qr[c] = qh[(int64_t)(i * 64 + t) * 64 + c];
  __shared__ float Ks[64][65];
  __shared__ float wm[TM_MAX_NT];
  float m = -1e30f, l = 0.f;
  for (int pass = 0; pass < 2; ++pass) {
    const float lse = m + logf(l);
    for (int j = 0; j < g.nt; ++j) {
      __syncthreads();
      for (int e = t; e < 64 * 64; e += 64) Ks[e >> 6][e & 63] = kh[((int64_t)j * 64 + (e >> 6)) * 64 + (e & 63)];
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

hipError_t launch_tilemap(const Geo &g, veda_dtype dt, const void *q, const void *k, float scale,
                          const int32_t *q_tiles, int n_sel, float *tilemap, float *lse, hipStream_t st) {
  const dim3 grid(n_sel, g.H, g.B);
  if (dt == VEDA_BF16)
    tilemap_bf16_kernel<<<grid, 256, 0, st>>>((const __bf16 *)q, (const __bf16 *)k, scale * TM_LOG2E, q_tiles, n_sel,
                                              tilemap, lse, g);
  else
    tilemap_f32_kernel<<<grid, 64, 0, st>>>((const float *)q, (const float *)k, scale, q_tiles, n_sel, tilemap, lse,
                                            g);
  return hipGetLastError();
}

}  // namespace veda
