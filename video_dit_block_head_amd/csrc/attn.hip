// Tile-skipping attention forward.  [Technical Summary: Veda, §2.3 Hardware-Efficient
// Implementation: only the selected, non-contiguous key/value tiles are fetched]
//
// bf16 path (d = 128, P = 128), gfx950 MFMA v_mfma_f32_32x32x16_bf16:
//  - one workgroup (4 waves) per query tile; wave w owns queries 32w .. 32w+31;
//  - the kept K tile ([key][d]) and V tile ([d][key], channel-major in HBM) are staged in
//    LDS with XOR swizzles that make the MFMA operand reads bank-conflict free;
//  - S^T = K Q^T (32 keys x 32 queries per MFMA block) puts one query per lane column, so
//    the row max / sum need one exchange between lane halves; O^T = V^T P^T keeps every
//    lane's accumulators on its own query, so the online-softmax rescale is lane-local;
//  - softmax in fp32 in the log2 domain (scale * log2 e folded into one multiply), P
//    rounded to bf16 (nearest-even) for the P V product, 1/l applied in fp32 at the end.
//
// MFMA 32x32x16 operand layout (lane l, 0..63): A[m = l%32][k = 8*(l/32) + 0..7],
// B[k = 8*(l/32) + 0..7][n = l%32], D[m = 8*(r/4) + 4*(l/32) + r%4][n = l%32], r = 0..15.
#include "common.h"
#include "kernels.h"

namespace veda {

static constexpr float LOG2E = 1.4426950408889634f;
static constexpr float LN2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16_t mfma32(const bf16x8_t &a, const bf16x8_t &b, const f32x16_t &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t pack_bf16x8(float x0, float x1, float x2, float x3, float x4, float x5, float x6,
                                                float x7) {
  bf16x8_t r;
  r[0] = (__bf16)x0;
  r[1] = (__bf16)x1;
  r[2] = (__bf16)x2;
  r[3] = (__bf16)x3;
  r[4] = (__bf16)x4;
  r[5] = (__bf16)x5;
  r[6] = (__bf16)x6;
  r[7] = (__bf16)x7;
  return r;
}

// Stage one 128x128 bf16 K tile (row-major) and V tile (channel-major) into LDS.
//  K: 16-byte chunk c of row r at chunk slot c ^ (r & 15).
//  V: 8-byte granule g of row r at granule slot g ^ (r & 31).
__device__ __forceinline__ void stage_kv(const uint4 *__restrict__ ksrc, const uint4 *__restrict__ vsrc, uint4 *Ks,
                                         uint4 *Vs, int t) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int ci = t + 256 * e;
    const int r = ci >> 4, c = ci & 15;
    const uint4 kv = ksrc[ci];
    uint4 vv = vsrc[ci];
    Ks[r * 16 + (c ^ (r & 15))] = kv;
    if (r & 1) vv = make_uint4(vv.z, vv.w, vv.x, vv.y);
    Vs[r * 16 + (c ^ ((r & 31) >> 1))] = vv;
  }
}

__global__ void __launch_bounds__(256) attn_bf16_kernel(const __bf16 *__restrict__ q, const __bf16 *__restrict__ k,
                                                        const __bf16 *__restrict__ vt,
                                                        const int32_t *__restrict__ kv_idx, int kk, float c2,
                                                        __bf16 *__restrict__ o, float *__restrict__ lse, Geo g) {
  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, lr = lane & 31, hi = lane >> 5;
  const int64_t head = ((int64_t)b * g.H + h) * (int64_t)g.N * 128;
  const __bf16 *qh = q + head, *kh = k + head, *vh = vt + head;
  const int32_t *list = kv_idx + (((int64_t)b * g.H + h) * g.nt + i) * kk;

  __shared__ uint4 Ks[128 * 16];
  __shared__ uint4 Vs[128 * 16];
  const char *Vb = reinterpret_cast<const char *>(Vs);

  const int qrow = i * 128 + 32 * w + lr;
  bf16x8_t qf[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) qf[s] = *reinterpret_cast<const bf16x8_t *>(qh + (int64_t)qrow * 128 + 16 * s + 8 * hi);

  f32x16_t acc_o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_o[db][r] = 0.f;
  float m_run = -1e30f, l_run = 0.f;

  for (int tt = 0; tt < kk; ++tt) {
    const int j = min(max(list[tt], 0), g.nt - 1);  // out-of-range entries are clamped
    __syncthreads();
    stage_kv(reinterpret_cast<const uint4 *>(kh + (int64_t)j * 128 * 128),
             reinterpret_cast<const uint4 *>(vh + (int64_t)j * 128 * 128), Ks, Vs, t);
    __syncthreads();

    f32x16_t acc_s[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) acc_s[kb][r] = 0.f;
      const int row = 32 * kb + lr;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int c = 2 * s + hi;
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t *>(&Ks[row * 16 + (c ^ (row & 15))]);
        acc_s[kb] = mfma32(a, qf[s], acc_s[kb]);
      }
    }

    float mx = -1e30f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc_s[kb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx * c2);
    const float alpha = exp2f(m_run - m_new);
    float lsum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2f(fmaf(acc_s[kb][r], c2, -m_new));
        acc_s[kb][r] = p;
        lsum += p;
      }
    l_run = fmaf(l_run, alpha, lsum);
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc_o[db][r] *= alpha;

#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const f32x16_t &ps = acc_s[s >> 1];
      const int r0 = 8 * (s & 1);
      const bf16x8_t pb = pack_bf16x8(ps[r0], ps[r0 + 1], ps[r0 + 2], ps[r0 + 3], ps[r0 + 4], ps[r0 + 5], ps[r0 + 6],
                                      ps[r0 + 7]);
      const int g0 = 4 * s + hi, g1 = 4 * s + 2 + hi;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int drow = 32 * db + lr;
        const bf16x4_t lo = *reinterpret_cast<const bf16x4_t *>(Vb + drow * 256 + ((g0 ^ (drow & 31)) << 3));
        const bf16x4_t hi4 = *reinterpret_cast<const bf16x4_t *>(Vb + drow * 256 + ((g1 ^ (drow & 31)) << 3));
        const bf16x8_t a = __builtin_shufflevector(lo, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
        acc_o[db] = mfma32(a, pb, acc_o[db]);
      }
    }
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.0f / l_tot;
  __bf16 *orow = o + head + (int64_t)qrow * 128;
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
  if (lse != nullptr && hi == 0) lse[((int64_t)b * g.H + h) * g.N + qrow] = (m_run + log2f(l_tot)) * LN2;
}

// fp32 path (d = 64, P = 64): one thread per query row, keys one at a time from LDS.
__global__ void __launch_bounds__(64) attn_f32_kernel(const float *__restrict__ q, const float *__restrict__ k,
                                                      const float *__restrict__ vt, const int32_t *__restrict__ kv_idx,
                                                      int kk, float scale, float *__restrict__ o,
                                                      float *__restrict__ lse, Geo g) {
  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z, t = threadIdx.x;
  const int64_t head = ((int64_t)b * g.H + h) * (int64_t)g.N * 64;
  const int32_t *list = kv_idx + (((int64_t)b * g.H + h) * g.nt + i) * kk;
  const int qrow = i * 64 + t;
  float qr[64], acc[64];
#pragma unroll
  for (int c = 0; c < 64; ++c) {
    qr[c] = q[head + (int64_t)qrow * 64 + c];
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
      Ks[r][c] = k[head + ((int64_t)j * 64 + r) * 64 + c];  // row r = key, c = channel
      Vs[c][r] = vt[head + ((int64_t)j * 64 + r) * 64 + c];  // channel-major: r = channel, c = key
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
  for (int c = 0; c < 64; ++c) o[head + (int64_t)qrow * 64 + c] = acc[c] * inv;
  if (lse != nullptr) lse[((int64_t)b * g.H + h) * g.N + qrow] = m + logf(l);
}

hipError_t launch_sparse_attn(const Geo &g, veda_dtype dt, const void *q, const void *k, const void *v,
                              const int32_t *kv_idx, int kk, float scale, void *o, float *lse, hipStream_t st) {
  const dim3 grid(g.nt, g.H, g.B);
  if (dt == VEDA_BF16)
    attn_bf16_kernel<<<grid, 256, 0, st>>>((const __bf16 *)q, (const __bf16 *)k, (const __bf16 *)v, kv_idx, kk,
                                           scale * LOG2E, (__bf16 *)o, lse, g);
  else
    attn_f32_kernel<<<grid, 64, 0, st>>>((const float *)q, (const float *)k, (const float *)v, kv_idx, kk, scale,
                                         (float *)o, lse, g);
  return hipGetLastError();
}

}  // namespace veda
