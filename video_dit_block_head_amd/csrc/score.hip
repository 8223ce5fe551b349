// Distilled tile scoring: TripPool descriptors -> per-head MLP -> tile scores -> row
// softmax / top-k.  [Technical Summary: Veda, §2.1 Distilled Tile Scoring]
//
//  pool_kernel   HBM-bound stream over Q and K tiles; one workgroup per (tile, head, b, Q|K).
//  mlp_kernel    y = GELU(desc W1) W2 on 32 descriptors per workgroup, fp32 FMA.
//  score_kernel  16 query-tile rows per workgroup, one wave per 4 rows; row held in
//                registers (lane owns columns lane, lane+64, ...); softmax and top-k are
//                wave-level (ballot/popcount), deterministic.
//  topk_kernel   standalone top-k, one wave per row.
#include "common.h"
#include "kernels.h"

namespace veda {

static constexpr int MLP_ROWS = 32;

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t score_workspace_bytes(const Geo &g, int hidden, int mlp_out) {
  (void)hidden;
  const size_t nt = (size_t)g.B * g.H * g.nt;
  return 2 * align256(nt * 3 * g.d * sizeof(float)) + align256(2 * nt * mlp_out * sizeof(float));
}

// ---------------------------------------------------------------------------------------
// TripPool.  Thread (row group rg = t/16, chunk = t%16) accumulates rows rg, rg+16, ... of
// its 16-byte channel chunk; partials are combined in a fixed order (deterministic).
template <int EB>
__global__ void __launch_bounds__(256) pool_kernel(const uint8_t *__restrict__ q, const uint8_t *__restrict__ k,
                                                   float *__restrict__ qdesc, float *__restrict__ kdesc, Geo g) {
  constexpr int EPC = 16 / EB;
  const int j = blockIdx.x, h = blockIdx.y, b = blockIdx.z >> 1, which = blockIdx.z & 1;
  const uint8_t *src = (which ? k : q) + ((((int64_t)b * g.H + h) * g.N + (int64_t)j * g.P) * g.d) * EB;
  const int chunk = threadIdx.x & 15, rg = threadIdx.x >> 4;
  float s[EPC], mx[EPC], mn[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) {
    s[e] = 0.f;
    mx[e] = -INFINITY;
    mn[e] = INFINITY;
  }
  const int64_t row_bytes = (int64_t)g.d * EB;
  for (int o = rg; o < g.P; o += 16) {
    const uint4 v = *reinterpret_cast<const uint4 *>(src + o * row_bytes + chunk * 16);
    float x[EPC];
    if (EB == 2) {
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[2 * e] = __uint_as_float(w[e] << 16);
        x[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
      }
    } else {
      x[0] = __uint_as_float(v.x);
      x[1] = __uint_as_float(v.y);
      x[2] = __uint_as_float(v.z);
      x[3] = __uint_as_float(v.w);
    }
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      s[e] += x[e];
      mx[e] = fmaxf(mx[e], x[e]);
      mn[e] = fminf(mn[e], x[e]);
    }
  }
  __shared__ float part[3][16][128];
#pragma unroll
  for (int e = 0; e < EPC; ++e) {
    part[0][rg][chunk * EPC + e] = s[e];
    part[1][rg][chunk * EPC + e] = mx[e];
    part[2][rg][chunk * EPC + e] = mn[e];
  }
  __syncthreads();
  if (threadIdx.x < g.d) {
    const int c = threadIdx.x;
    float ss = 0.f, xx = -INFINITY, nn = INFINITY;
    for (int r = 0; r < 16; ++r) {
      ss += part[0][r][c];
      xx = fmaxf(xx, part[1][r][c]);
      nn = fminf(nn, part[2][r][c]);
    }
    float *dst = (which ? kdesc : qdesc) + (((int64_t)b * g.H + h) * g.nt + j) * 3 * g.d;
    dst[c] = ss * (1.0f / (float)g.P);  // P is a power of two: exact
    dst[g.d + c] = xx;
    dst[2 * g.d + c] = nn;
  }
}

// ---------------------------------------------------------------------------------------
// Per-head MLP on MLP_ROWS descriptors.  Layer 1: thread t owns hidden unit t for all rows
// (descriptors transposed in LDS so a k-step is 8 broadcast 16-byte reads).  Layer 2:
// thread (o = t%64, group = t/64) owns output o for rows 8*group .. 8*group+7.
__device__ __forceinline__ float gelu_erf(float x) { return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f)); }

__global__ void __launch_bounds__(256) mlp_kernel(const float *__restrict__ qdesc, const float *__restrict__ kdesc,
                                                  const float *__restrict__ w1q, const float *__restrict__ w2q,
                                                  const float *__restrict__ w1k, const float *__restrict__ w2k,
                                                  float *__restrict__ y, Geo g, int hidden, int mout) {
  constexpr int R = MLP_ROWS, RS = R + 4;  // padded row stride (floats)
  const int D3 = 3 * g.d;
  const int r0 = blockIdx.x * R, h = blockIdx.y, b = blockIdx.z >> 1, which = blockIdx.z & 1;
  const float *desc = (which ? kdesc : qdesc) + (((int64_t)b * g.H + h) * g.nt) * D3;
  const float *W1 = (which ? w1k : w1q) + (int64_t)h * D3 * hidden;
  const float *W2 = (which ? w2k : w2q) + (int64_t)h * hidden * mout;
  __shared__ __attribute__((aligned(16))) float buf[384 * RS];  // descT [D3][RS], then hidT [hidden][RS]
  const int t = threadIdx.x;
  for (int e = t; e < R * D3; e += 256) {
    const int r = e / D3, c = e % D3;
    buf[c * RS + r] = (r0 + r < g.nt) ? desc[(int64_t)(r0 + r) * D3 + c] : 0.f;
  }
  __syncthreads();
  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.f;
  if (t < hidden) {
    for (int c = 0; c < D3; ++c) {
      const float w = W1[(int64_t)c * hidden + t];
      const float4 *dv = reinterpret_cast<const float4 *>(&buf[c * RS]);
#pragma unroll
      for (int r4 = 0; r4 < R / 4; ++r4) {
        const float4 dd = dv[r4];
        acc[4 * r4 + 0] = fmaf(dd.x, w, acc[4 * r4 + 0]);
        acc[4 * r4 + 1] = fmaf(dd.y, w, acc[4 * r4 + 1]);
        acc[4 * r4 + 2] = fmaf(dd.z, w, acc[4 * r4 + 2]);
        acc[4 * r4 + 3] = fmaf(dd.w, w, acc[4 * r4 + 3]);
      }
    }
  }
  __syncthreads();  // every thread is done reading descT
  if (t < hidden) {
    float4 *hv = reinterpret_cast<float4 *>(&buf[t * RS]);
#pragma unroll
    for (int r4 = 0; r4 < R / 4; ++r4)
      hv[r4] = make_float4(gelu_erf(acc[4 * r4]), gelu_erf(acc[4 * r4 + 1]), gelu_erf(acc[4 * r4 + 2]),
                           gelu_erf(acc[4 * r4 + 3]));
  }
  __syncthreads();
  const int o = t & 63, grp = t >> 6;
  if (o < mout) {
    float a2[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) a2[i] = 0.f;
    for (int c = 0; c < hidden; ++c) {
      const float w = W2[(int64_t)c * mout + o];
      const float4 *hv = reinterpret_cast<const float4 *>(&buf[c * RS + grp * 8]);
      const float4 x0 = hv[0], x1 = hv[1];
      a2[0] = fmaf(x0.x, w, a2[0]);
      a2[1] = fmaf(x0.y, w, a2[1]);
      a2[2] = fmaf(x0.z, w, a2[2]);
      a2[3] = fmaf(x0.w, w, a2[3]);
      a2[4] = fmaf(x1.x, w, a2[4]);
      a2[5] = fmaf(x1.y, w, a2[5]);
      a2[6] = fmaf(x1.z, w, a2[6]);
      a2[7] = fmaf(x1.w, w, a2[7]);
    }
    float *yo = y + ((((int64_t)which * g.B + b) * g.H + h) * g.nt) * mout;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = r0 + grp * 8 + i;
      if (r < g.nt) yo[(int64_t)r * mout + o] = a2[i];
    }
  }
}

// ---------------------------------------------------------------------------------------
// Tile scores S = scale * y_q y_k^T for 16 query-tile rows, then per-row outputs.
// Each dot product uses four interleaved fp32 partial sums (lower rounding error).
template <int MAXM>
__global__ void __launch_bounds__(256) score_kernel(const float *__restrict__ y, Geo g, int mout, float scale,
                                                    float *__restrict__ scores, float *__restrict__ probs, int topk,
                                                    int32_t *__restrict__ idx) {
  const int i0 = blockIdx.x * 16, h = blockIdx.y, b = blockIdx.z;
  const int nt = g.nt;
  const float *yq = y + (((int64_t)b * g.H + h) * nt) * mout;
  const float *yk = y + ((((int64_t)g.B + b) * g.H + h) * nt) * mout;
  __shared__ __attribute__((aligned(16))) float sq[16][64];
  __shared__ __attribute__((aligned(16))) float sk[64][68];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  for (int e = t; e < 16 * 64; e += 256) {
    const int r = e >> 6, c = e & 63;
    sq[r][c] = (i0 + r < nt && c < mout) ? yq[(int64_t)(i0 + r) * mout + c] : 0.f;
  }
  float sc[4][MAXM];
#pragma unroll
  for (int m = 0; m < MAXM; ++m) {
    __syncthreads();
    for (int e = t; e < 64 * 64; e += 256) {
      const int r = e >> 6, c = e & 63, jj = 64 * m + r;
      sk[r][c] = (jj < nt && c < mout) ? yk[(int64_t)jj * mout + c] : 0.f;
    }
    __syncthreads();
    float acc[4][4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
#pragma unroll
      for (int p = 0; p < 4; ++p) acc[rr][p] = 0.f;
#pragma unroll 4
    for (int c = 0; c < 64; c += 4) {
      const float4 kv = *reinterpret_cast<const float4 *>(&sk[lane][c]);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const float4 qv = *reinterpret_cast<const float4 *>(&sq[4 * w + rr][c]);
        acc[rr][0] = fmaf(qv.x, kv.x, acc[rr][0]);
        acc[rr][1] = fmaf(qv.y, kv.y, acc[rr][1]);
        acc[rr][2] = fmaf(qv.z, kv.z, acc[rr][2]);
        acc[rr][3] = fmaf(qv.w, kv.w, acc[rr][3]);
      }
    }
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) sc[rr][m] = ((acc[rr][0] + acc[rr][1]) + (acc[rr][2] + acc[rr][3])) * scale;
  }
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int i = i0 + 4 * w + rr;
    if (i >= nt) continue;  // wave-uniform
    const int64_t row = ((int64_t)b * g.H + h) * nt + i;
    if (scores != nullptr) {
#pragma unroll
      for (int m = 0; m < MAXM; ++m) {
        const int jj = 64 * m + lane;
        if (jj < nt) scores[row * nt + jj] = sc[rr][m];
      }
    }
    if (probs != nullptr) {
      float mx = -INFINITY;
#pragma unroll
      for (int m = 0; m < MAXM; ++m)
        if (64 * m + lane < nt) mx = fmaxf(mx, sc[rr][m]);
      mx = wave_max(mx);
      float e[MAXM], sum = 0.f;
#pragma unroll
      for (int m = 0; m < MAXM; ++m) {
        e[m] = (64 * m + lane < nt) ? expf(sc[rr][m] - mx) : 0.f;
        sum += e[m];
      }
      sum = wave_sum(sum);
      const float inv = 1.0f / sum;
#pragma unroll
      for (int m = 0; m < MAXM; ++m) {
        const int jj = 64 * m + lane;
        if (jj < nt) probs[row * nt + jj] = e[m] * inv;
      }
    }
    if (topk > 0) {
      uint32_t key[MAXM];
#pragma unroll
      for (int m = 0; m < MAXM; ++m) key[m] = (64 * m + lane < nt) ? float_key(sc[rr][m]) : 0u;
      wave_topk<MAXM>(key, nt, topk, lane, idx + row * topk, nullptr);
    }
  }
}

template <int MAXM>
__global__ void __launch_bounds__(256) topk_kernel(const float *__restrict__ scores, int64_t rows, int n_cols, int k,
                                                   int32_t *__restrict__ idx, uint8_t *__restrict__ mask) {
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
  wave_topk<MAXM>(key, n_cols, k, lane, idx + row * k, mask ? mask + row * n_cols : nullptr);
}

// ---------------------------------------------------------------------------------------
template <int MAXM>
static void launch_score_t(const Geo &g, const float *y, int mout, float scale, float *scores, float *probs, int topk,
                           int32_t *idx, hipStream_t st) {
  score_kernel<MAXM><<<dim3((g.nt + 15) / 16, g.H, g.B), 256, 0, st>>>(y, g, mout, scale, scores, probs, topk, idx);
}

hipError_t launch_score(const Geo &g, veda_dtype dt, const void *q, const void *k, const float *w1q,
                        const float *w2q, const float *w1k, const float *w2k, int hidden, int mlp_out, float scale,
                        float *scores, float *probs, float *q_desc, float *k_desc, int topk, int32_t *idx,
                        void *ws, hipStream_t st) {
  const size_t nt_all = (size_t)g.B * g.H * g.nt;
  uint8_t *p = (uint8_t *)ws;
  float *qd = q_desc ? q_desc : (float *)p;
  p += align256(nt_all * 3 * g.d * sizeof(float));
  float *kd = k_desc ? k_desc : (float *)p;
  p += align256(nt_all * 3 * g.d * sizeof(float));
  float *y = (float *)p;

  const dim3 pg(g.nt, g.H, 2 * g.B);
  if (dt == VEDA_BF16)
    pool_kernel<2><<<pg, 256, 0, st>>>((const uint8_t *)q, (const uint8_t *)k, qd, kd, g);
  else
    pool_kernel<4><<<pg, 256, 0, st>>>((const uint8_t *)q, (const uint8_t *)k, qd, kd, g);
  mlp_kernel<<<dim3((g.nt + MLP_ROWS - 1) / MLP_ROWS, g.H, 2 * g.B), 256, 0, st>>>(qd, kd, w1q, w2q, w1k, w2k, y, g,
                                                                                 hidden, mlp_out);
  if (g.nt <= 64)
    launch_score_t<1>(g, y, mlp_out, scale, scores, probs, topk, idx, st);
  else if (g.nt <= 256)
    launch_score_t<4>(g, y, mlp_out, scale, scores, probs, topk, idx, st);
  else if (g.nt <= 640)
    launch_score_t<10>(g, y, mlp_out, scale, scores, probs, topk, idx, st);
  else
    launch_score_t<20>(g, y, mlp_out, scale, scores, probs, topk, idx, st);
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
