// Distillation step of the tile-score estimator.  [Technical Summary: Veda, §2.1 Distilled
// Tile Scoring, "Optimization": a row-wise KL divergence aligns the estimator's tile-score
// distribution with the full-attention reference; the backbone features that feed the
// estimator are stop-gradient, so only the per-head MLP is trained]
//
// For every sampled query tile a (tile i = q_tiles[b, h, a]) of every head:
//   p_a = M[b, h, a, :] / sum_j M[b, h, a, j]        (max-pooled map, normalised per row)
//   s_a = score_scale * y_q[a] . y_k[:]              (estimator logits; y_q[a] is tile i's)
//   L   = mean over all B*H*n_sel rows of KL(p_a || softmax(s_a))
// and the gradients of L with respect to W1 [H, 3d, 256] and W2 [H, 256, 64] (one MLP per
// head, shared by the Q-tile and K-tile descriptors), y = GELU(D W1) W2.
//   dL/ds_a = (softmax(s_a) - p_a) / R
//   dy of Q row a (one row per list entry; an unlisted Q tile gets no gradient, and a tile
//            listed twice has two rows) = score_scale * dL/ds_a . y_k
//   dy_k[j] = score_scale * sum_a dL/ds_a[j] y_q[a]
//   dW2 = sum over the Q and K rows of H1^T dy,  dZ1 = (dy W2^T) * GELU'(Z1),  dW1 = sum D^T dZ1
// Kernels (all deterministic: fixed-order reductions, no atomics):
//   pool_mlp (score.hip)  descriptors D, pre-activations Z1 and outputs y of the listed Q
//                         tiles and of every K tile
//   kl_grad_kernel        one wave per sampled row: logits, softmax, KL, dL/ds, and that
//                         row's dy = score_scale * dL/ds_a . y_k
//   dyk_kernel            dy_k[j] (one wave per key tile)
//   mlp_bwd_rows_kernel   per 32 rows: H1 = GELU(Z1), dZ1 = (dy W2^T) GELU'(Z1), with the
//                         pre-activation Z1 = D W1 kept by the forward pooling kernel
//   atb_mfma_kernel       dW1 = D^T dZ1 and dW2 = H1^T dy per head on fp32 MFMA, 64 x 64
//                         tiles, four waves per tile over quarters of the rows
//   loss_kernel, sgd_kernel
// The step is small next to the forward path (a few GFLOP); fp32 throughout.
#include "common.h"
#include "kernels.h"

namespace veda {

static constexpr int DS_HID = 256, DS_OUT = 64;

static inline size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace layout (floats): y [2][B][H][n_t][64] | D [2][B][H][n_t][3d] | dS [B][H][n_sel][n_t]
// | dY [2][B][H][n_t][64] | H1 [2][B][H][n_t][256] | dZ1 (same) | loss [B*H*n_sel].  In the Q
// half of y, D, dY, H1 and dZ1, row a of a (b, h) block is list entry a (n_sel <= n_t rows).
struct DistillWs {
  float *y, *desc, *ds, *dy, *h1, *dz1, *loss;
};

static size_t ws_parts(const Geo &g, int n_sel, size_t *off) {
  const size_t rows = 2 * (size_t)g.B * g.H * g.nt, sel = (size_t)g.B * g.H * n_sel;
  const size_t sz[7] = {rows * DS_OUT, rows * 3 * g.d, sel * g.nt, rows * DS_OUT, rows * DS_HID, rows * DS_HID, sel};
  size_t o = 0;
  for (int i = 0; i < 7; ++i) {
    off[i] = o;
    o += al256(sz[i] * sizeof(float));
  }
  return o;
}

size_t distill_workspace_bytes(const Geo &g, int n_sel) {
  size_t off[7];
  return ws_parts(g, n_sel, off);
}

__device__ __forceinline__ float gelu_f(float x) { return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f)); }
__device__ __forceinline__ float gelu_grad(float x) {
  // d/dx [x Phi(x)] = Phi(x) + x phi(x)
  return 0.5f * (1.0f + erff(x * 0.70710678118654752f)) + x * 0.3989422804014327f * expf(-0.5f * x * x);
}

// One wave per sampled row (b, h, a); 4 rows per workgroup.
template <int MAXM>
__global__ void __launch_bounds__(256) kl_grad_kernel(const float *__restrict__ y, int n_sel,
                                                      const float *__restrict__ target, float scale,
                                                      float inv_rows, float *__restrict__ ds, float *__restrict__ dyq,
                                                      float *__restrict__ loss_rows, Geo g, HeadShapes hs) {
  __shared__ float dsl[4][64 * MAXM];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * 4 + wv;  // (b*H + h)*n_sel + a
  if (row >= (int64_t)g.B * g.H * n_sel) return;      // whole wave; no barrier follows
  const int64_t bh = row / n_sel;
  const int nt = g.nt;
  // this head's key tiles: the columns past them (padded tilings) are not in the softmax,
  // carry no target and get no gradient
  const int hh = (int)(bh % g.H);
  const int nth = g.padded ? head_tiles(hs.s[hh][0], hs.s[hh][1], hs.s[hh][2], g.T, g.Hs, g.Ws) : nt;
  const int64_t a = row - bh * n_sel;       // list position: the Q rows are the listed tiles
  const float *yq = y + (bh * nt + a) * DS_OUT;
  const float *yk = y + (((int64_t)g.B * g.H + bh) * nt) * DS_OUT;
  const float *m = target + row * nt;
  float s[MAXM], mt[MAXM];
  float mx = -INFINITY, msum = 0.f;
#pragma unroll
  for (int u = 0; u < MAXM; ++u) {
    const int j = 64 * u + lane;
    s[u] = -INFINITY;
    mt[u] = 0.f;
    if (j < nth) {
      const float4 *kr = reinterpret_cast<const float4 *>(yk + (int64_t)j * DS_OUT);
      const float4 *qr = reinterpret_cast<const float4 *>(yq);
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < DS_OUT / 4; ++c) {
        const float4 a = qr[c], b = kr[c];
        acc = fmaf(a.x, b.x, acc);
        acc = fmaf(a.y, b.y, acc);
        acc = fmaf(a.z, b.z, acc);
        acc = fmaf(a.w, b.w, acc);
      }
      s[u] = acc * scale;
      mt[u] = m[j];
      mx = fmaxf(mx, s[u]);
      msum += mt[u];
    }
  }
  mx = wave_max(mx);
  msum = wave_sum(msum);
  float se = 0.f;
#pragma unroll
  for (int u = 0; u < MAXM; ++u)
    if (64 * u + lane < nth) se += expf(s[u] - mx);
  se = wave_sum(se);
  const float lse = mx + logf(se), inv_m = 1.0f / msum;
  float kl = 0.f;
#pragma unroll
  for (int u = 0; u < MAXM; ++u) {
    const int j = 64 * u + lane;
    if (j < nth) {
      const float p = mt[u] * inv_m, logq = s[u] - lse;
      if (p > 0.f) kl += p * (logf(p) - logq);
      const float d = (expf(logq) - p) * inv_rows;
      ds[row * nt + j] = d;
      dsl[wv][j] = d;
    } else if (j < nt) {
      ds[row * nt + j] = 0.f;
      dsl[wv][j] = 0.f;
    }
  }
  kl = wave_sum(kl);
  if (lane == 0) loss_rows[row] = kl;
  // g_a[c] = scale * sum_j dS[j] y_k[j][c]: lane c walks the row that this wave's lanes
  // have just written to LDS (the fence completes those writes and orders the reads after)
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
  float acc = 0.f;
  for (int j = 0; j < nt; ++j) acc = fmaf(dsl[wv][j], yk[(int64_t)j * DS_OUT + lane], acc);
  dyq[(bh * nt + a) * DS_OUT + lane] = acc * scale;  // dy of Q row a (one row per list entry)
}

// dy_k[b, h, j][c] = scale * sum_a dS[a][j] y_q[a][c] (Q row a is list entry a), in order of a.
__global__ void __launch_bounds__(64) dyk_kernel(int n_sel, const float *__restrict__ ds, const float *__restrict__ y,
                                                 float scale, float *__restrict__ dy, Geo g) {
  const int j = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int c = threadIdx.x;
  const int64_t kbase = (int64_t)g.B * g.H;
  float acc = 0.f;
  for (int a = 0; a < n_sel; ++a) acc = fmaf(ds[(bh * n_sel + a) * g.nt + j], y[(bh * g.nt + a) * DS_OUT + c], acc);
  dy[((kbase + bh) * g.nt + j) * DS_OUT + c] = acc * scale;
}

// 32 rows of one (Q|K, b, h) block of nrows rows (Q: the list entries, K: every tile),
// thread u = hidden unit u: the forward pass left the pre-activation Z1 = D W1 in h1; this
// replaces it by H1 = GELU(Z1) and writes dZ1 = (dy W2^T) * GELU'(Z1).
__global__ void __launch_bounds__(256) mlp_bwd_rows_kernel(const float *__restrict__ dy, const float *__restrict__ w2,
                                                           float *__restrict__ h1, float *__restrict__ dz1, int which,
                                                           int nrows, Geo g) {
  __shared__ float Yl[32 * DS_OUT];  // dy of the 32 rows
  const int ngrp = (nrows + 31) / 32;
  const int grp = blockIdx.x % ngrp;
  const int64_t wbh = (int64_t)which * g.B * g.H + blockIdx.x / ngrp;  // (which*B + b)*H + h
  const int h = (int)(wbh % g.H);
  const int r0 = grp * 32, nr = min(32, nrows - r0);
  const int u = threadIdx.x;
  for (int e = u; e < 32 * DS_OUT; e += 256) {
    const int r = e / DS_OUT;
    Yl[e] = r < nr ? dy[(wbh * g.nt + r0 + r) * DS_OUT + e % DS_OUT] : 0.f;
  }
  float z[32];
#pragma unroll
  for (int r = 0; r < 32; ++r) z[r] = r < nr ? h1[(wbh * g.nt + r0 + r) * DS_HID + u] : 0.f;
  __syncthreads();
  const float *W2 = w2 + ((int64_t)h * DS_HID + u) * DS_OUT;
  float dh[32];
#pragma unroll
  for (int r = 0; r < 32; ++r) dh[r] = 0.f;
  for (int o = 0; o < DS_OUT; ++o) {
    const float wv = W2[o];
#pragma unroll
    for (int r = 0; r < 32; ++r) dh[r] = fmaf(Yl[r * DS_OUT + o], wv, dh[r]);
  }
#pragma unroll
  for (int r = 0; r < 32; ++r) {
    if (r < nr) {
      const int64_t o = (wbh * g.nt + r0 + r) * DS_HID + u;
      h1[o] = gelu_f(z[r]);
      dz1[o] = dh[r] * gelu_grad(z[r]);
    }
  }
}

// C[h] (M x N) = sum over rows of A[row][m] * B[row][n], rows = the 2*B segments (Q|K, b) of
// n_t rows of head h (A row stride lda, B row stride ldb, floats), on fp32 MFMA 32x32x2
// (A[m = lane%32][k = lane/32], B[k = lane/32][n = lane%32], D[m = 8*(r/4) + 4*(lane/32) + r%4]
// [n = lane%32]).  One workgroup per 64 x 64 output tile (2 x 2 blocks): each of its four
// waves sums a contiguous quarter of the rows, two rows per step, with the operands loaded
// PF steps ahead in register rings; wave 0 then adds the four partial tiles in wave order.
// Every sum runs in a fixed order, so the result is deterministic.  M and N are multiples
// of 64.
__global__ void __launch_bounds__(256) atb_mfma_kernel(const float *__restrict__ A, int lda,
                                                       const float *__restrict__ Bm, int ldb, int M, int N,
                                                       float *__restrict__ C, int nq, Geo g) {
  constexpr int PF = 8;
  __shared__ float red[3][4][16][64];  // partial tiles of waves 1..3: [wave][block][r][lane]
  const int tm = blockIdx.x, tn = blockIdx.y, h = blockIdx.z;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, lr = lane & 31, kh = lane >> 5;
  // steps of two rows: first the B Q segments (nq rows each), then the B K segments (n_t rows)
  const int hq = (nq + 1) >> 1, hk = (g.nt + 1) >> 1, nsq = g.B * hq, nsteps = nsq + g.B * hk;
  const int q4 = (nsteps + 3) / 4, s_begin = wv * q4, s_end = min(nsteps, s_begin + q4);  // this wave's steps
  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][jj][r] = 0.f;
  const float *Ab = A + 64 * tm + lr, *Bb = Bm + 64 * tn + lr;
  auto load = [&](int s, float (&av)[2], float (&bv)[2]) {
    const bool qs = s < nsq;
    const int hs = qs ? hq : hk, s2 = qs ? s : s - nsq;
    const int sg = s2 / hs, row = 2 * (s2 - sg * hs) + kh;  // segment (b) within Q or K, and its row
    const bool ok = s < s_end && row < (qs ? nq : g.nt);
    const int64_t rr = ok ? (((int64_t)(qs ? 0 : g.B) + sg) * g.H + h) * g.nt + row : 0;  // clamped: in bounds
    av[0] = Ab[rr * lda];
    av[1] = Ab[rr * lda + 32];
    bv[0] = Bb[rr * ldb];
    bv[1] = Bb[rr * ldb + 32];
    if (!ok) av[0] = av[1] = 0.f;
  };
  float ar[PF][2], br[PF][2];
#pragma unroll
  for (int p = 0; p < PF; ++p) load(s_begin + p, ar[p], br[p]);
#pragma unroll 1
  for (int s0 = s_begin; s0 < s_end; s0 += PF) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      const float a0 = ar[p][0], a1 = ar[p][1], b0 = br[p][0], b1 = br[p][1];
      acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b0, acc[0][0], 0, 0, 0);
      acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b1, acc[0][1], 0, 0, 0);
      acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b0, acc[1][0], 0, 0, 0);
      acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b1, acc[1][1], 0, 0, 0);
      load(s0 + p + PF, ar[p], br[p]);
      __builtin_amdgcn_sched_barrier(0);  // keep each load a full ring ahead of its use
    }
  }
  // the four waves' partial sums, added in wave order by wave 0
  if (wv > 0) {
#pragma unroll
    for (int bk = 0; bk < 4; ++bk)
#pragma unroll
      for (int r = 0; r < 16; ++r) red[wv - 1][bk][r][lane] = acc[bk >> 1][bk & 1][r];
  }
  __syncthreads();
  if (wv == 0) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float v = acc[mb][nb][r];
#pragma unroll
          for (int o = 0; o < 3; ++o) v += red[o][2 * mb + nb][r][lane];
          const int m = 64 * tm + 32 * mb + 8 * (r >> 2) + 4 * kh + (r & 3), n = 64 * tn + 32 * nb + lr;
          C[((int64_t)h * M + m) * N + n] = v;
        }
  }
}

// loss = (sum of the row KLs) / rows, summed in a fixed order by one workgroup.
__global__ void __launch_bounds__(256) loss_kernel(const float *__restrict__ rows, int64_t n, float *__restrict__ loss) {
  __shared__ float red[256];
  float acc = 0.f;
  for (int64_t e = threadIdx.x; e < n; e += 256) acc += rows[e];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) loss[0] = red[0] / (float)n;
}

__global__ void __launch_bounds__(256) sgd_kernel(float *__restrict__ w, const float *__restrict__ dw, float lr,
                                                  int64_t n) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e < n) w[e] -= lr * dw[e];
}

template <int MAXM>
static void launch_kl(const Geo &g, const float *y, int n_sel, const float *target,
                      float scale, float inv_rows, const DistillWs &w, const HeadShapes &hs, hipStream_t st) {
  const int64_t rows = (int64_t)g.B * g.H * n_sel;
  kl_grad_kernel<MAXM><<<dim3((unsigned)((rows + 3) / 4)), 256, 0, st>>>(y, n_sel, target, scale, inv_rows, w.ds,
                                                                       w.dy, w.loss, g, hs);
}

hipError_t launch_distill(const Geo &g, const HeadShapes &hs, veda_dtype dt, const void *q, const void *k, float *w1,
                          float *w2, float score_scale, const int32_t *q_tiles, int n_sel, const float *target,
                          float *loss, float *dw1, float *dw2, float lr, void *ws, hipStream_t st) {
  size_t off[7];
  ws_parts(g, n_sel, off);
  char *base = static_cast<char *>(ws);
  DistillWs w{(float *)(base + off[0]), (float *)(base + off[1]), (float *)(base + off[2]), (float *)(base + off[3]),
              (float *)(base + off[4]), (float *)(base + off[5]), (float *)(base + off[6])};
  const int d3 = 3 * g.d;
  const size_t desc_half = (size_t)g.B * g.H * g.nt * d3;
  // forward: descriptors and MLP outputs of every Q and K tile (shared weights)
  // Q rows: the listed tiles only (an unlisted Q tile gets no gradient); the pre-activation
  // hidden layer goes to h1, which the backward rows kernel turns into GELU
  // (on a padded tiling the descriptors of the tiles past a head's own count, and so their
  // MLP outputs and gradients, are zero)
  const hipError_t pe = launch_pool_mlp(g, dt, q, k, w1, w2, w1, w2, w.y, w.desc, w.desc + desc_half, st, &hs,
                                        nullptr, false, w.h1, q_tiles, n_sel);
  if (pe != hipSuccess) return pe;
  const int64_t rows = (int64_t)g.B * g.H * n_sel;
  const float inv_rows = 1.0f / (float)rows;
  if (g.nt <= 64)
    launch_kl<1>(g, w.y, n_sel, target, score_scale, inv_rows, w, hs, st);
  else if (g.nt <= 256)
    launch_kl<4>(g, w.y, n_sel, target, score_scale, inv_rows, w, hs, st);
  else if (g.nt <= 640)
    launch_kl<10>(g, w.y, n_sel, target, score_scale, inv_rows, w, hs, st);
  else if (g.nt <= 1280)
    launch_kl<20>(g, w.y, n_sel, target, score_scale, inv_rows, w, hs, st);
  else  // the widest padded heads (e.g. (16, 2, 4) on T = 40: 1440 tiles)
    launch_kl<24>(g, w.y, n_sel, target, score_scale, inv_rows, w, hs, st);
  const dim3 gi(g.nt, g.B * g.H);
  dyk_kernel<<<gi, 64, 0, st>>>(n_sel, w.ds, w.y, score_scale, w.dy, g);
  const int ngrp = (g.nt + 31) / 32;
  const int ngrp_q = (n_sel + 31) / 32;
  mlp_bwd_rows_kernel<<<dim3(ngrp_q * g.B * g.H), 256, 0, st>>>(w.dy, w2, w.h1, w.dz1, 0, n_sel, g);
  mlp_bwd_rows_kernel<<<dim3(ngrp * g.B * g.H), 256, 0, st>>>(w.dy, w2, w.h1, w.dz1, 1, g.nt, g);
  // 3d is 384 (bf16) or 192 (fp32): both multiples of the 64-wide output tile
  atb_mfma_kernel<<<dim3(d3 / 64, DS_HID / 64, g.H), 256, 0, st>>>(w.desc, d3, w.dz1, DS_HID, d3, DS_HID, dw1,
                                                                     n_sel, g);
  atb_mfma_kernel<<<dim3(DS_HID / 64, DS_OUT / 64, g.H), 256, 0, st>>>(w.h1, DS_HID, w.dy, DS_OUT, DS_HID, DS_OUT, dw2,
                                                                        n_sel, g);
  loss_kernel<<<1, 256, 0, st>>>(w.loss, rows, loss);
  if (lr != 0.f) {
    const int64_t n1 = (int64_t)g.H * d3 * DS_HID, n2 = (int64_t)g.H * DS_HID * DS_OUT;
    sgd_kernel<<<dim3((unsigned)((n1 + 255) / 256)), 256, 0, st>>>(w1, dw1, lr, n1);
    sgd_kernel<<<dim3((unsigned)((n2 + 255) / 256)), 256, 0, st>>>(w2, dw2, lr, n2);
  }
  return hipGetLastError();
}

}  // namespace veda
