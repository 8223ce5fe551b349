// Per-head output error, the objective of the head-aware tiling search.
// [Technical Summary: Veda, §2.2 Head-Aware Tiling, "Offline Selection": the tiling of each
// head is chosen on calibration data by the error between the full-attention output and
// the sparse-attention output]
//
// One workgroup per (batch, head): 1024 threads stream that head's d-element rows of both
// raster tensors in 16-byte pieces (8 pieces of each tensor in flight per thread),
// accumulate sum (a - b)^2 and sum b^2 in fp32 per thread, and reduce in a fixed order
// (deterministic).  HBM-bound; the parallelism is B*H workgroups.
#include "common.h"
#include "kernels.h"

namespace veda {

static constexpr int SE_THREADS = 1024;
static constexpr int SE_UNROLL = 8;

template <int EB>
__global__ void __launch_bounds__(SE_THREADS) head_sq_error_kernel(const uint8_t *__restrict__ a,
                                                                   const uint8_t *__restrict__ b, int n_tokens,
                                                                   int heads, int head_dim, float *__restrict__ err,
                                                                   float *__restrict__ ref_sq) {
  constexpr int EPC = 16 / EB;  // elements per 16-byte piece
  const int h = blockIdx.x, bb = blockIdx.y, t = threadIdx.x;
  const int cpr = head_dim / EPC;                        // pieces per row
  const int64_t row_stride = (int64_t)heads * head_dim * EB;  // bytes between tokens
  const int64_t base = ((int64_t)bb * n_tokens * heads + h) * head_dim * EB;
  float se = 0.f, sr = 0.f;
  const int64_t total = (int64_t)n_tokens * cpr;
  auto accum = [&](const uint4 &va, const uint4 &vb) {
    const uint32_t wa[4] = {va.x, va.y, va.z, va.w}, wb[4] = {vb.x, vb.y, vb.z, vb.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (EB == 2) {
        const float a0 = __uint_as_float(wa[i] << 16), a1 = __uint_as_float(wa[i] & 0xFFFF0000u);
        const float b0 = __uint_as_float(wb[i] << 16), b1 = __uint_as_float(wb[i] & 0xFFFF0000u);
        se = fmaf(a0 - b0, a0 - b0, se);
        se = fmaf(a1 - b1, a1 - b1, se);
        sr = fmaf(b0, b0, sr);
        sr = fmaf(b1, b1, sr);
      } else {
        const float a0 = __uint_as_float(wa[i]), b0 = __uint_as_float(wb[i]);
        se = fmaf(a0 - b0, a0 - b0, se);
        sr = fmaf(b0, b0, sr);
      }
    }
  };
  // SE_UNROLL pieces per thread in flight: all loads of a step are issued before any use
  int64_t e0 = t;
  for (; e0 + (SE_UNROLL - 1) * SE_THREADS < total; e0 += SE_UNROLL * SE_THREADS) {
    uint4 va[SE_UNROLL], vb[SE_UNROLL];
#pragma unroll
    for (int u = 0; u < SE_UNROLL; ++u) {
      const int64_t e = e0 + (int64_t)u * SE_THREADS, n = e / cpr;
      const int64_t o = base + n * row_stride + (e % cpr) * 16;
      va[u] = *reinterpret_cast<const uint4 *>(a + o);
      vb[u] = *reinterpret_cast<const uint4 *>(b + o);
    }
#pragma unroll
    for (int u = 0; u < SE_UNROLL; ++u) accum(va[u], vb[u]);
  }
  for (int64_t e = e0; e < total; e += SE_THREADS) {  // tail: fewer than SE_UNROLL pieces left
    const int64_t n = e / cpr;
    const int64_t o = base + n * row_stride + (e % cpr) * 16;
    accum(*reinterpret_cast<const uint4 *>(a + o), *reinterpret_cast<const uint4 *>(b + o));
  }
  __shared__ float red[2][SE_THREADS];
  red[0][t] = se;
  red[1][t] = sr;
  __syncthreads();
  for (int s = SE_THREADS / 2; s > 0; s >>= 1) {
    if (t < s) {
      red[0][t] += red[0][t + s];
      red[1][t] += red[1][t + s];
    }
    __syncthreads();
  }
  if (t == 0) {
    err[(int64_t)bb * heads + h] = red[0][0];
    if (ref_sq != nullptr) ref_sq[(int64_t)bb * heads + h] = red[1][0];
  }
}

hipError_t launch_head_sq_error(int batch, int n_tokens, int heads, int head_dim, veda_dtype dt, const void *a,
                                const void *b, float *err, float *ref_sq, hipStream_t st) {
  const dim3 grid(heads, batch);
  if (dt == VEDA_BF16)
    head_sq_error_kernel<2><<<grid, SE_THREADS, 0, st>>>((const uint8_t *)a, (const uint8_t *)b, n_tokens, heads,
                                                          head_dim, err, ref_sq);
  else
    head_sq_error_kernel<4><<<grid, SE_THREADS, 0, st>>>((const uint8_t *)a, (const uint8_t *)b, n_tokens, heads,
                                                          head_dim, err, ref_sq);
  return hipGetLastError();
}

}  // namespace veda
