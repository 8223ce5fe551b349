// Per-head output error, the objective of the head-aware tiling search.
// [Technical Summary: Veda, §2.2 Head-Aware Tiling, "Offline Selection": the tiling of each
// head is chosen on calibration data by the error between the full-attention output and
// the sparse-attention output]
//
// Each head's N tokens are cut into C contiguous chunks; one 256-thread workgroup per
// (head, chunk, batch) streams the chunk's d-element rows of both raster tensors in 16-byte
// pieces (8 pieces of each tensor in flight per thread), accumulates sum (a - b)^2 and
// sum b^2 in fp32 and writes one partial pair.  A second kernel adds each head's C partials
// in a fixed order, and then the batches in ascending order, so the result is
// deterministic.  HBM-bound; B*H*C workgroups (C up to 256) keep every CU streaming, where
// one workgroup per head would leave most of them idle.
#include "common.h"
#include "kernels.h"

namespace veda {

static constexpr int SE_THREADS = 256;
static constexpr int SE_UNROLL = 8;
static constexpr int SE_MAX_CHUNKS = 256;

int head_sq_error_chunks(int n_tokens) { return (int)std::min<int64_t>(((int64_t)n_tokens + 255) / 256, SE_MAX_CHUNKS); }

template <int EB>
__global__ void __launch_bounds__(SE_THREADS) head_sq_error_kernel(const uint8_t *__restrict__ a,
                                                                   const uint8_t *__restrict__ b, int n_tokens,
                                                                   int heads, int head_dim, int chunks,
                                                                   float2 *__restrict__ part) {
  const int h = blockIdx.x, c = blockIdx.y, bb = blockIdx.z, t = threadIdx.x;
  const int n0 = (int)((int64_t)n_tokens * c / chunks), n1 = (int)((int64_t)n_tokens * (c + 1) / chunks);
  const int cpr = head_dim * EB / 16;                          // 16-byte pieces per row
  const int64_t row_stride = (int64_t)heads * head_dim * EB;  // bytes between tokens
  const int64_t base = (((int64_t)bb * n_tokens + n0) * heads + h) * head_dim * EB;
  float se = 0.f, sr = 0.f;
  const int total = (n1 - n0) * cpr;  // pieces of this chunk (< 2^31, checked by the caller)
  auto piece = [&](int e) { return base + (int64_t)(e / cpr) * row_stride + (e % cpr) * 16; };
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
  int e0 = t;
  for (; e0 + (SE_UNROLL - 1) * SE_THREADS < total; e0 += SE_UNROLL * SE_THREADS) {
    uint4 va[SE_UNROLL], vb[SE_UNROLL];
#pragma unroll
    for (int u = 0; u < SE_UNROLL; ++u) {
      const int64_t o = piece(e0 + u * SE_THREADS);
      va[u] = load_stream16(a + o);
      vb[u] = load_stream16(b + o);
    }
#pragma unroll
    for (int u = 0; u < SE_UNROLL; ++u) accum(va[u], vb[u]);
  }
  for (int e = e0; e < total; e += SE_THREADS) {  // tail: fewer than SE_UNROLL pieces left
    const int64_t o = piece(e);
    accum(load_stream16(a + o), load_stream16(b + o));
  }
  se = wave_sum(se);
  sr = wave_sum(sr);
  __shared__ float red[2][SE_THREADS / 64];
  const int lane = t & 63, w = t >> 6;
  if (lane == 0) {
    red[0][w] = se;
    red[1][w] = sr;
  }
  __syncthreads();
  if (t == 0) {
    float2 r = {0.f, 0.f};
#pragma unroll
    for (int i = 0; i < SE_THREADS / 64; ++i) {
      r.x += red[0][i];
      r.y += red[1][i];
    }
    part[((int64_t)bb * heads + h) * chunks + c] = r;
  }
}

// One wave per head: for b = 0, 1, ... in turn, lane l adds that (batch, head)'s partials
// l, l + 64, ... in order and a fixed butterfly adds the lanes (err[b, h]); the batch sum
// adds those per-batch results in ascending b.
__global__ void __launch_bounds__(256) head_sq_error_sum_kernel(const float2 *__restrict__ part, int chunks,
                                                                int batch, int heads, float *__restrict__ err,
                                                                float *__restrict__ err_batch_sum,
                                                                float *__restrict__ ref_sq) {
  const int h = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (h >= heads) return;  // whole wave
  float total = 0.f;
  for (int bb = 0; bb < batch; ++bb) {
    const int64_t row = (int64_t)bb * heads + h;
    float se = 0.f, sr = 0.f;
    for (int c = lane; c < chunks; c += 64) {
      const float2 p = part[row * chunks + c];
      se += p.x;
      sr += p.y;
    }
    se = wave_sum(se);
    sr = wave_sum(sr);
    total += se;
    if (lane == 0) {
      err[row] = se;
      if (ref_sq != nullptr) ref_sq[row] = sr;
    }
  }
  if (lane == 0 && err_batch_sum != nullptr) err_batch_sum[h] = total;
}

hipError_t launch_head_sq_error(int batch, int n_tokens, int heads, int head_dim, veda_dtype dt, const void *a,
                                const void *b, float *err, float *err_batch_sum, float *ref_sq, void *ws,
                                hipStream_t st) {
  const int chunks = head_sq_error_chunks(n_tokens);
  float2 *part = static_cast<float2 *>(ws);
  const dim3 grid(heads, chunks, batch);
  if (dt == VEDA_BF16)
    head_sq_error_kernel<2><<<grid, SE_THREADS, 0, st>>>((const uint8_t *)a, (const uint8_t *)b, n_tokens, heads,
                                                          head_dim, chunks, part);
  else
    head_sq_error_kernel<4><<<grid, SE_THREADS, 0, st>>>((const uint8_t *)a, (const uint8_t *)b, n_tokens, heads,
                                                          head_dim, chunks, part);
  head_sq_error_sum_kernel<<<dim3((heads + 3) / 4), 256, 0, st>>>(part, chunks, batch, heads, err, err_batch_sum,
                                                                   ref_sq);
  return hipGetLastError();
}

}  // namespace veda
