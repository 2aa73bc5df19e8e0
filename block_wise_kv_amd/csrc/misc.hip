// Embedding gather and the final RMSNorm of the block rows.
#include "common.h"
#include "internal.h"

namespace fdllm {

// Sum over the 256 threads of a block; every thread gets the result.
__device__ __forceinline__ float block_sum256(float v, float* red) {
  v = warp_sum(v);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wv] = v;
  __syncthreads();
  return ((red[0] + red[1]) + red[2]) + red[3];
}

// h[m][:] = embed[x[b][row0 + r]] (m = b * rows + r) as float32, and the row's
// sum of squares per 256-column tile into ssq[t][m] (what the next GEMM's
// on-the-fly RMSNorm reads).
template <typename T>
__global__ __launch_bounds__(256) void embed_kernel(const int32_t* __restrict__ x, int seq_len,
                                                    int row0, int rows, int vocab,
                                                    const typename T::store_t* __restrict__ emb,
                                                    int d, float* __restrict__ h,
                                                    float* __restrict__ ssq, int M) {
  __shared__ float red[4];
  const int m = blockIdx.x;
  const int b = m / rows, r = m % rows;
  int tok = x[(size_t)b * seq_len + row0 + r];
  tok = min(max(tok, 0), vocab - 1);  // ids are validated on the host; never read out of bounds
  const typename T::store_t* e = emb + (size_t)tok * d;
  for (int t = 0; t < d / 256; ++t) {
    const int col = t * 256 + threadIdx.x;
    const float v = T::to_f(e[col]);
    h[(size_t)m * d + col] = v;
    const float s = block_sum256(v * v, red);
    if (threadIdx.x == 0) ssq[(size_t)t * M + m] = s;
  }
}

hipError_t launch_embed(int dt, const int32_t* x, int seq_len, int batch, int row0, int rows,
                        const void* embed, int d, float* h, float* ssq, int vocab,
                        hipStream_t st) {
  const int M = batch * rows;
  if (M <= 0) return hipSuccess;
  if (dt == kBF16)
    hipLaunchKernelGGL(embed_kernel<BF16>, dim3(M), dim3(256), 0, st, x, seq_len, row0, rows,
                       vocab, (const uint16_t*)embed, d, h, ssq, M);
  else
    hipLaunchKernelGGL(embed_kernel<F32>, dim3(M), dim3(256), 0, st, x, seq_len, row0, rows, vocab,
                       (const float*)embed, d, h, ssq, M);
  return hipGetLastError();
}

// hidden[b][j][:] = h[m] * rsqrt(sum_t ssq[t][m] / d + eps) * gain (float32),
// m = b * rows + off + j.
template <typename T>
__global__ __launch_bounds__(256) void final_norm_kernel(const float* __restrict__ h,
                                                         const float* __restrict__ ssq, int d,
                                                         int M, int rows, int off, int blk_len,
                                                         const typename T::store_t* __restrict__ gain,
                                                         float eps, float* __restrict__ out) {
  const int o = blockIdx.x;
  const int b = o / blk_len, j = o % blk_len;
  const int m = b * rows + off + j;
  float s = 0.f;
  for (int t = 0; t < d / 256; ++t) s += ssq[(size_t)t * M + m];
  const float rinv = rsqrtf(s / (float)d + eps);
  for (int col = threadIdx.x; col < d; col += 256)
    out[(size_t)o * d + col] = h[(size_t)m * d + col] * rinv * T::to_f(gain[col]);
}

hipError_t launch_final_norm(int dt, const float* h, const float* ssq, int d, int batch, int rows,
                             int off, int blk_len, const void* gain, float eps, void* hidden,
                             hipStream_t st) {
  const int n = batch * blk_len;
  const int M = batch * rows;
  if (dt == kBF16)
    hipLaunchKernelGGL(final_norm_kernel<BF16>, dim3(n), dim3(256), 0, st, h, ssq, d, M, rows, off,
                       blk_len, (const uint16_t*)gain, eps, (float*)hidden);
  else
    hipLaunchKernelGGL(final_norm_kernel<F32>, dim3(n), dim3(256), 0, st, h, ssq, d, M, rows, off,
                       blk_len, (const float*)gain, eps, (float*)hidden);
  return hipGetLastError();
}

}  // namespace fdllm
