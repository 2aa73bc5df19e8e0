// Embedding gather and the final RMSNorm of the block rows.
#include "common.h"
#include "internal.h"

namespace fdllm {

// h[m][:] = embed[x[b][row0 + r]] (m = b * rows + r) as float32, the row's
// sum of squares per 256-column tile into ssq[t][m] (from which the next
// GEMM's epilogue takes the RMSNorm row factor), and h * gain in the split
// activation layout (the next GEMM's input). Thread c8 handles columns
// 8 c8 .. 8 c8 + 7; the 32 threads of a 256-column tile are one half wave.
template <typename T>
__global__ __launch_bounds__(256) void embed_kernel(const int32_t* __restrict__ x, int seq_len,
                                                    int row0, int rows, int vocab,
                                                    const typename T::store_t* __restrict__ emb,
                                                    int d, float* __restrict__ h,
                                                    float* __restrict__ ssq, int M,
                                                    const typename T::store_t* __restrict__ gain,
                                                    char* __restrict__ xs) {
  using E = typename T::store_t;
  const int m = blockIdx.x;
  const int b = m / rows, r = m % rows;
  int tok = x[(size_t)b * seq_len + row0 + r];
  tok = min(max(tok, 0), vocab - 1);  // ids are validated on the host; never read out of bounds
  const E* e = emb + (size_t)tok * d;
  for (int c8 = threadIdx.x; c8 < d / 8; c8 += 256) {
    const int col = 8 * c8;
    float v[8], o[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = T::to_f(e[col + j]);
    *(float4*)(h + (size_t)m * d + col) = make_float4(v[0], v[1], v[2], v[3]);
    *(float4*)(h + (size_t)m * d + col + 4) = make_float4(v[4], v[5], v[6], v[7]);
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) s += v[j] * v[j];
#pragma unroll
    for (int o2 = 16; o2 > 0; o2 >>= 1) s += __shfl_xor(s, o2);
    if ((c8 & 31) == 0) ssq[(size_t)(c8 >> 5) * M + m] = s;
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = v[j] * T::to_f(gain[col + j]);
    XSplit<T>::store8(xs, d >> 5, m, col, o);
  }
}

hipError_t launch_embed(int dt, const int32_t* x, int seq_len, int batch, int row0, int rows,
                        const void* embed, int d, float* h, float* ssq, int vocab,
                        const void* gain, void* xs, hipStream_t st) {
  const int M = batch * rows;
  if (M <= 0) return hipSuccess;
  if (dt == kBF16)
    hipLaunchKernelGGL(embed_kernel<BF16>, dim3(M), dim3(256), 0, st, x, seq_len, row0, rows,
                       vocab, (const uint16_t*)embed, d, h, ssq, M, (const uint16_t*)gain,
                       (char*)xs);
  else
    hipLaunchKernelGGL(embed_kernel<F32>, dim3(M), dim3(256), 0, st, x, seq_len, row0, rows, vocab,
                       (const float*)embed, d, h, ssq, M, (const float*)gain, (char*)xs);
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
