// Embedding gather and the final RMSNorm of the block rows.
#include <algorithm>

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
  __shared__ float s_rinv;
  const int o = blockIdx.x;
  const int b = o / blk_len, j = o % blk_len;
  const int m = b * rows + off + j;
  // the row's d / 256 (<= 32) partial sums of squares: one load per lane of
  // the first wave, summed by a fixed butterfly
  if (threadIdx.x < 64) {
    float s = threadIdx.x < d / 256 ? ssq[(size_t)threadIdx.x * M + m] : 0.f;
#pragma unroll
    for (int k = 1; k < 64; k <<= 1) s += __shfl_xor(s, k);
    if (threadIdx.x == 0) s_rinv = rsqrtf(s / (float)d + eps);
  }
  __syncthreads();
  const float rinv = s_rinv;
  for (int c4 = threadIdx.x; c4 < d / 4; c4 += 256) {
    const float4 v = *(const float4*)(h + (size_t)m * d + 4 * c4);
    const int col = 4 * c4;
    *(float4*)(out + (size_t)o * d + col) =
        make_float4(v.x * rinv * T::to_f(gain[col]), v.y * rinv * T::to_f(gain[col + 1]),
                    v.z * rinv * T::to_f(gain[col + 2]), v.w * rinv * T::to_f(gain[col + 3]));
  }
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

// Value rows -> tile layout. One workgroup per (sequence, kv head, 32-key
// tile): the tile's rows are read coalesced (key-major, D contiguous) into
// LDS and written as the tile's [D][32] block, each row d with the 32 keys
// at their permuted columns (vtile_col), zero past kv_len.
template <typename T>
__global__ __launch_bounds__(256) void tile_values_kernel(const typename T::store_t* __restrict__ v,
                                                          typename T::store_t* __restrict__ vt,
                                                          int kv_len, int D, int tiles) {
  using E = typename T::store_t;
  __shared__ E s_v[32][128 + 1];
  const int tile = blockIdx.x % tiles;
  const size_t bh = blockIdx.x / tiles;
  const E* src = v + bh * (size_t)kv_len * D;
  E* dst = vt + (bh * tiles + tile) * (size_t)D * 32;
  for (int i = threadIdx.x; i < 32 * D; i += 256) {
    const int k = i / D, d = i % D, key = tile * 32 + k;
    s_v[k][d] = key < kv_len ? src[(size_t)key * D + d] : E(0);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 32 * D; i += 256) {
    const int d = i / 32, col = i % 32;
    // the logical key stored at this column (inverse of vtile_col)
    const int k = 4 * (col / 8) + (((col / 4) & 1) ? 16 : 0) + col % 4;
    dst[(size_t)d * 32 + col] = s_v[k][d];
  }
}

hipError_t launch_tile_values(int dt, const void* v, void* vt, int batch, int hkv, int kv_len, int D,
                              hipStream_t st) {
  const int tiles = (kv_len + 31) / 32;
  const int n = batch * hkv * tiles;
  if (n <= 0) return hipSuccess;
  if (D > 128) return hipErrorInvalidValue;
  if (dt == kBF16)
    hipLaunchKernelGGL(tile_values_kernel<BF16>, dim3(n), dim3(256), 0, st, (const uint16_t*)v,
                       (uint16_t*)vt, kv_len, D, tiles);
  else
    hipLaunchKernelGGL(tile_values_kernel<F32>, dim3(n), dim3(256), 0, st, (const float*)v,
                       (float*)vt, kv_len, D, tiles);
  return hipGetLastError();
}

// Streaming read: a grid of at most 8 workgroups per CU strides over the
// buffer; per iteration a workgroup reads 32 KB contiguous (8 independent
// 16-byte loads per thread in flight), and at the end writes the XOR of the
// words it read (so the compiler keeps every load). A measurement of the HBM
// read rate a kernel of this library can reach, not part of the method.
constexpr int kStreamUnroll = 8;
constexpr int kStreamMaxBlocks = 256 * 8;

__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* __restrict__ buf, size_t n16,
                                                          float* __restrict__ out) {
  const size_t step = (size_t)gridDim.x * 256 * kStreamUnroll;
  uint32_t acc = 0;
  for (size_t base = (size_t)blockIdx.x * 256 * kStreamUnroll + threadIdx.x; base < n16; base += step) {
    uint4 a[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) {
      const size_t j = base + (size_t)u * 256;
      a[u] = j < n16 ? buf[j] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) acc ^= a[u].x ^ a[u].y ^ a[u].z ^ a[u].w;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o);
  __shared__ uint32_t s[4];
  if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = (float)(s[0] ^ s[1] ^ s[2] ^ s[3]);
}

int stream_read_blocks(size_t bytes) {
  const size_t per = (size_t)256 * kStreamUnroll * 16;
  return (int)std::min<size_t>((bytes + per - 1) / per, kStreamMaxBlocks);
}

hipError_t launch_stream_read(const void* buf, size_t bytes, float* out, hipStream_t st) {
  const int n = stream_read_blocks(bytes);
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(stream_read_kernel, dim3(n), dim3(256), 0, st, (const uint4*)buf, bytes / 16, out);
  return hipGetLastError();
}

// Cosine similarity of two key/value snapshots in the cache layout ([commentary]
// 3.4.2, the measurement behind the approximate cache: how much a token's
// K and V move between two decoding steps). One workgroup per (sequence,
// row): the token's K over all kv heads (Hkv * D values) and its V likewise,
// reduced in a fixed order; cos = <a, b> / sqrt(|a|^2 |b|^2), 0 when either
// norm is 0. out[(seq * nrows + r) * 2 + {0: K, 1: V}].
template <typename T>
__global__ __launch_bounds__(256) void kv_cosine_kernel(
    const typename T::store_t* __restrict__ ka, const typename T::store_t* __restrict__ va,
    const typename T::store_t* __restrict__ kb, const typename T::store_t* __restrict__ vb,
    int hkv, int cap, int D, int row0, int nrows, float* __restrict__ out) {
  __shared__ float s_red[4][6];
  const int o = blockIdx.x;
  const int seq = o / nrows, r = o % nrows, row = row0 + r;
  const int vcap = (cap + 31) & ~31;
  float acc[6] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f};  // K: ab aa bb, V: ab aa bb
  for (int i = threadIdx.x; i < hkv * D; i += 256) {
    const int h = i / D, d = i % D;
    const size_t kofs = (((size_t)seq * hkv + h) * cap + row) * D + d;
    const size_t vofs = ((size_t)seq * hkv + h) * vcap * D + vtile_off(row, d, D);
    const float x = T::to_f(ka[kofs]), y = T::to_f(kb[kofs]);
    const float u = T::to_f(va[vofs]), w = T::to_f(vb[vofs]);
    acc[0] += x * y; acc[1] += x * x; acc[2] += y * y;
    acc[3] += u * w; acc[4] += u * u; acc[5] += w * w;
  }
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int q = 0; q < 6; ++q) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc[q] += __shfl_xor(acc[q], off);
    if (lane == 0) s_red[wv][q] = acc[q];
  }
  __syncthreads();
  if (threadIdx.x < 2) {
    const int base = threadIdx.x * 3;
    float t[3];
#pragma unroll
    for (int q = 0; q < 3; ++q)
      t[q] = ((s_red[0][base + q] + s_red[1][base + q]) + s_red[2][base + q]) + s_red[3][base + q];
    const float den = t[1] * t[2];
    out[(size_t)o * 2 + threadIdx.x] = den > 0.f ? t[0] / sqrtf(den) : 0.f;
  }
}

hipError_t launch_kv_cosine(int dt, const void* ka, const void* va, const void* kb, const void* vb,
                            int batch, int hkv, int cap, int D, int row0, int nrows, float* out,
                            hipStream_t st) {
  const int n = batch * nrows;
  if (n <= 0) return hipSuccess;
  if (dt == kBF16)
    hipLaunchKernelGGL(kv_cosine_kernel<BF16>, dim3(n), dim3(256), 0, st, (const uint16_t*)ka,
                       (const uint16_t*)va, (const uint16_t*)kb, (const uint16_t*)vb, hkv, cap, D,
                       row0, nrows, out);
  else
    hipLaunchKernelGGL(kv_cosine_kernel<F32>, dim3(n), dim3(256), 0, st, (const float*)ka,
                       (const float*)va, (const float*)kb, (const float*)vb, hkv, cap, D, row0,
                       nrows, out);
  return hipGetLastError();
}

}  // namespace fdllm
