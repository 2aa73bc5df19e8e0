// Confidence-aware parallel unmasking from logits ([commentary] 3.4.3 "The
// Core Idea", "Threshold Strategy"): per still-masked block row, the softmax
// max, argmax and normaliser over the vocabulary, then the threshold selection
// with the progress guarantee, then the commit.
//
// Workgroups own (row, vocabulary chunk) pairs and stream only rows that are
// still masked (16-byte coalesced loads); each reduces its chunk to
// (max, argmax, sum exp) and the last workgroup of a sequence merges the
// chunks in chunk order and selects. NaN logits count as -inf.
#include "common.h"
#include "internal.h"
#include "select.h"

namespace fdllm {

template <typename T>
__device__ __forceinline__ void load8(const typename T::store_t* p, float* z);
template <>
__device__ __forceinline__ void load8<BF16>(const uint16_t* p, float* z) {
  uint4 v = ld_nt_u4(p);
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    z[2 * i] = __uint_as_float(w[i] << 16);
    z[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
template <>
__device__ __forceinline__ void load8<F32>(const float* p, float* z) {
  float4 a = ld_nt_f4(p);
  float4 b = ld_nt_f4((const float4*)p + 1);
  z[0] = a.x; z[1] = a.y; z[2] = a.z; z[3] = a.w;
  z[4] = b.x; z[5] = b.y; z[6] = b.z; z[7] = b.w;
}

template <typename T>
__global__ __launch_bounds__(256) void unmask_logits_kernel(
    const typename T::store_t* __restrict__ logits, int32_t* __restrict__ x,
    uint8_t* __restrict__ masked, int seq_len, int blk_start, int blk_len, int vocab, int chunks,
    int chunk_len, float tau, int step, int T_, float* conf, int32_t* argmax, int32_t* counts,
    float4* __restrict__ stats, int* __restrict__ tickets) {
  __shared__ float4 s_red[4];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int per_seq = blk_len * chunks;
  const int b = blockIdx.x / per_seq;
  const int rem = blockIdx.x % per_seq;
  const int j = rem / chunks, c = rem % chunks;
  const size_t row = (size_t)b * blk_len + j;
  const bool active = masked[(size_t)b * seq_len + blk_start + j] != 0;

  SoftStat st = stat_empty();
  if (active) {
    const typename T::store_t* zr = logits + row * vocab;
    const int beg = c * chunk_len, end = min(vocab, beg + chunk_len);
    constexpr int kU = 4;  // loads in flight per thread
    int i = beg + 8 * tid;
    for (; i + 8 * 256 * (kU - 1) < end; i += 8 * 256 * kU) {
      float z[kU][8];
#pragma unroll
      for (int u = 0; u < kU; ++u) load8<T>(zr + i + u * 8 * 256, z[u]);
#pragma unroll
      for (int u = 0; u < kU; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float v = z[u][e];
          stat_push(st, v != v ? -INFINITY : v, i + u * 8 * 256 + e);
        }
    }
    for (; i < end; i += 8 * 256) {
      float z[8];
      load8<T>(zr + i, z);
#pragma unroll
      for (int e = 0; e < 8; ++e) stat_push(st, z[e] != z[e] ? -INFINITY : z[e], i + e);
    }
  }
  st = stat_wave_reduce(st);
  if (lane == 0) s_red[wv] = make_float4(st.m, __int_as_float(st.a), st.s, 0.f);
  __syncthreads();
  if (tid == 0) {
    SoftStat t = stat_empty();
#pragma unroll
    for (int q = 0; q < 4; ++q) t = stat_merge(t, SoftStat{s_red[q].x, __float_as_int(s_red[q].y), s_red[q].z});
    st_agent4(agent_rsrc(stats + row * chunks), c * 16, f32x4_t{t.m, __int_as_float(t.a), t.s, 0.f});
  }
  if (!last_arrival(tickets + b, per_seq)) return;
  if (wv != 0) return;
  float myc = 0.f;
  int mya = -1;
  if (lane < blk_len) {
    SoftStat t = stat_empty();
    const auto rs = agent_rsrc(stats + ((size_t)b * blk_len + lane) * chunks);
    for (int q = 0; q < chunks; ++q) {
      f32x4_t s4 = ld_agent4(rs, q * 16);
      t = stat_merge(t, SoftStat{s4[0], __float_as_int(s4[1]), s4[2]});
    }
    if (t.s > 0.f) {
      myc = 1.f / t.s;
      mya = t.a;
    }
  }
  select_and_commit(lane, myc, mya, x + (size_t)b * seq_len, masked + (size_t)b * seq_len,
                    blk_start, blk_len, tau, step, T_, conf ? conf + (size_t)b * blk_len : nullptr,
                    argmax ? argmax + (size_t)b * blk_len : nullptr,
                    counts ? counts + 2 * b : nullptr);
}

int unmask_chunks(int vocab) {
  // enough workgroups per row to fill the chip at 256 rows
  int c = 4;
  while (c > 1 && vocab / c < 8 * 256) c >>= 1;
  return c;
}

hipError_t launch_unmask_logits(int dt, const void* logits, int32_t* x, uint8_t* masked, int batch,
                                int seq_len, int blk_start, int blk_len, int vocab, float tau,
                                int step, int steps_per_block, float* conf, int32_t* argmax,
                                int32_t* counts, float4* stats, int* tickets, hipStream_t st) {
  const int chunks = unmask_chunks(vocab);
  const int chunk_len = (int)round_up((vocab + chunks - 1) / chunks, 8);
  const int grid = batch * blk_len * chunks;
  if (dt == kBF16)
    hipLaunchKernelGGL(unmask_logits_kernel<BF16>, dim3(grid), dim3(256), 0, st,
                       (const uint16_t*)logits, x, masked, seq_len, blk_start, blk_len, vocab,
                       chunks, chunk_len, tau, step, steps_per_block, conf, argmax, counts, stats,
                       tickets);
  else
    hipLaunchKernelGGL(unmask_logits_kernel<F32>, dim3(grid), dim3(256), 0, st,
                       (const float*)logits, x, masked, seq_len, blk_start, blk_len, vocab, chunks,
                       chunk_len, tau, step, steps_per_block, conf, argmax, counts, stats, tickets);
  return hipGetLastError();
}

}  // namespace fdllm
