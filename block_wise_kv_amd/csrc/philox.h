// Philox-4x64-10 counter-based generator (Salmon, Moraes, Dror, Shaw,
// "Parallel random numbers: as easy as 1, 2, 3", SC 2011) and the draws the
// stochastic tau-leaping step makes from it ([commentary] 3.4.1 "The Reverse
// Generation Process (with tau-leaping)").
//
// Draws of sequence `seq` under `seed` (key = (seed, seq)):
//  * token noise of vocabulary ids 4q .. 4q+3 at block position `pos`, step
//    `step`: words 0..3 of counter (q, pos, step, 1); u = ((w >> 41) + 0.5)
//    * 2^-23 (exact in float32, strictly inside (0, 1)) and G = -log(-log u)
//    in float32 (Gumbel-max: argmax of z + G is a draw from softmax(z));
//  * the fill decision of that position: word 0 of counter (0, pos, step, 2)
//    as u = (w >> 11) * 2^-53 in float64, filled when u < 1 / (T - step).
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

namespace fdllm {

struct U64x4 {
  uint64_t w[4];
};

__device__ __forceinline__ U64x4 philox4x64(uint64_t c0, uint64_t c1, uint64_t c2, uint64_t c3,
                                            uint64_t k0, uint64_t k1) {
  constexpr uint64_t kM0 = 0xD2E7470EE14C6C93ull, kM1 = 0xCA5A826395121157ull;
  constexpr uint64_t kW0 = 0x9E3779B97F4A7C15ull, kW1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t hi0 = __umul64hi(kM0, c0), lo0 = kM0 * c0;
    const uint64_t hi1 = __umul64hi(kM1, c2), lo1 = kM1 * c2;
    const uint64_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
    k0 += kW0;
    k1 += kW1;
  }
  return U64x4{{c0, c1, c2, c3}};
}

__device__ __forceinline__ float gumbel_of(uint64_t w) {
  const float u = ((float)(uint32_t)(w >> 41) + 0.5f) * 1.1920928955078125e-7f;  // 2^-23
  return -logf(-logf(u));
}

__device__ __forceinline__ bool tau_leap_fill(uint32_t seed, int seq, int pos, int step, int T) {
  const U64x4 r = philox4x64(0, (uint64_t)pos, (uint64_t)step, 2, seed, (uint64_t)seq);
  const double u = (double)(r.w[0] >> 11) * 1.1102230246251565e-16;  // 2^-53
  return u < 1.0 / (double)(T - step);
}

}  // namespace fdllm
