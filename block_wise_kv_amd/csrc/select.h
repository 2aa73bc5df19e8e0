// Confidence merge and threshold selection, shared by the LM-head epilogue and
// the logits-in unmask kernel.
#pragma once

#include "common.h"

namespace fdllm {

// Partial softmax statistics of a slice of one logits row: max, argmax (as a
// float-encoded int) and sum exp(z - max). Combining two slices is exact up
// to rounding; ties in the max keep the lower vocabulary id.
struct SoftStat {
  float m;
  int a;
  float s;
};

__device__ __forceinline__ SoftStat stat_empty() { return {-INFINITY, 0x7fffffff, 0.f}; }

__device__ __forceinline__ SoftStat stat_merge(SoftStat x, SoftStat y) {
  float M = fmaxf(x.m, y.m);
  SoftStat r;
  r.m = M;
  r.a = x.m > y.m ? x.a : (y.m > x.m ? y.a : min(x.a, y.a));
  if (M == -INFINITY) {
    r.s = 0.f;
  } else {
    // a side holding the maximum keeps its sum as is (also when M = +inf)
    r.s = (x.m == M ? x.s : x.s * __expf(x.m - M)) + (y.m == M ? y.s : y.s * __expf(y.m - M));
  }
  return r;
}

// Adds one logit with vocabulary id `id` (ids visited in increasing order by a
// thread, so a later equal value never replaces the argmax).
__device__ __forceinline__ void stat_push(SoftStat& st, float z, int id) {
  if (z > st.m) {
    st.s = st.s * __expf(st.m - z) + 1.f;
    st.m = z;
    st.a = id;
  } else {
    st.s += __expf(z - st.m);
  }
}

__device__ __forceinline__ SoftStat stat_shfl_xor(SoftStat v, int o) {
  SoftStat r;
  r.m = __shfl_xor(v.m, o);
  r.a = __shfl_xor(v.a, o);
  r.s = __shfl_xor(v.s, o);
  return r;
}

// Reduction over the 64 lanes of a wave, fixed butterfly order.
__device__ __forceinline__ SoftStat stat_wave_reduce(SoftStat v) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) v = stat_merge(v, stat_shfl_xor(v, o));
  return v;
}

// Threshold selection for one sequence's block, one lane per block position
// (blk_len <= 64). `c`, `a` are the lane's confidence and argmax. Commits the
// masked positions with c >= tau; if fewer than the quota
// q = max(1, ceil(U / (T - step))) are, commits the q most confident masked
// positions (lower position first on equal confidence). Writes x and the
// masked flags of committed positions and the optional outputs.
__device__ inline void select_and_commit(int lane, float c, int a, int32_t* x_seq,
                                         uint8_t* masked_seq, int blk_start, int blk_len,
                                         float tau, int step, int T, float* conf_out,
                                         int32_t* argmax_out, int32_t* counts_out) {
  bool in = lane < blk_len;
  bool m = in && masked_seq[blk_start + lane] != 0;
  uint64_t mmask = __ballot(m);
  int U = __popcll(mmask);
  int left_steps = T - step;
  int quota = U > 0 ? max(1, (U + left_steps - 1) / left_steps) : 0;
  uint64_t amask = __ballot(m && c >= tau);
  uint64_t sel = amask;
  if (__popcll(amask) < quota) {
    sel = 0;
    for (int r = 0; r < quota; ++r) {
      bool cand = m && !((sel >> lane) & 1ull);
      float bc = cand ? c : -1.f;
      int bl = cand ? lane : 64;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        float oc = __shfl_xor(bc, o);
        int ol = __shfl_xor(bl, o);
        if (oc > bc || (oc == bc && ol < bl)) {
          bc = oc;
          bl = ol;
        }
      }
      if (bl < 64) sel |= 1ull << bl;
    }
  }
  if ((sel >> lane) & 1ull) {
    x_seq[blk_start + lane] = a;
    masked_seq[blk_start + lane] = 0;
  }
  if (in) {
    if (conf_out) conf_out[lane] = c;
    if (argmax_out) argmax_out[lane] = a;
  }
  if (lane == 0 && counts_out) {
    int n = __popcll(sel);
    counts_out[0] = n;
    counts_out[1] = U - n;
  }
}

}  // namespace fdllm
