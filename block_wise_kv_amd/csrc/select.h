// Confidence merge and threshold selection, shared by the LM-head epilogue and
// the logits-in unmask kernel.
#pragma once

#include "common.h"
#include "philox.h"

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
  // A side holding the maximum keeps its sum as is: its exponent is 0 and
  // exp(0) is exactly 1 (also when M = +-inf, where x.m - M is not a number;
  // two empty sides give 0 + 0). Selects rather than branches, so a run of
  // merges stays straight-line code.
  const float dx = x.m == M ? 0.f : x.m - M;
  const float dy = y.m == M ? 0.f : y.m - M;
  r.s = x.s * __expf(dx) + y.s * __expf(dy);
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

// Running best of z + G (Gumbel-max draw): score and vocabulary id; ties
// keep the lower id.
struct SampStat {
  float m;
  int a;
};
__device__ __forceinline__ SampStat samp_empty() { return {-INFINITY, 0x7fffffff}; }
__device__ __forceinline__ SampStat samp_merge(SampStat x, SampStat y) {
  if (y.m > x.m || (y.m == x.m && y.a < x.a)) return y;
  return x;
}
__device__ __forceinline__ SampStat samp_shfl_xor(SampStat v, int o) {
  return SampStat{__shfl_xor(v.m, o), __shfl_xor(v.a, o)};
}
__device__ __forceinline__ SampStat samp_wave_reduce(SampStat v) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) v = samp_merge(v, samp_shfl_xor(v, o));
  return v;
}

// The selection rule of a step: threshold tau, or the factor rule
// (factor > 0), or fixed top-K (topk > 0), or stochastic tau-leaping
// (sampling != 0, draws keyed by seed).
struct SelectRule {
  float tau = 0.9f;
  float factor = 0.f;
  int topk = 0;
  int sampling = 0;
  uint32_t seed = 0;
};

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

// Selection for one sequence's block, one lane per block position
// (blk_len <= 64). `c`, `a` are the lane's confidence and argmax, `tok` its
// sampled token (used with sampling only). With the threshold rule
// ([commentary] 3.4.3 "Threshold Strategy") the masked positions with
// c >= tau; with factor > 0 the factor rule (same section, "Factor
// Strategy"): the n most confident masked positions for the largest n with
// (n + 1) * (1 - c_(n)) < factor (the left side grows with n, so the
// positions passing their own rank's test are exactly the top n*); with
// topk > 0 (the fixed top-K baseline) the topk most confident masked
// positions. Each of these commits at least the quota q = max(1, ceil(U /
// (T - step))) most confident ones (lower position first on equal
// confidence) and writes the argmax. With sampling ([commentary] 3.4.1
// "The Reverse Generation Process (with tau-leaping)") each masked position
// is filled with probability 1 / (T - step) by its own draw (philox.h, key
// (seed, seq)) and takes its sampled token. Writes x and the masked flags
// of committed positions and the optional outputs.
__device__ inline void select_and_commit(int lane, float c, int a, int tok, int32_t* x_seq,
                                         uint8_t* masked_seq, int seq, int blk_start, int blk_len,
                                         const SelectRule& rule, int step, int T,
                                         float* conf_out, int32_t* argmax_out,
                                         int32_t* counts_out) {
  bool in = lane < blk_len;
  bool m = in && masked_seq[blk_start + lane] != 0;
  uint64_t mmask = __ballot(m);
  int U = __popcll(mmask);
  int left_steps = T - step;
  int quota = U > 0 ? max(1, (U + left_steps - 1) / left_steps) : 0;
  // rank of this lane among the masked lanes: higher confidence first,
  // lower position first on equal confidence
  auto rank_of = [&]() {
    int r = 0;
    for (int j = 0; j < 64; ++j) {
      const float cj = __shfl(c, j);
      r += (((mmask >> j) & 1ull) && (cj > c || (cj == c && j < lane))) ? 1 : 0;
    }
    return r;
  };
  uint64_t sel;
  int commit_id = a;
  if (rule.sampling) {
    sel = __ballot(m && tau_leap_fill(rule.seed, seq, blk_start + lane, step, T));
    commit_id = tok;
  } else if (rule.topk > 0) {
    const int r = rank_of();
    sel = __ballot(m && r < max(rule.topk, quota));
  } else if (rule.factor > 0.f) {
    const int r = rank_of();
    const bool ok = m && (float)(r + 2) * (1.f - c) < rule.factor;
    const int n = max(__popcll(__ballot(ok)), quota);
    sel = __ballot(m && r < n);
  } else {
    sel = __ballot(m && c >= rule.tau);
    if (__popcll(sel) < quota) {
      const int r = rank_of();
      sel = __ballot(m && r < quota);
    }
  }
  if ((sel >> lane) & 1ull) {
    x_seq[blk_start + lane] = commit_id;
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
