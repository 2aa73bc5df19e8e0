// Confidence-aware parallel unmasking from logits ([commentary] 3.4.3 "The
// Core Idea", "Threshold Strategy"): per still-masked block row, the softmax
// max, argmax and normaliser over the vocabulary, then the threshold selection
// with the progress guarantee, then the commit.
//
// Two launches. The first has one workgroup per (row, vocabulary chunk of
// 16384 logits) and streams only rows that are still masked. A thread takes
// the chunk as 2 steps of 4 groups of 8 logits, all loads issued before the
// first step is reduced. Per step it takes the maximum,
// the first id holding it (only where the running maximum rises) and the
// sum of exp(z - max) without branches, folding into a running
// (max, argmax, sum). The second launch has one wave per sequence: lane j
// merges row j's chunks in chunk order and the wave selects. (A completion
// counter shared by the workgroups of a sequence would serialise hundreds
// of device-scope atomics on one address.)
// NaN logits count as -inf; +inf logits share the mass equally (each adds
// 1 at the maximum).
#include <mutex>

#include "common.h"
#include "internal.h"
#include "select.h"

// Fixed statistics scratch of the allocation-free logits-in unmask: one
// copy per GPU, held until the process ends, shared by every call on that
// GPU. Its host-side name is not a device address; host code uses only the
// per-device address hipGetSymbolAddress returns (unmask_static_scratch).
static __device__ __align__(256) unsigned char
    scratch[fdllm::kStaticUnmaskEntries * (sizeof(float4) + sizeof(float2))];

namespace fdllm {

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t unmask_static_scratch(float4** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // the current device's copy
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = (float4*)g_scratch_ptr[dev];
  return hipSuccess;
}

// 8 logits as they sit in memory (one or two 16-byte loads) and as floats.
template <typename T> struct Raw8;
template <> struct Raw8<BF16> {
  u32x4_t w;
  __device__ __forceinline__ void load(const uint16_t* p) {
    w = __builtin_nontemporal_load((const u32x4_t*)p);
  }
  __device__ __forceinline__ void fill_neg_inf() { w = u32x4_t{0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u}; }
  __device__ __forceinline__ void to_f(float* z) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      z[2 * i] = __uint_as_float(w[i] << 16);
      z[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};
template <> struct Raw8<F32> {
  f32x4_t a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = __builtin_nontemporal_load((const f32x4_t*)p);
    b = __builtin_nontemporal_load((const f32x4_t*)p + 1);
  }
  __device__ __forceinline__ void fill_neg_inf() {
    a = f32x4_t{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    b = a;
  }
  __device__ __forceinline__ void to_f(float* z) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      z[i] = a[i];
      z[4 + i] = b[i];
    }
  }
};

constexpr int kUnmaskGroups = 4;                             // 8-logit groups per thread per step
// Two steps (16384 logits) per workgroup: at 32 rows the 8 chunks of a
// 126464-id row give 256 workgroups, one per CU (6.9 -> 5.4 us measured for
// the statistics kernel, against 4 chunks of 32768); at 256 rows it times the
// same as 4 steps, and 1 step is slower there.
constexpr int kUnmaskSteps = 2;                              // steps per workgroup
constexpr int kUnmaskStep = 256 * kUnmaskGroups * 8;         // logits per step
constexpr int kUnmaskSpan = kUnmaskStep * kUnmaskSteps;      // logits per workgroup

// Loads one step: group u of thread tid covers logits i0 + (u * 256 + tid) * 8
// .. + 7. FULL: the whole step lies inside the row (no bounds tests).
template <typename T, bool FULL>
__device__ __forceinline__ void load_step(Raw8<T>* r, const typename T::store_t* zr, int i0,
                                          int vocab, int tid) {
#pragma unroll
  for (int u = 0; u < kUnmaskGroups; ++u) {
    const int i = i0 + (u * 256 + tid) * 8;
    if (FULL || i < vocab)
      r[u].load(zr + i);
    else
      r[u].fill_neg_inf();
  }
}

// Where a row's sampling draws come from (philox.h): key (seed, seq),
// counters (id / 4, pos, step, 1).
struct DrawAt {
  uint32_t seed;
  int seq, pos, step;
};

// Folds one step's logits (ids i0 + (u * 256 + tid) * 8 + e) into the running
// statistics of this thread, whose earlier ids are all lower. SAMPLE: also
// the best z + G (Gumbel-max draw).
template <typename T, bool SAMPLE>
__device__ __forceinline__ void fold_step(SoftStat& st, SampStat& ss, const Raw8<T>* r, int i0,
                                          int tid, int vocab, const DrawAt& at) {
  float z[kUnmaskGroups][8];
#pragma unroll
  for (int u = 0; u < kUnmaskGroups; ++u) r[u].to_f(z[u]);
  if constexpr (SAMPLE) {
#pragma unroll
    for (int u = 0; u < kUnmaskGroups; ++u) {
      const int id0 = i0 + (u * 256 + tid) * 8;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const U64x4 w = philox4x64((uint64_t)((id0 >> 2) + h), (uint64_t)at.pos, (uint64_t)at.step, 1,
                                   at.seed, (uint64_t)at.seq);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int id = id0 + 4 * h + e;
          const float v = z[u][4 * h + e];
          // ids past the row and NaN logits never win
          const float sc = v + gumbel_of(w.w[e]);
          if (id < vocab && sc > ss.m) ss = SampStat{sc, id};
        }
      }
    }
  }
  float m = -INFINITY;  // v_max ignores NaN operands
#pragma unroll
  for (int u = 0; u < kUnmaskGroups; ++u)
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, z[u][e]);
  if (!(m > -INFINITY)) return;  // nothing but -inf and NaN
  constexpr float kLog2e = 1.4426950408889634f;
  if (m > st.m) {
    int a = 0;  // slot u * 8 + e of the first logit equal to m
#pragma unroll
    for (int u = kUnmaskGroups - 1; u >= 0; --u)
#pragma unroll
      for (int e = 7; e >= 0; --e) a = z[u][e] == m ? u * 8 + e : a;
    st.s = st.m == -INFINITY ? 0.f : st.s * __builtin_amdgcn_exp2f((st.m - m) * kLog2e);
    st.m = m;
    st.a = i0 + ((a >> 3) * 256 + tid) * 8 + (a & 7);
  }
  const float mL = st.m * kLog2e;
  float s = 0.f;
#pragma unroll
  for (int u = 0; u < kUnmaskGroups; ++u)
#pragma unroll
    for (int e = 0; e < 8; ++e) s += __builtin_amdgcn_exp2f(fmaf(z[u][e], kLog2e, -mL));
  if (s != s) {  // a NaN logit, or an infinite maximum: redo the step with care
    s = 0.f;
#pragma unroll
    for (int u = 0; u < kUnmaskGroups; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = z[u][e];
        // exp(inf - inf) taken as 1 per infinite logit; NaN and -inf add 0
        s += st.m == INFINITY ? (v == INFINITY ? 1.f : 0.f)
                              : __builtin_amdgcn_exp2f(fmaxf(fmaf(v, kLog2e, -mL), -256.f));
      }
  }
  st.s += s;
}

// This thread's share of the chunk of row zr starting at logit beg. Every
// step's loads are issued first and the steps are folded as they arrive:
// with all of a launch's workgroups resident at once, a pipeline only one
// step deep lines up their load and arithmetic phases, so HBM time and VALU
// time add; with the whole chunk in flight they overlap. FULL: the chunk
// lies inside the row.
template <typename T, bool FULL, bool SAMPLE>
__device__ __forceinline__ SoftStat chunk_stat(const typename T::store_t* zr, int beg, int vocab,
                                               int tid, SampStat& ss, const DrawAt& at) {
  SoftStat st = stat_empty();
  Raw8<T> r[kUnmaskSteps][kUnmaskGroups];
#pragma unroll
  for (int k = 0; k < kUnmaskSteps; ++k)
    load_step<T, FULL>(r[k], zr, beg + k * kUnmaskStep, vocab, tid);
  // keep every load issued ahead of the arithmetic (the scheduler would
  // otherwise hoist conversions between them and wait early)
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int k = 0; k < kUnmaskSteps; ++k)
    fold_step<T, SAMPLE>(st, ss, r[k], beg + k * kUnmaskStep, tid, vocab, at);
  return st;
}

template <typename T, bool SAMPLE>
__global__ __launch_bounds__(256) void unmask_stats_kernel(
    const typename T::store_t* __restrict__ logits, const uint8_t* __restrict__ masked,
    int seq_len, int blk_start, int blk_len, int vocab, int chunks, float4* __restrict__ stats,
    float2* __restrict__ sstats, uint32_t seed, int step) {
  __shared__ float4 s_red[4];
  __shared__ float2 s_sred[4];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int per_seq = blk_len * chunks;
  const int b = blockIdx.x / per_seq;
  const int rem = blockIdx.x % per_seq;
  const int j = rem / chunks, c = rem % chunks;
  if (masked[(size_t)b * seq_len + blk_start + j] == 0) return;  // committed row: not read
  const size_t row = (size_t)b * blk_len + j;
  const typename T::store_t* zr = logits + row * vocab;
  const int beg = c * kUnmaskSpan;
  const DrawAt at{seed, b, blk_start + j, step};
  SampStat ss = samp_empty();
  SoftStat st = beg + kUnmaskSpan <= vocab ? chunk_stat<T, true, SAMPLE>(zr, beg, vocab, tid, ss, at)
                                           : chunk_stat<T, false, SAMPLE>(zr, beg, vocab, tid, ss, at);
  st = stat_wave_reduce(st);
  if (lane == 0) s_red[wv] = make_float4(st.m, __int_as_float(st.a), st.s, 0.f);
  if constexpr (SAMPLE) {
    ss = samp_wave_reduce(ss);
    if (lane == 0) s_sred[wv] = make_float2(ss.m, __int_as_float(ss.a));
  }
  __syncthreads();
  if (tid == 0) {
    SoftStat t = stat_empty();
#pragma unroll
    for (int q = 0; q < 4; ++q) t = stat_merge(t, SoftStat{s_red[q].x, __float_as_int(s_red[q].y), s_red[q].z});
    stats[row * chunks + c] = make_float4(t.m, __int_as_float(t.a), t.s, 0.f);
    if constexpr (SAMPLE) {
      SampStat u = samp_empty();
#pragma unroll
      for (int q = 0; q < 4; ++q) u = samp_merge(u, SampStat{s_sred[q].x, __float_as_int(s_sred[q].y)});
      sstats[row * chunks + c] = make_float2(u.m, __int_as_float(u.a));
    }
  }
}

// One wave per sequence: lane j < blk_len merges row j's chunk statistics
// (rows no longer masked report confidence 0, argmax -1) and the wave runs
// the selection and the commit.
__global__ __launch_bounds__(64) void unmask_select_kernel(
    int32_t* __restrict__ x, uint8_t* __restrict__ masked, int seq_len, int blk_start, int blk_len,
    int chunks, SelectRule rule, int step, int T_, float* conf, int32_t* argmax,
    int32_t* counts, const float4* __restrict__ stats, const float2* __restrict__ sstats) {
  const int lane = threadIdx.x, b = blockIdx.x;
  float myc = 0.f;
  int mya = -1, mytok = -1;
  if (lane < blk_len && masked[(size_t)b * seq_len + blk_start + lane] != 0) {
    SoftStat t = stat_empty();
    const float4* rs = stats + ((size_t)b * blk_len + lane) * chunks;
    constexpr int kB = 8;  // chunk statistics in flight per lane
    for (int q0 = 0; q0 < chunks; q0 += kB) {
      float4 s4[kB];
#pragma unroll
      for (int q = 0; q < kB; ++q)
        if (q0 + q < chunks) s4[q] = rs[q0 + q];
#pragma unroll
      for (int q = 0; q < kB; ++q)
        if (q0 + q < chunks) t = stat_merge(t, SoftStat{s4[q].x, __float_as_int(s4[q].y), s4[q].z});
    }
    if (t.s > 0.f) {
      myc = 1.f / t.s;
      mya = t.a;
    }
    if (rule.sampling) {
      SampStat u = samp_empty();
      const float2* rs2 = sstats + ((size_t)b * blk_len + lane) * chunks;
      for (int q = 0; q < chunks; ++q) u = samp_merge(u, SampStat{rs2[q].x, __float_as_int(rs2[q].y)});
      mytok = u.m > -INFINITY ? u.a : -1;
    }
  }
  select_and_commit(lane, myc, mya, mytok, x + (size_t)b * seq_len, masked + (size_t)b * seq_len,
                    b, blk_start, blk_len, rule, step, T_,
                    conf ? conf + (size_t)b * blk_len : nullptr,
                    argmax ? argmax + (size_t)b * blk_len : nullptr,
                    counts ? counts + 2 * b : nullptr);
}

int unmask_chunks(int vocab) { return (vocab + kUnmaskSpan - 1) / kUnmaskSpan; }

template <typename T, bool SAMPLE>
static void launch_stats(const void* logits, const uint8_t* masked, int grid, int seq_len,
                         int blk_start, int blk_len, int vocab, int chunks, float4* stats,
                         float2* sstats, uint32_t seed, int step, hipStream_t st) {
  hipLaunchKernelGGL((unmask_stats_kernel<T, SAMPLE>), dim3(grid), dim3(256), 0, st,
                     (const typename T::store_t*)logits, masked, seq_len, blk_start, blk_len, vocab,
                     chunks, stats, sstats, seed, step);
}

hipError_t launch_unmask_logits(int dt, const void* logits, int32_t* x, uint8_t* masked, int batch,
                                int seq_len, int blk_start, int blk_len, int vocab,
                                const SelectRuleArgs& ra, int step, int steps_per_block,
                                float* conf, int32_t* argmax, int32_t* counts, float4* stats,
                                hipStream_t st) {
  const int chunks = unmask_chunks(vocab);
  const int grid = batch * blk_len * chunks;
  float2* sstats = (float2*)(stats + (size_t)batch * blk_len * chunks);
  const bool smp = ra.sampling != 0;
  if (dt == kBF16) {
    if (smp) launch_stats<BF16, true>(logits, masked, grid, seq_len, blk_start, blk_len, vocab, chunks, stats, sstats, ra.seed, step, st);
    else launch_stats<BF16, false>(logits, masked, grid, seq_len, blk_start, blk_len, vocab, chunks, stats, sstats, ra.seed, step, st);
  } else {
    if (smp) launch_stats<F32, true>(logits, masked, grid, seq_len, blk_start, blk_len, vocab, chunks, stats, sstats, ra.seed, step, st);
    else launch_stats<F32, false>(logits, masked, grid, seq_len, blk_start, blk_len, vocab, chunks, stats, sstats, ra.seed, step, st);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  SelectRule rule;
  rule.tau = ra.tau;
  rule.factor = ra.factor;
  rule.topk = ra.topk;
  rule.sampling = ra.sampling;
  rule.seed = ra.seed;
  hipLaunchKernelGGL(unmask_select_kernel, dim3(batch), dim3(64), 0, st, x, masked, seq_len,
                     blk_start, blk_len, chunks, rule, step, steps_per_block, conf, argmax, counts,
                     stats, (const float2*)sstats);
  return hipGetLastError();
}

}  // namespace fdllm
